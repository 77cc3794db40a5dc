// HIP kernels of ART-terminated decode attention for CDNA4 (gfx950).
//
// Method: gist.science technical summary of "ART: Runtime Attention
// Termination" (arXiv 2606.00024), sections 2.1-2.4: tile-wise online-softmax
// attention whose running output is probed after every KV tile; the traversal
// of a query head stops once the probe's norm change and direction change are
// both below their thresholds for `patience` consecutive tiles, tile 0 always
// evaluated.  V-row skip: puntofijo.es article on skipping V dequantisation
// where the softmax weight is negligible.
//
// Work decomposition.  A group is one (batch row, KV head); its G query heads
// share every K/V load.  Work is done by independent worker waves (four per
// work-group, no block-level barriers).
//  * ART mode: a persistent grid of worker waves takes tiles of a group in
//    ascending order from a per-group atomic counter, computes each tile's
//    local softmax partial (max, sum, V accumulator per head) and publishes it
//    in a per-group ring of slots.  Whoever finishes a tile tries to take the
//    group lock and folds every ready tile, in tile order, into the group's
//    running state; the fold evaluates the stop rule exactly as a sequential
//    traversal would, writes the output of each head as it stops, and lowers
//    the group's allocation bound once every head has stopped, so tiles past
//    the stop are never fetched (only tiles already in flight are wasted).
//    Results do not depend on which wave computed which tile: partials are
//    computed identically and folded in a fixed order.
//  * Full mode (no stop rule, no V skip): a static split of each group's tiles
//    over worker waves, each keeping a running state in registers, followed
//    by an in-order combine of the splits.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "art_internal.h"

namespace art {
namespace {

constexpr float kNegInf = -INFINITY;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ------------------------------------------------------------------ atomics (agent scope)
__device__ __forceinline__ int ld_rlx(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_acq(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_sc(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_SEQ_CST, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rlx(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_SEQ_CST, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int faa(int* p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool cas_sc(int* p, int expect, int desired) {
    return __hip_atomic_compare_exchange_strong(p, &expect, desired, __ATOMIC_SEQ_CST,
                                                __ATOMIC_SEQ_CST, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_rel() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acq() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
// orders LDS accesses of one wave (lanes of a wave may read what others wrote)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ------------------------------------------------------------------ element conversions
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Eight consecutive cache elements starting at element `off` (a multiple of 8), widened to fp32.
template <int KV>
__device__ __forceinline__ void load8(const void* base, long long off, float (&o)[8]) {
    if constexpr (KV == ART_F32) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4* p = reinterpret_cast<const f4*>(static_cast<const float*>(base) + off);
        f4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    } else if constexpr (KV == ART_BF16) {
        typedef unsigned u4 __attribute__((ext_vector_type(4)));
        const u4* p = reinterpret_cast<const u4*>(static_cast<const uint16_t*>(base) + off);
        u4 a = __builtin_nontemporal_load(p);
        o[0] = bf16lo(a.x); o[1] = bf16hi(a.x); o[2] = bf16lo(a.y); o[3] = bf16hi(a.y);
        o[4] = bf16lo(a.z); o[5] = bf16hi(a.z); o[6] = bf16lo(a.w); o[7] = bf16hi(a.w);
    } else {
        typedef unsigned u2 __attribute__((ext_vector_type(2)));
        const u2* p = reinterpret_cast<const u2*>(static_cast<const int8_t*>(base) + off);
        u2 a = __builtin_nontemporal_load(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[i] = (float)(int8_t)(a.x >> (8 * i));
            o[4 + i] = (float)(int8_t)(a.y >> (8 * i));
        }
    }
}

// APL consecutive elements (APL = 1 or 2) starting at element `off`, widened to fp32.
template <int KV, int APL>
__device__ __forceinline__ void load_small(const void* base, long long off, float (&o)[APL]) {
    if constexpr (KV == ART_F32) {
        const float* p = static_cast<const float*>(base) + off;
        if constexpr (APL == 2) {
            typedef float f2 __attribute__((ext_vector_type(2)));
            f2 a = __builtin_nontemporal_load(reinterpret_cast<const f2*>(p));
            o[0] = a.x; o[1] = a.y;
        } else {
            o[0] = __builtin_nontemporal_load(p);
        }
    } else if constexpr (KV == ART_BF16) {
        const uint16_t* p = static_cast<const uint16_t*>(base) + off;
        if constexpr (APL == 2) {
            uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
            o[0] = bf16lo(w); o[1] = bf16hi(w);
        } else {
            o[0] = bf16lo(__builtin_nontemporal_load(p));
        }
    } else {
        const int8_t* p = static_cast<const int8_t*>(base) + off;
        if constexpr (APL == 2) {
            uint16_t w = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
            o[0] = (float)(int8_t)(w & 0xff); o[1] = (float)(int8_t)(w >> 8);
        } else {
            o[0] = (float)__builtin_nontemporal_load(p);
        }
    }
}

// Row index of cached position j of (b, kv head g); ok=false on an invalid block id.
__device__ __forceinline__ long long row_index(const Params& P, int b, int g, int j, bool& ok) {
    if (P.block_size == 0) return ((long long)b * P.Hkv + g) * P.max_ctx + j;
    const int blk = P.block_table[(long long)b * P.mbps + j / P.block_size];
    if (blk < 0 || blk >= P.num_blocks) {
        ok = false;
        return 0;
    }
    return ((long long)blk * P.Hkv + g) * P.block_size + (j % P.block_size);
}

// ------------------------------------------------------------------ generic tile (VALU)
//
// One wave computes one tile: lane l scores token t*T + l (+64), the tile max
// and sum per head are wave reductions, the kept weights go through LDS and the
// V accumulation maps lane l to head dims l*APL .. l*APL+APL-1.
template <int D, int KV>
struct GenericTile {
    static constexpr int APL = D / 64;

    __device__ static void load_q(const Params& P, int b, int g, float* q_lds) {
        const int lane = lane_id();
        for (int i = lane; i < P.G * D; i += 64) {
            const long long off = ((long long)b * P.Hq + (long long)g * P.G) * D + i;
            q_lds[i] = P.q_dtype == ART_F32 ? static_cast<const float*>(P.q)[off]
                                            : bf16lo(static_cast<const uint16_t*>(P.q)[off]);
        }
        wave_lds_sync();
    }

    // Returns false if `hook` asked to abandon the tile.  hook(m_loc, Mt) fills
    // Mt with the running max through this tile (used by the V skip only).
    template <class Hook>
    __device__ static bool compute(const Params& P, int b, int g, int n, int t, const float* q_lds,
                                   float* p_lds, float (&m_loc)[kMaxG], float (&l_loc)[kMaxG],
                                   float (&acc)[kMaxG][APL], int& err, int& kept, Hook&& hook) {
        const int lane = lane_id();
        const int G = P.G, T = P.T;
        const int j0 = t * T;
        float s[2][kMaxG];
        bool valid[2];
        int bad = 0;
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const int jj = ps * 64 + lane;
            const int j = j0 + jj;
            valid[ps] = jj < T && j < n;
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) s[ps][h] = 0.f;
            if (valid[ps]) {
                bool ok = true;
                const long long r = row_index(P, b, g, j, ok);
                if (!ok) {
                    bad = 1;
                    valid[ps] = false;
                } else {
                    const float sc = (KV == ART_I8 ? f16_to_f32(P.ks[r]) : 1.f) * P.inv_sqrt_d;
                    for (int c = 0; c < D; c += 8) {
                        float kk[8];
                        load8<KV>(P.k, r * D + c, kk);
#pragma unroll
                        for (int h = 0; h < kMaxG; ++h) {
                            if (h < G) {
                                const float* qq = q_lds + h * D + c;
                                float a = 0.f;
#pragma unroll
                                for (int i = 0; i < 8; ++i) a = fmaf(qq[i], kk[i], a);
                                s[ps][h] += a;
                            }
                        }
                    }
#pragma unroll
                    for (int h = 0; h < kMaxG; ++h) s[ps][h] *= sc;
                }
            }
        }
        err |= (__ballot(bad) != 0ull);
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            float mx = kNegInf;
#pragma unroll
            for (int ps = 0; ps < 2; ++ps)
                if (valid[ps]) mx = fmaxf(mx, s[ps][h]);
            m_loc[h] = h < G ? wave_max(mx) : kNegInf;
        }
        float Mt[kMaxG];
        if (!hook(m_loc, Mt)) return false;
        float lsum[kMaxG];
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) lsum[h] = 0.f;
        uint64_t keep_mask[2];
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const int jj = ps * 64 + lane;
            bool row_keep = false;
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) {
                if (h < G) {
                    const float p = valid[ps] ? expf(s[ps][h] - m_loc[h]) : 0.f;
                    lsum[h] += p;
                    const bool keep = valid[ps] && (!P.vskip || expf(s[ps][h] - Mt[h]) >= P.v_skip_eps);
                    row_keep |= keep;
                    if (jj < T) p_lds[h * T + jj] = keep ? p : 0.f;
                }
            }
            keep_mask[ps] = __ballot(row_keep);
        }
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) l_loc[h] = h < G ? wave_sum(lsum[h]) : 0.f;
        wave_lds_sync();
#pragma unroll
        for (int h = 0; h < kMaxG; ++h)
#pragma unroll
            for (int i = 0; i < APL; ++i) acc[h][i] = 0.f;
        kept = __builtin_popcountll(keep_mask[0]) + __builtin_popcountll(keep_mask[1]);
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            uint64_t m = keep_mask[ps];
            while (m) {
                const int jj = ps * 64 + __builtin_ctzll(m);
                m &= m - 1;
                bool ok = true;
                const long long r = row_index(P, b, g, j0 + jj, ok);
                const float vsc = KV == ART_I8 ? f16_to_f32(P.vs[r]) : 1.f;
                float vv[APL];
                load_small<KV, APL>(P.v, r * D + lane * APL, vv);
#pragma unroll
                for (int i = 0; i < APL; ++i) vv[i] *= vsc;
#pragma unroll
                for (int h = 0; h < kMaxG; ++h) {
                    if (h < G) {
                        const float pv = p_lds[h * T + jj];
#pragma unroll
                        for (int i = 0; i < APL; ++i) acc[h][i] = fmaf(pv, vv[i], acc[h][i]);
                    }
                }
            }
        }
        wave_lds_sync();  // p_lds is rewritten by the next tile
        return true;
    }

    // Store a tile (or split) partial in the common slot format.
    __device__ static void store_partial(const Params& P, float* slot, const float (&m)[kMaxG],
                                         const float (&l)[kMaxG], const float (&acc)[kMaxG][APL],
                                         int err, int kept) {
        const int lane = lane_id();
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) {
                if (h < P.G) {
                    slot[h] = m[h];
                    slot[16 + h] = l[h];
                }
            }
            reinterpret_cast<int*>(slot)[32] = err;
            reinterpret_cast<int*>(slot)[33] = kept;
        }
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            if (h < P.G) {
                float* dst = slot + kSlotHeader + h * D + lane * APL;
#pragma unroll
                for (int i = 0; i < APL; ++i) dst[i] = acc[h][i];
            }
        }
    }
};

// ------------------------------------------------------------------ fold of partials
//
// Lane mapping used by the fold, the combine and the init: lane l serves head
// hb*4 + (l >> 4) of head block hb and head dims 8*(l & 15) .. +7.
struct FoldLanes {
    int hl, cid, HB;
    bool cvalid;
    __device__ FoldLanes(const Params& P) {
        const int lane = lane_id();
        hl = lane >> 4;
        cid = lane & 15;
        HB = (P.G + 3) >> 2;
        cvalid = cid < (P.D >> 3);
    }
};

__device__ __forceinline__ void write_head_out(const Params& P, int grp, int h, const FoldLanes& fl,
                                               const float (&a8)[8], float L, int err, int U) {
    const int b = grp / P.Hkv, g = grp % P.Hkv;
    const long long row = (long long)b * P.Hq + (long long)g * P.G + h;
    if (fl.cvalid) {
        float* o = P.out + row * P.D + 8 * fl.cid;
        const float inv = 1.f / L;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = err ? NAN : a8[i] * inv;
    }
    if (fl.cid == 0) P.tiles_used[row] = err ? -1 : U;
}

// Try to take the group lock and fold every ready tile in order.
__device__ void try_advance(const Params& P, int grp) {
    GroupCtl* C = P.ctl + grp;
    const int lane = lane_id();
    const FoldLanes fl(P);
    const int G = P.G, D = P.D;
    for (;;) {
        int got = 0;
        if (lane == 0) got = cas_sc(&C->lock, 0, 1);
        if (!__shfl(got, 0)) return;
        int f = ld_rlx(&C->frontier);
        const int nt = ld_rlx(&C->nt);
        if (f >= ld_rlx(&C->bound)) {
            // the group has finished: its heads are written, nothing more to fold
            fence_rel();
            if (lane == 0) st_sc(&C->lock, 0);
            return;
        }
        float M[4], L[4], a8[4][8], prev[4][8], pn[4];
        int streak[4], U[4], err[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            const int h = hb * 4 + fl.hl;
            U[hb] = 0;  // absent heads count as finished
            M[hb] = kNegInf; L[hb] = 0.f; pn[hb] = 0.f; streak[hb] = 0; err[hb] = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) { a8[hb][i] = 0.f; prev[hb][i] = 0.f; }
            if (hb < fl.HB && h < G) {
                const HeadState& hs = P.heads[(long long)grp * G + h];
                M[hb] = hs.M; L[hb] = hs.L; streak[hb] = hs.streak; U[hb] = hs.U; err[hb] = hs.err;
                pn[hb] = hs.pn;
#pragma unroll
                for (int i = 0; i < 8; ++i) prev[hb][i] = hs.prev[i];
                if (fl.cvalid) {
                    const float* a = P.acc + ((long long)grp * G + h) * D + 8 * fl.cid;
#pragma unroll
                    for (int i = 0; i < 8; ++i) a8[hb][i] = a[i];
                }
            }
        }
        bool finished = false;
        for (;;) {
            const int tau = f + lane;
            const bool ok = tau < nt &&
                            ld_rlx(&P.ring_tag[(long long)grp * kRing + (tau & (kRing - 1))]) == tau + 1;
            const uint64_t m = __ballot(ok);
            const int k = (~m == 0ull) ? 64 : __builtin_ctzll(~m);
            if (k == 0) break;
            fence_acq();
            int folded = 0;
            for (int i = 0; i < k; ++i) {
                const int tt = f + i;
                const float* slot = P.ring + ((long long)grp * kRing + (tt & (kRing - 1))) * P.slot;
                const int serr = reinterpret_cast<const int*>(slot)[32];
                int n_active = 0;
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) {
                    const int h = hb * 4 + fl.hl;
                    const bool active = hb < fl.HB && h < G && U[hb] < 0;
                    int stop = 0;
                    if (active) {
                        const float ml = slot[h], ll = slot[16 + h];
                        const float mn = fmaxf(M[hb], ml);
                        const float al = M[hb] == kNegInf ? 0.f : expf(M[hb] - mn);
                        const float be = expf(ml - mn);
                        L[hb] = al * L[hb] + be * ll;
                        if (fl.cvalid) {
                            const float* a = slot + kSlotHeader + h * D + 8 * fl.cid;
#pragma unroll
                            for (int j = 0; j < 8; ++j) a8[hb][j] = al * a8[hb][j] + be * a[j];
                        }
                        M[hb] = mn;
                        err[hb] |= serr;
                        if (fl.cid == 0) {
                            // probe: dims 0..7 of the normalised running output
                            float x[8], xn2 = 0.f;
                            const float invL = 1.f / L[hb];
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                x[j] = a8[hb][j] * invL;
                                xn2 += x[j] * x[j];
                            }
                            const float xn = sqrtf(xn2);
                            if (tt >= 1) {
                                float ds, dd;
                                if (xn == 0.f || pn[hb] == 0.f) {
                                    ds = dd = INFINITY;
                                } else {
                                    ds = fabsf(xn - pn[hb]) / pn[hb];
                                    // 1 - cos as half the squared distance of the unit vectors
                                    const float ix = 1.f / xn, ip = 1.f / pn[hb];
                                    float s2 = 0.f;
#pragma unroll
                                    for (int j = 0; j < 8; ++j) {
                                        const float dlt = x[j] * ix - prev[hb][j] * ip;
                                        s2 += dlt * dlt;
                                    }
                                    dd = 0.5f * s2;
                                }
                                const bool pass = P.art && ds < P.eps_scale && dd < P.eps_dir;
                                streak[hb] = pass ? streak[hb] + 1 : 0;
                                stop = streak[hb] >= P.patience;
                            }
#pragma unroll
                            for (int j = 0; j < 8; ++j) prev[hb][j] = x[j];
                            pn[hb] = xn;
                        }
                    }
                    stop = __shfl(stop, lane & ~15);
                    if (stop) {
                        U[hb] = tt + 1;
                        write_head_out(P, grp, h, fl, a8[hb], L[hb], err[hb], U[hb]);
                    }
                    n_active += (fl.cid == 0 && hb < fl.HB && h < G && U[hb] < 0) ? 1 : 0;
                }
                ++folded;
                if (__ballot(n_active > 0) == 0ull) {
                    finished = true;
                    break;
                }
            }
            f += folded;
            if (finished || f >= nt) break;
        }
        if (!finished && f >= nt) {
            // no stop: every tile was used
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                const int h = hb * 4 + fl.hl;
                if (hb < fl.HB && h < G && U[hb] < 0) {
                    U[hb] = nt;
                    write_head_out(P, grp, h, fl, a8[hb], L[hb], err[hb], nt);
                }
            }
            finished = true;
        }
        if (!finished) {
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                const int h = hb * 4 + fl.hl;
                if (hb < fl.HB && h < G) {
                    HeadState& hs = P.heads[(long long)grp * G + h];
                    if (fl.cid == 0) {
                        hs.M = M[hb]; hs.L = L[hb]; hs.streak = streak[hb]; hs.U = U[hb];
                        hs.err = err[hb]; hs.pn = pn[hb];
#pragma unroll
                        for (int i = 0; i < 8; ++i) hs.prev[i] = prev[hb][i];
                    }
                    if (fl.cvalid && U[hb] < 0) {
                        float* a = P.acc + ((long long)grp * G + h) * D + 8 * fl.cid;
#pragma unroll
                        for (int i = 0; i < 8; ++i) a[i] = a8[hb][i];
                    }
                }
            }
        }
        if (lane == 0) {
            st_rlx(&C->frontier, f);
            if (finished) st_rlx(&C->bound, f);
        }
        fence_rel();
        if (lane == 0) st_sc(&C->lock, 0);
        if (finished) return;
        // a tile finished while we held the lock may have found it taken
        int again = 0;
        if (lane == 0)
            again = f < nt && ld_sc(&P.ring_tag[(long long)grp * kRing + (f & (kRing - 1))]) == f + 1;
        if (!__shfl(again, 0)) return;
    }
}

// ------------------------------------------------------------------ tile scheduling
// >= 0: the tile taken; -1: group exhausted; -2: ring full (try elsewhere)
__device__ int take_tile(const Params& P, int grp) {
    int r = 0;
    if (lane_id() == 0) {
        GroupCtl* C = P.ctl + grp;
        const int bd = ld_rlx(&C->bound), nx = ld_rlx(&C->next);
        if (nx >= bd) {
            r = -1;
        } else if (nx - ld_rlx(&C->frontier) >= kRing) {
            r = -2;
        } else {
            const int t = faa(&C->next, 1);
            r = t < ld_rlx(&C->bound) ? t : -1;
        }
    }
    return __shfl(r, 0);
}

// Records that a wait ran past kSpinLimit; every worker then leaves.
__device__ void give_up(const Params& P) { st_rlx(P.abort_flag, 1); }
__device__ bool aborted(const Params& P) { return ld_rlx(P.abort_flag) != 0; }

// Waits until slot t % kRing is free; false if the group stopped before tile t
// (or the kernel is giving up).
__device__ bool wait_slot(const Params& P, int grp, int t) {
    int ok = 1;
    if (lane_id() == 0) {
        GroupCtl* C = P.ctl + grp;
        for (int spin = 0;; ++spin) {
            if (t >= ld_rlx(&C->bound)) { ok = 0; break; }
            if (t - ld_acq(&C->frontier) < kRing) break;
            if (spin >= kSpinLimit) { give_up(P); ok = 0; break; }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    return __shfl(ok, 0) != 0;
}

// Next group with tiles left (and room in its ring), scanning forward from grp; -1 when none.
__device__ int next_group(const Params& P, int grp) {
    const int lane = lane_id();
    for (int spin = 0;; ++spin) {
        if (spin >= kSpinLimit || aborted(P)) {
            if (lane == 0) give_up(P);
            return -1;
        }
        bool any_left = false;
        for (int base = 0; base < P.NG; base += 64) {
            const int k = base + lane;
            const int cand = (grp + 1 + k) % P.NG;
            bool has = false, room = false;
            if (k < P.NG) {
                GroupCtl* C = P.ctl + cand;
                const int nx = ld_rlx(&C->next), bd = ld_rlx(&C->bound), fr = ld_rlx(&C->frontier);
                has = nx < bd;
                room = nx - fr < kRing;
            }
            const uint64_t m = __ballot(has && room);
            if (m) return (grp + 1 + base + __builtin_ctzll(m)) % P.NG;
            any_left |= __ballot(has) != 0ull;
        }
        if (!any_left) return -1;
        __builtin_amdgcn_s_sleep(8);
    }
}

// ------------------------------------------------------------------ kernels
__global__ __launch_bounds__(256) void art_init_kernel(Params P) {
    const int grp = blockIdx.x;
    const int tid = threadIdx.x;
    const int b = grp / P.Hkv, g = grp % P.Hkv;
    const int n = P.ctx_lens[b];
    const bool bad = n < 0 || n > P.cap;
    const int nt = (bad || n == 0) ? 0 : (n + P.T - 1) / P.T;
    GroupCtl* C = P.ctl + grp;
    if (tid == 0) {
        C->next = 0; C->lock = 0; C->frontier = 0; C->bound = nt; C->nt = nt; C->n = n;
        if (grp == 0) *P.abort_flag = 0;
    }
    for (int h = tid; h < P.G; h += blockDim.x) {
        HeadState& hs = P.heads[(long long)grp * P.G + h];
        hs.M = kNegInf; hs.L = 0.f; hs.streak = 0; hs.U = nt > 0 ? -1 : 0; hs.err = 0; hs.pn = 0.f;
        for (int i = 0; i < 8; ++i) hs.prev[i] = 0.f;
    }
    for (int i = tid; i < P.G * P.D; i += blockDim.x) P.acc[(long long)grp * P.G * P.D + i] = 0.f;
    for (int i = tid; i < kRing; i += blockDim.x) P.ring_tag[(long long)grp * kRing + i] = 0;
    if (P.vskip)
        for (int i = tid; i < P.nt_max; i += blockDim.x) P.vmax_tag[(long long)grp * P.nt_max + i] = 0;
    // outputs of finished rows now; the others are marked unfinished (-2, NaN)
    // until the fold writes them
    const long long row0 = (long long)b * P.Hq + (long long)g * P.G;
    for (int i = tid; i < P.G * P.D; i += blockDim.x)
        P.out[row0 * P.D + i] = (nt == 0 && !bad) ? 0.f : NAN;
    for (int h = tid; h < P.G; h += blockDim.x) P.tiles_used[row0 + h] = nt > 0 ? -2 : (bad ? -1 : 0);
}

template <int D, int KV>
__global__ __launch_bounds__(256) void art_persistent_kernel(Params P) {
    using Tile = GenericTile<D, KV>;
    extern __shared__ float lds[];
    const int wv = wave_id(), lane = lane_id();
    const int per_wave = P.G * D + P.G * P.T;
    float* q_lds = lds + wv * per_wave;
    float* p_lds = q_lds + P.G * D;
    const int worker = blockIdx.x * kWavesPerWG + wv;
    if (worker >= P.workers) return;
    int grp = worker % P.NG;
    int qgrp = -1;
    for (;;) {
        if (aborted(P)) break;
        const int t = take_tile(P, grp);
        if (t < 0) {
            grp = next_group(P, grp);
            if (grp < 0) break;
            continue;
        }
        const int b = grp / P.Hkv, g = grp % P.Hkv;
        if (grp != qgrp) {
            Tile::load_q(P, b, g, q_lds);
            qgrp = grp;
        }
        if (!wait_slot(P, grp, t)) continue;
        GroupCtl* C = P.ctl + grp;
        const int n = ld_rlx(&C->n);
        float m_loc[kMaxG], l_loc[kMaxG], acc[kMaxG][Tile::APL];
        int err = 0, kept = 0;
        const int vbase = grp * P.nt_max;
        auto hook = [&](const float (&ml)[kMaxG], float (&Mt)[kMaxG]) -> bool {
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) Mt[h] = ml[h];
            if (!P.vskip) return true;
            // publish this tile's maxima, then take the max over all earlier tiles
            float* vm = P.vmax + ((long long)vbase + t) * 16;
            if (lane == 0)
#pragma unroll
                for (int h = 0; h < kMaxG; ++h)
                    if (h < P.G) vm[h] = ml[h];
            fence_rel();
            if (lane == 0) st_rlx(&P.vmax_tag[vbase + t], 1);
            for (int base = 0; base < t; base += 64) {
                const int tau = base + lane;
                const bool need = tau < t;
                for (int spin = 0;; ++spin) {
                    const bool ready = !need || ld_rlx(&P.vmax_tag[vbase + tau]) != 0;
                    if (__ballot(!ready) == 0ull) break;
                    if (ld_rlx(&C->bound) <= t) return false;
                    if (spin >= kSpinLimit) {
                        if (lane == 0) give_up(P);
                        return false;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                fence_acq();
                const float* src = P.vmax + ((long long)vbase + tau) * 16;
#pragma unroll
                for (int h = 0; h < kMaxG; ++h) {
                    if (h < P.G) Mt[h] = fmaxf(Mt[h], wave_max(need ? src[h] : kNegInf));
                }
            }
            return true;
        };
        if (!Tile::compute(P, b, g, n, t, q_lds, p_lds, m_loc, l_loc, acc, err, kept, hook)) continue;
        float* slot = P.ring + ((long long)grp * kRing + (t & (kRing - 1))) * P.slot;
        Tile::store_partial(P, slot, m_loc, l_loc, acc, err, kept);
        fence_rel();
        if (lane == 0) {
            st_rlx(&P.ring_tag[(long long)grp * kRing + (t & (kRing - 1))], t + 1);
            if (P.stats) {
                atomicAdd(reinterpret_cast<unsigned long long*>(P.stats + 0), 1ull);
                atomicAdd(reinterpret_cast<unsigned long long*>(P.stats + 1), (unsigned long long)kept);
            }
        }
        try_advance(P, grp);
    }
}

template <int D, int KV>
__global__ __launch_bounds__(256) void art_full_kernel(Params P) {
    using Tile = GenericTile<D, KV>;
    extern __shared__ float lds[];
    const int wv = wave_id(), lane = lane_id();
    const int per_wave = P.G * D + P.G * P.T;
    float* q_lds = lds + wv * per_wave;
    float* p_lds = q_lds + P.G * D;
    const int worker = blockIdx.x * kWavesPerWG + wv;
    if (worker >= P.NG * P.splits) return;
    const int grp = worker / P.splits, sp = worker % P.splits;
    const int b = grp / P.Hkv, g = grp % P.Hkv;
    const int n = P.ctx_lens[b];
    const bool bad = n < 0 || n > P.cap;
    const int nt = bad ? 0 : (n + P.T - 1) / P.T;
    const int t0 = sp * P.tiles_per_split;
    const int t1 = min(t0 + P.tiles_per_split, nt);
    float M[kMaxG], L[kMaxG], A[kMaxG][Tile::APL];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
        M[h] = kNegInf; L[h] = 0.f;
#pragma unroll
        for (int i = 0; i < Tile::APL; ++i) A[h][i] = 0.f;
    }
    int err = 0, kept_total = 0;
    if (t0 < t1) Tile::load_q(P, b, g, q_lds);
    auto hook = [&](const float (&ml)[kMaxG], float (&Mt)[kMaxG]) -> bool {
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) Mt[h] = ml[h];
        return true;
    };
    for (int t = t0; t < t1; ++t) {
        float ml[kMaxG], ll[kMaxG], a[kMaxG][Tile::APL];
        int kept = 0;
        Tile::compute(P, b, g, n, t, q_lds, p_lds, ml, ll, a, err, kept, hook);
        kept_total += kept;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            if (h < P.G) {
                const float mn = fmaxf(M[h], ml[h]);
                const float al = M[h] == kNegInf ? 0.f : expf(M[h] - mn);
                const float be = expf(ml[h] - mn);
                L[h] = al * L[h] + be * ll[h];
#pragma unroll
                for (int i = 0; i < Tile::APL; ++i) A[h][i] = al * A[h][i] + be * a[h][i];
                M[h] = mn;
            }
        }
    }
    float* slot = P.partials + ((long long)grp * P.splits + sp) * P.slot;
    Tile::store_partial(P, slot, M, L, A, err, kept_total);
    if (P.stats && lane == 0 && t1 > t0) {
        atomicAdd(reinterpret_cast<unsigned long long*>(P.stats + 0), (unsigned long long)(t1 - t0));
        atomicAdd(reinterpret_cast<unsigned long long*>(P.stats + 1), (unsigned long long)kept_total);
    }
}

// One wave per group: merge the splits in order and write the outputs.
__global__ __launch_bounds__(64) void art_combine_kernel(Params P) {
    const int grp = blockIdx.x;
    const FoldLanes fl(P);
    const int G = P.G, D = P.D;
    const int b = grp / P.Hkv, g = grp % P.Hkv;
    const int n = P.ctx_lens[b];
    const bool bad = n < 0 || n > P.cap;
    const int nt = bad ? 0 : (n + P.T - 1) / P.T;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
        const int h = hb * 4 + fl.hl;
        if (hb >= fl.HB || h >= G) continue;
        float M = kNegInf, L = 0.f, a8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        int err = bad ? 1 : 0;
        for (int sp = 0; sp < P.splits; ++sp) {
            const float* slot = P.partials + ((long long)grp * P.splits + sp) * P.slot;
            const float ll = slot[16 + h];
            err |= reinterpret_cast<const int*>(slot)[32];
            if (!(ll > 0.f)) continue;  // empty split
            const float ml = slot[h];
            const float mn = fmaxf(M, ml);
            const float al = M == kNegInf ? 0.f : expf(M - mn);
            const float be = expf(ml - mn);
            L = al * L + be * ll;
            if (fl.cvalid) {
                const float* a = slot + kSlotHeader + h * D + 8 * fl.cid;
#pragma unroll
                for (int j = 0; j < 8; ++j) a8[j] = al * a8[j] + be * a[j];
            }
            M = mn;
        }
        if (nt == 0 && !bad) {
            const long long row = (long long)b * P.Hq + (long long)g * G + h;
            if (fl.cvalid)
                for (int j = 0; j < 8; ++j) P.out[row * D + 8 * fl.cid + j] = 0.f;
            if (fl.cid == 0) P.tiles_used[row] = 0;
        } else {
            write_head_out(P, grp, h, fl, a8, L, err, nt);
        }
    }
}

template <int D, int KV>
int launch_art_t(const Params& p, hipStream_t s) {
    hipLaunchKernelGGL(art_init_kernel, dim3(p.NG), dim3(256), 0, s, p);
    const size_t lds = (size_t)kWavesPerWG * (p.G * D + p.G * p.T) * sizeof(float);
    const int blocks = (p.workers + kWavesPerWG - 1) / kWavesPerWG;
    hipLaunchKernelGGL((art_persistent_kernel<D, KV>), dim3(blocks), dim3(256), lds, s, p);
    return (int)hipGetLastError();
}

template <int D, int KV>
int launch_full_t(const Params& p, hipStream_t s) {
    const size_t lds = (size_t)kWavesPerWG * (p.G * D + p.G * p.T) * sizeof(float);
    const int blocks = (p.NG * p.splits + kWavesPerWG - 1) / kWavesPerWG;
    hipLaunchKernelGGL((art_full_kernel<D, KV>), dim3(blocks), dim3(256), lds, s, p);
    hipLaunchKernelGGL(art_combine_kernel, dim3(p.NG), dim3(64), 0, s, p);
    return (int)hipGetLastError();
}

}  // namespace

int launch_art(const Params& p, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (p.NG == 0) return 0;
    if (p.D == 64) {
        if (p.kv_dtype == ART_F32) return launch_art_t<64, ART_F32>(p, s);
        if (p.kv_dtype == ART_BF16) return launch_art_t<64, ART_BF16>(p, s);
        return launch_art_t<64, ART_I8>(p, s);
    }
    if (p.kv_dtype == ART_F32) return launch_art_t<128, ART_F32>(p, s);
    if (p.kv_dtype == ART_BF16) return launch_art_t<128, ART_BF16>(p, s);
    return launch_art_t<128, ART_I8>(p, s);
}

int launch_full(const Params& p, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (p.NG == 0) return 0;
    if (p.D == 64) {
        if (p.kv_dtype == ART_F32) return launch_full_t<64, ART_F32>(p, s);
        if (p.kv_dtype == ART_BF16) return launch_full_t<64, ART_BF16>(p, s);
        return launch_full_t<64, ART_I8>(p, s);
    }
    if (p.kv_dtype == ART_F32) return launch_full_t<128, ART_F32>(p, s);
    if (p.kv_dtype == ART_BF16) return launch_full_t<128, ART_BF16>(p, s);
    return launch_full_t<128, ART_I8>(p, s);
}

}  // namespace art
