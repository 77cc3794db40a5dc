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
//
// Tile computation.  bf16/int8 caches with head dim 128 and bf16 queries use
// matrix cores for the scores: each 16-token page of K is the A operand of
// four v_mfma_f32_16x16x32_bf16 (one per 32 head dims) against the group's
// queries as the B operand (heads padded to 16 columns).  Softmax and the
// P.V accumulation run on the vector ALUs from 128-bit V loads (one wave
// instruction reads four whole 256-byte rows).  Other shapes use a plain
// vector-ALU tile.
//
// Cross-wave data.  Everything one wave publishes for another (ring slots,
// the group's running state, tile maxima, counters) is written and read with
// agent-scope relaxed atomics, which gfx950 performs as coherent (sc1)
// accesses; a producer waits for its stores to complete before it stores the
// flag that publishes them.  No L2 writeback or invalidate is ever issued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "art_internal.h"

namespace art {
namespace {

constexpr float kNegInf = -INFINITY;

typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// wave index within the work-group (wave-uniform, so kept in a scalar register)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
// lane 0's value, as a wave-uniform (scalar) value
__device__ __forceinline__ int bcast0(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------------------ coherent accesses
template <class T>
__device__ __forceinline__ T cld(const T* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void cst(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// a wave-uniform value in scalar registers
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ unsigned long long uni64(unsigned long long x) {
    return ((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
           (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)x);
}

__device__ __forceinline__ int faa(int* p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool cas(int* p, int expect, int desired) {
    return __hip_atomic_compare_exchange_strong(p, &expect, desired, __ATOMIC_RELAXED,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every memory access this wave issued has completed.  Shared
// data is only accessed coherently, so completed stores are visible to any
// later coherent load: a flag stored after drain() publishes them.
__device__ __forceinline__ void drain() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// orders LDS accesses of one wave (lanes of a wave may read what others wrote)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// e^x from the hardware base-2 exponential (a couple of ulp; e^-inf = 0)
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ------------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
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
__device__ __forceinline__ float sbyte(uint32_t w, int k) { return (float)(int)(int8_t)(w >> (8 * k)); }
// signed 4-bit code k of a 32-bit word (code k in bits 4k..4k+3), sign-extended
__device__ __forceinline__ float snib(uint32_t w, int k) { return (float)((int)(w << (28 - 4 * k)) >> 28); }
// two small integers (|x| <= 128) as a packed bf16 pair: exact, since they need at most 8 bits,
// so the upper halves of their fp32 words are their bf16 values (one v_perm_b32: bytes 0-3 of
// the selection come from the second operand, 4-7 from the first)
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Eight consecutive cache elements starting at element `off` (a multiple of 8), widened to fp32.
template <int KV>
__device__ __forceinline__ void load8(const void* base, long long off, float (&o)[8]) {
    if constexpr (KV == ART_F32) {
        const f4* p = reinterpret_cast<const f4*>(static_cast<const float*>(base) + off);
        f4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    } else if constexpr (KV == ART_BF16) {
        const u4* p = reinterpret_cast<const u4*>(static_cast<const uint16_t*>(base) + off);
        u4 a = __builtin_nontemporal_load(p);
        o[0] = bf16lo(a.x); o[1] = bf16hi(a.x); o[2] = bf16lo(a.y); o[3] = bf16hi(a.y);
        o[4] = bf16lo(a.z); o[5] = bf16hi(a.z); o[6] = bf16lo(a.w); o[7] = bf16hi(a.w);
    } else if constexpr (KV == ART_I8) {
        const u2* p = reinterpret_cast<const u2*>(static_cast<const int8_t*>(base) + off);
        u2 a = __builtin_nontemporal_load(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[i] = sbyte(a.x, i);
            o[4 + i] = sbyte(a.y, i);
        }
    } else {
        // int4: element e in the low (even e) or high (odd e) nibble of byte e / 2
        const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(base) + off / 2);
        const uint32_t a = __builtin_nontemporal_load(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = snib(a, i);
    }
}

// APL consecutive elements (APL = 1 or 2) starting at element `off`, widened to fp32.
template <int KV, int APL>
__device__ __forceinline__ void load_small(const void* base, long long off, float (&o)[APL]) {
    if constexpr (KV == ART_F32) {
        const float* p = static_cast<const float*>(base) + off;
        if constexpr (APL == 2) {
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
    } else if constexpr (KV == ART_I8) {
        const int8_t* p = static_cast<const int8_t*>(base) + off;
        if constexpr (APL == 2) {
            uint16_t w = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
            o[0] = sbyte(w, 0); o[1] = sbyte(w, 1);
        } else {
            o[0] = (float)__builtin_nontemporal_load(p);
        }
    } else {
        const uint32_t w = __builtin_nontemporal_load(static_cast<const uint8_t*>(base) + off / 2);
        if constexpr (APL == 2) {  // off is even: both nibbles of one byte
            o[0] = snib(w, 0); o[1] = snib(w, 1);
        } else {
            o[0] = snib(w, (int)(off & 1));
        }
    }
}

// The sequence group grp = (b, kv head g) reads -- its length, block-table
// row and tile list: row b's, or with per-head tables its own, i.e.
// grp / seq_div with seq_div = Hkv or 1.  The quotient is taken by a
// multiply-high and shift with the host's constants (exact for grp < 2^31),
// cheap enough to recompute wherever a tile needs it.
__device__ __forceinline__ int seq_of(const Params& P, int grp) {
    return (int)(((unsigned long long)(unsigned)grp * P.seq_m) >> P.seq_sh);
}

// Query heads of group grp: G, except that when a KV head's gq query heads do
// not split evenly (kv_shift > 0) its last group holds fewer.
__device__ __forceinline__ int heads_in(const Params& P, int grp) {
    const int s = (grp % P.Hkv) & ((1 << P.kv_shift) - 1);
    return min(P.G, P.gq - s * P.G);
}
// Row of q, out and tiles_used ([batch][query head]) of head h of group grp.
__device__ __forceinline__ long long qrow(const Params& P, int grp, int h) {
    const int b = grp / P.Hkv, gv = grp % P.Hkv;
    return (long long)b * P.Hq + (long long)(gv >> P.kv_shift) * P.gq + (gv & ((1 << P.kv_shift) - 1)) * P.G + h;
}

// Row index of cached position j of (b, kv head g); ok=false on an invalid block id.
// g counts groups (query-head splits of a KV head, kv_shift); the cache has
// hkv_cache heads and group g reads head g >> kv_shift.
__device__ __forceinline__ long long row_index(const Params& P, int b, int g, int j, bool& ok) {
    const int gc = g >> P.kv_shift;
    if (P.block_size == 0) return ((long long)b * P.hkv_cache + gc) * P.max_ctx + j;
    const int blk = P.block_table[(long long)seq_of(P, b * P.Hkv + g) * P.mbps + j / P.block_size];
    if (blk < 0 || blk >= P.num_blocks) {
        ok = false;
        return 0;
    }
    return ((long long)blk * P.hkv_cache + gc) * P.block_size + (j % P.block_size);
}

// The tile visited at step t of sequence sq (seq_of), which has nt tiles.  The tile sequence
// may be reordered (ART summary, section 2.4: recency- or importance-first;
// the result does not depend on the order, and block 0, the attention sink,
// is evaluated first): ascending; tile 0 then the most recent first; or the
// caller's list, whose step 0 must name tile 0 and later steps tiles
// 1..nt-1 -- any other entry gives -1 and the tile reports an error.  Steps
// past the row's tiles map to themselves (no position of them exists).
__device__ __forceinline__ int tile_at(const Params& P, int sq, int nt, int t) {
    if (P.order == ART_ORDER_ASCENDING || t < 0 || t >= nt) return t;
    if (P.order == ART_ORDER_RECENT) return t == 0 ? 0 : nt - t;
    const int e = P.tile_perm[(long long)sq * P.perm_stride + t];
    if (t == 0) return e == 0 ? 0 : -1;
    return (e >= 1 && e < nt) ? e : -1;
}

// ------------------------------------------------------------------ tile output
//
// "Fold mapping", shared by every consumer of partials: lane l serves head
// hb*4 + (l >> 4) of head block hb and head dims 8*(l & 15) .. +7.
template <int HBM>
struct TileOutT {
    float m[kMaxG];   // tile max per head (wave-uniform)
    float l[kMaxG];   // tile softmax sum per head, relative to m (wave-uniform)
    float a[HBM][8];  // V accumulator, fold mapping (head blocks 0..HBM-1)
    float mf[HBM];    // streamed tiles: m of the lane's head in the fold mapping
    float lf[HBM];    // streamed tiles: l of the lane's head in the fold mapping
    int err;          // an invalid block id was met
    int kept;         // V rows loaded
};

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

// ------------------------------------------------------------------ generic tile (vector ALU)
//
// Any dtype, head dim 64 or 128, G <= 16.  Lane l scores token t*T + l (+64),
// the tile max and sum per head are wave reductions, the kept weights go
// through LDS and the V accumulation maps lane l to head dims l*APL..; the
// accumulator is finally transposed to the fold mapping through LDS.
template <int D, int KV>
struct GenericTile {
    static constexpr int APL = D / 64;
    static constexpr int HBM = 4;
    using Out = TileOutT<HBM>;

    __host__ __device__ static size_t lds_floats(const Params& P) {
        return (size_t)P.G * D + (size_t)(P.G * P.T > P.G * D ? P.G * P.T : P.G * D);
    }

    float* q_lds;
    float* p_lds;

    __device__ __forceinline__ void load_q(const Params& P, int b, int g, float* lds) {
        q_lds = lds;
        p_lds = lds + P.G * D;
        const int lane = lane_id();
        for (int i = lane; i < P.G * D; i += 64) {
            const long long off = ((long long)b * P.Hq + (long long)g * P.G) * D + i;
            q_lds[i] = P.q_dtype == ART_F32 ? static_cast<const float*>(P.q)[off]
                                            : bf16lo(static_cast<const uint16_t*>(P.q)[off]);
        }
        wave_lds_sync();
    }

    template <class Hook>
    __device__ __forceinline__ bool compute(const Params& P, int b, int g, int n, int t, Hook&& hook, Out& o) {
        const int lane = lane_id();
        const int G = P.G, T = P.T;
        const int pt = tile_at(P, seq_of(P, b * P.Hkv + g), (n + T - 1) / T, t);  // the tile of step t
        const int j0 = pt * T;
        float s[2][kMaxG];
        bool valid[2];
        int bad = pt < 0;
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const int jj = ps * 64 + lane;
            const int j = j0 + jj;
            valid[ps] = pt >= 0 && jj < T && j < n;
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) s[ps][h] = 0.f;
            if (valid[ps]) {
                bool ok = true;
                const long long r = row_index(P, b, g, j, ok);
                if (!ok) {
                    bad = 1;
                    valid[ps] = false;
                } else {
                    const float sc = (KV == ART_I8 || KV == ART_I4 ? f16_to_f32(P.ks[r]) : 1.f) * P.inv_sqrt_d;
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
        o.err = __ballot(bad) != 0ull;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            float mx = kNegInf;
#pragma unroll
            for (int ps = 0; ps < 2; ++ps)
                if (valid[ps]) mx = fmaxf(mx, s[ps][h]);
            o.m[h] = h < G ? wave_max(mx) : kNegInf;
        }
        float Mt[kMaxG];
        if (!hook(o.m, Mt)) return false;
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
                    const float p = valid[ps] ? expf(s[ps][h] - o.m[h]) : 0.f;
                    lsum[h] += p;
                    const bool keep = valid[ps] && (!P.vskip || s[ps][h] - Mt[h] >= P.v_skip_ln);
                    row_keep |= keep;
                    if (jj < T) p_lds[h * T + jj] = keep ? p : 0.f;
                }
            }
            keep_mask[ps] = __ballot(row_keep);
        }
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) o.l[h] = h < G ? wave_sum(lsum[h]) : 0.f;
        wave_lds_sync();
        float acc[kMaxG][APL];
#pragma unroll
        for (int h = 0; h < kMaxG; ++h)
#pragma unroll
            for (int i = 0; i < APL; ++i) acc[h][i] = 0.f;
        o.kept = __builtin_popcountll(keep_mask[0]) + __builtin_popcountll(keep_mask[1]);
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            uint64_t m = keep_mask[ps];
            while (m) {
                const int jj = ps * 64 + __builtin_ctzll(m);
                m &= m - 1;
                bool ok = true;
                const long long r = row_index(P, b, g, j0 + jj, ok);
                const float vsc = KV == ART_I8 || KV == ART_I4 ? f16_to_f32(P.vs[r]) : 1.f;
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
        // transpose the accumulator to the fold mapping (p_lds is free again)
        wave_lds_sync();
        float* x = p_lds;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h)
            if (h < G)
#pragma unroll
                for (int i = 0; i < APL; ++i) x[h * D + lane * APL + i] = acc[h][i];
        wave_lds_sync();
        const int hl = lane >> 4, cid = lane & 15;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            const int h = hb * 4 + hl;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                o.a[hb][j] = (h < G && 8 * cid < D) ? x[h * D + 8 * cid + j] : 0.f;
        }
        wave_lds_sync();
        return true;
    }
};

// ------------------------------------------------------------------ matrix-core tile
//
// bf16 or int8 cache, head dim 128, bf16 queries, G <= 8, tile of PAGES
// 16-token pages.  Scores: lane l holds the A operand row l&15 of a page
// (128-bit loads of head dims 32s + 8(l>>4) .. +7 for s = 0..3) and the B
// operand column l&15 = head; the 16x16 result gives lane l the scores of
// tokens 4(l>>4)+i of that page for head l&15.  P.V: lane l accumulates head
// dims 8(l&15)..+7 over rows 4v + (l>>4) of every page, reading the kept
// weights of its rows from LDS; the four row groups are summed through LDS
// into the fold mapping at the end.
template <int KV, int PAGES, int GMAX>
struct FastTile {
    static constexpr int T = 16 * PAGES;
    static constexpr int D = 128;
    static constexpr int EB = KV == ART_I8 ? 1 : 2;  // bytes per cache element
    static constexpr int HBM = GMAX / 4;
    using Out = TileOutT<HBM>;
    typedef typename std::conditional<KV == ART_I8, u2, u4>::type kvec;  // 8 elements

    __host__ __device__ static size_t lds_floats(const Params& P) {
        return (size_t)(T * GMAX > 4 * P.G * D ? T * GMAX : 4 * P.G * D);
    }

    bf16x8 qB[4];
    float* lds;

    __device__ __forceinline__ void load_q(const Params& P, int b, int g, float* lds_wave) {
        lds = lds_wave;
        const int lane = lane_id(), h = lane & 15, kg = lane >> 4;
        const uint16_t* q = static_cast<const uint16_t*>(P.q);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u4 v = {0u, 0u, 0u, 0u};
            if (h < P.G)
                v = *reinterpret_cast<const u4*>(q + ((long long)b * P.Hq + (long long)g * P.G + h) * D +
                                                 32 * s + 8 * kg);
            qB[s] = __builtin_bit_cast(bf16x8, v);
        }
    }

    __device__ static kvec load_kv(const void* base, long long elem) {
        return __builtin_nontemporal_load(
            reinterpret_cast<const kvec*>(static_cast<const char*>(base) + elem * EB));
    }

    template <class Hook>
    __device__ __forceinline__ bool compute(const Params& P, int b, int g, int n, int t, Hook&& hook, Out& o) {
        const int lane = lane_id(), r16 = lane & 15, rg = lane >> 4;
        const int G = P.G;
        const int pt = tile_at(P, seq_of(P, b * P.Hkv + g), (n + T - 1) / T, t);  // the tile of step t
        const int tok0 = pt * T;
        // pages of the tile: first row index and validity (wave-uniform)
        long long prow[PAGES];
        bool pval[PAGES];
        int bad = pt < 0;
#pragma unroll
        for (int p = 0; p < PAGES; ++p) {
            const int tokp = tok0 + 16 * p;
            pval[p] = pt >= 0 && tokp < n;
            prow[p] = 0;
            if (pval[p]) {
                bool ok = true;
                prow[p] = row_index(P, b, g, tokp, ok);
                if (!ok) { pval[p] = false; bad = 1; }
            }
        }
        // K loads (A operand layout) and, without V skip, the V loads right away
        const kvec zero = {};
        kvec kr[PAGES][4], vr[PAGES][4];
#pragma unroll
        for (int p = 0; p < PAGES; ++p)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kr[p][s] = pval[p] ? load_kv(P.k, (prow[p] + r16) * D + 32 * s + 8 * rg) : zero;
        if (!P.vskip) {
#pragma unroll
            for (int p = 0; p < PAGES; ++p)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = 4 * v + rg;
                    vr[p][v] = (pval[p] && tok0 + 16 * p + row < n)
                                   ? load_kv(P.v, (prow[p] + row) * D + 8 * r16) : zero;
                }
        }
        // int8 key scales of the score rows 4*rg + i of every page
        float ksc[PAGES][4];
#pragma unroll
        for (int p = 0; p < PAGES; ++p)
#pragma unroll
            for (int i = 0; i < 4; ++i) ksc[p][i] = P.inv_sqrt_d;
        if constexpr (KV == ART_I8) {
#pragma unroll
            for (int p = 0; p < PAGES; ++p) {
                if (pval[p]) {
                    const u2 w = *reinterpret_cast<const u2*>(P.ks + prow[p] + 4 * rg);
                    ksc[p][0] = f16_to_f32(w.x & 0xffff) * P.inv_sqrt_d;
                    ksc[p][1] = f16_to_f32(w.x >> 16) * P.inv_sqrt_d;
                    ksc[p][2] = f16_to_f32(w.y & 0xffff) * P.inv_sqrt_d;
                    ksc[p][3] = f16_to_f32(w.y >> 16) * P.inv_sqrt_d;
                }
            }
        }
        // scores on the matrix cores
        float s[PAGES][4];
        float mx = kNegInf;
#pragma unroll
        for (int p = 0; p < PAGES; ++p) {
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                bf16x8 a;
                if constexpr (KV == ART_I8) {
                    const u2 w = kr[p][st];
                    u4 c;
                    c.x = bf16_pair(sbyte(w.x, 0), sbyte(w.x, 1));
                    c.y = bf16_pair(sbyte(w.x, 2), sbyte(w.x, 3));
                    c.z = bf16_pair(sbyte(w.y, 0), sbyte(w.y, 1));
                    c.w = bf16_pair(sbyte(w.y, 2), sbyte(w.y, 3));
                    a = __builtin_bit_cast(bf16x8, c);
                } else {
                    a = __builtin_bit_cast(bf16x8, kr[p][st]);
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[st], acc, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = pval[p] && tok0 + 16 * p + 4 * rg + i < n;
                s[p][i] = valid ? acc[i] * ksc[p][i] : kNegInf;
                mx = fmaxf(mx, s[p][i]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));  // tile max of head r16, in every lane of that head
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) o.m[h] = (h < GMAX && h < G) ? __shfl(mx, h) : kNegInf;
        float Mt[kMaxG];
        if (!hook(o.m, Mt)) return false;
        float mt = Mt[0];
#pragma unroll
        for (int h = 1; h < GMAX; ++h)
            if (r16 == h) mt = Mt[h];
        // weights: exp(s - tile max); the V skip compares against the running max
        float* pl = lds;  // [T tokens][GMAX heads]
        float lsum = 0.f;
        uint64_t keep_rows = 0;
#pragma unroll
        for (int p = 0; p < PAGES; ++p) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = s[p][i] != kNegInf;
                const float pr = valid ? expf(s[p][i] - mx) : 0.f;
                lsum += pr;
                const bool keep = valid && r16 < G && (!P.vskip || s[p][i] - mt >= P.v_skip_ln);
                const int tok = 16 * p + 4 * rg + i;
                if (r16 < GMAX) pl[tok * GMAX + r16] = keep ? pr : 0.f;
                const uint64_t bal = __ballot(keep);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if ((bal >> (16 * q)) & 0xffffull) keep_rows |= 1ull << (16 * p + 4 * q + i);
            }
        }
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) o.l[h] = (h < GMAX && h < G) ? __shfl(lsum, h) : 0.f;
        o.err = __ballot(bad) != 0ull;
        o.kept = __builtin_popcountll(keep_rows);
        if (P.vskip) {
            // V rows no head keeps are neither loaded nor dequantised
#pragma unroll
            for (int p = 0; p < PAGES; ++p)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = 4 * v + rg;
                    vr[p][v] = (pval[p] && ((keep_rows >> (16 * p + row)) & 1ull))
                                   ? load_kv(P.v, (prow[p] + row) * D + 8 * r16) : zero;
                }
        }
        wave_lds_sync();
        // P.V on the vector ALUs
        float acc[GMAX][8];
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
#pragma unroll
        for (int p = 0; p < PAGES; ++p) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tok = 16 * p + 4 * v + rg;
                float pw[GMAX];
                const f4 w0 = *reinterpret_cast<const f4*>(pl + tok * GMAX);
                pw[0] = w0.x; pw[1] = w0.y; pw[2] = w0.z; pw[3] = w0.w;
                if constexpr (GMAX == 8) {
                    const f4 w1 = *reinterpret_cast<const f4*>(pl + tok * GMAX + 4);
                    pw[4] = w1.x; pw[5] = w1.y; pw[6] = w1.z; pw[7] = w1.w;
                }
                float vf[8];
                if constexpr (KV == ART_I8) {
                    const float vs =
                        (pval[p] && tok0 + tok < n) ? f16_to_f32(P.vs[prow[p] + 4 * v + rg]) : 0.f;
#pragma unroll
                    for (int h = 0; h < GMAX; ++h) pw[h] *= vs;
                    const u2 w = vr[p][v];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        vf[k] = sbyte(w.x, k);
                        vf[4 + k] = sbyte(w.y, k);
                    }
                } else {
                    const u4 w = vr[p][v];
                    vf[0] = bf16lo(w.x); vf[1] = bf16hi(w.x); vf[2] = bf16lo(w.y); vf[3] = bf16hi(w.y);
                    vf[4] = bf16lo(w.z); vf[5] = bf16hi(w.z); vf[6] = bf16lo(w.w); vf[7] = bf16hi(w.w);
                }
#pragma unroll
                for (int h = 0; h < GMAX; ++h) {
                    if (h < G) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(pw[h], vf[j], acc[h][j]);
                    }
                }
            }
        }
        // sum the four row groups into the fold mapping
        wave_lds_sync();
        float* x = lds;  // [4 row groups][G][128]
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            if (h < G) {
                f4* d = reinterpret_cast<f4*>(x + (rg * G + h) * D + 8 * r16);
                d[0] = f4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
                d[1] = f4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
            }
        }
        wave_lds_sync();
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            const int h = hb * 4 + rg;
#pragma unroll
            for (int j = 0; j < 8; ++j) o.a[hb][j] = 0.f;
            if (h < G) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f4* src = reinterpret_cast<const f4*>(x + (q * G + h) * D + 8 * r16);
                    const f4 u = src[0], w = src[1];
                    o.a[hb][0] += u.x; o.a[hb][1] += u.y; o.a[hb][2] += u.z; o.a[hb][3] += u.w;
                    o.a[hb][4] += w.x; o.a[hb][5] += w.y; o.a[hb][6] += w.z; o.a[hb][7] += w.w;
                }
            }
        }
        wave_lds_sync();
        return true;
    }
};

// ------------------------------------------------------------------ streamed matrix-core tiles
//
// bf16 or int8 cache, head dim 128, bf16 queries, G <= GMAX (4 or 8), tiles
// of 64 tokens, no V skip.  A wave streams 32-token units (two 16-token
// pages) through a two-deep pipeline: while one unit is consumed, the next
// one is loading.  Every load instruction of a wave reads whole rows (1 KB of
// contiguous memory for bf16):
//  * K goes straight to LDS (global_load_lds_dwordx4, no registers) with the
//    16-byte chunks of each row permuted by XOR with the row index, so the
//    matrix-core operand reads below are free of bank conflicts;
//  * V goes to registers in the layout the P.V accumulation uses.
// Scores: lane l reads from LDS the A operand row l&15 of a page (head dims
// 32s + 8(l>>4) .. +7 for s = 0..3) and holds the B operand column l&15 =
// head (queries, heads padded to 16 columns); the 16x16 result gives lane l
// the scores of tokens 4(l>>4)+i of the page for head l&15.  P.V: lane l
// accumulates head dims 8(l&15)..+7 over rows 4v + (l>>4) of each page, with
// the weights of its rows read from LDS.  Units of one tile (ART mode) or of
// a whole split range (full mode) accumulate into one running (max, sum,
// accumulator) state that flush() reduces into the fold mapping.  ORD: the
// art_order the call visits the tiles in (tile_at), fixed at compile time so
// that each instance carries only its own remap (none for ascending).
template <int KV, int GMAX, int ORD = ART_ORDER_ASCENDING, int NB = 2>
struct Stream {
    static constexpr int D = 128, UP = 2, T = 64, PAGES = 4;
    static constexpr int ORDER = ORD;
    static constexpr int KVT = KV, GM = GMAX;
    static constexpr int NBUF = NB;  // unit buffers (a tile is two units: NB = 4 holds two tiles)
    static_assert(PAGES == kStepPages, "step-table records hold one block id per page");
    static constexpr bool SCALED = KV == ART_I8 || KV == ART_I4;  // codes times per-row fp16 scales
    static constexpr int HBM = GMAX / 4;
    static constexpr int HEADS = GMAX;           // query heads per KV head at most
    static constexpr int ROWB = KV == ART_I4 ? D / 2 : KV == ART_I8 ? D : 2 * D;  // bytes of one cache row
    static constexpr int PAGEB = 16 * ROWB;      // bytes of one 16-row page
    static constexpr int KDMA = PAGEB / 1024;    // LDS-direct loads per page
    static constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
    // vector-memory instructions one issue() emits (all unconditional)
    static constexpr int OPS = UP * (4 + KDMA + (SCALED ? 2 : 0));
    // resident waves per SIMD the register budget is cut for (two when it fits without heavy spills)
    static constexpr int MIN_WAVES = GMAX == 4 ? 2 : 1;
    // waves of a team (one work-group, one CU): as many as are resident on a CU
    static constexpr int TEAM = 4 * MIN_WAVES;
    using Out = TileOutT<HBM>;
    // 8 elements of a V row
    typedef typename std::conditional<KV == ART_I4, uint32_t,
                                      typename std::conditional<KV == ART_I8, u2, u4>::type>::type vvec;

    static constexpr int LDS_FLOATS = (NB * UP * PAGEB) / 4;
    __host__ __device__ static size_t lds_floats(const Params&) { return LDS_FLOATS; }

    struct TileRef {             // one tile of one group (wave-uniform)
        int grp, t, n;
        long long prow[PAGES];   // row index of the first token of each page
        int pmask;               // bit p: page p starts below n and has a valid block
        int err;                 // an invalid block id was met in the tile
    };

    vvec vb[NB][UP][4];
    // int8/int4: the fp16 key and value scales of the lane's four rows per
    // page, as loaded (two per word); widened where they are used, so that no
    // wait for their loads sits in issue() (the wait counter is in order: it
    // would also wait for every load issued before them)
    u2 ksr[NB][UP];
    u2 vsr[NB][UP];
    // scale i (0..3) of a pair of words
    __device__ __forceinline__ static float scale_of(const u2& w, int i) {
        const uint32_t x = i < 2 ? w.x : w.y;
        return f16_to_f32((i & 1) ? (uint16_t)(x >> 16) : (uint16_t)(x & 0xffff));
    }
    bf16x8 qB[4];
    float m_run, l_run;          // per head (lane & 15): running max and (this lane's part of the) sum
    // P.V accumulators in the matrix-core output layout: cacc[j][c] of lane
    // (n, mb) = (lane & 15, lane >> 4) holds head 4mb + c, head dim 8n + j
    f4 cacc[8];
    char* kl;                    // LDS: [NB buffers][UP pages][PAGEB]

    __device__ __forceinline__ void init(float* lds_wave) {
        kl = reinterpret_cast<char*>(lds_wave);
        reset();
    }

    __device__ __forceinline__ void reset() {
        m_run = kNegInf;
        l_run = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) cacc[j] = f4{0.f, 0.f, 0.f, 0.f};
    }

    __device__ __forceinline__ void load_q(const Params& P, int grp) {
        const int lane = lane_id(), h = lane & 15, kg = lane >> 4;
        const uint16_t* q = static_cast<const uint16_t*>(P.q);
        const int hv = heads_in(P, grp);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u4 v = {0u, 0u, 0u, 0u};
            if (h < hv) v = *reinterpret_cast<const u4*>(q + qrow(P, grp, h) * D + 32 * s + 8 * kg);
            qB[s] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // the tile visited at step t (tile_at) of group grp's row of n positions
    __device__ __forceinline__ static int phys(const Params& P, int grp, int n, int t) {
        if constexpr (ORD == ART_ORDER_ASCENDING) {
            return t;
        } else if constexpr (ORD == ART_ORDER_RECENT) {
            const int nt = (n + T - 1) / T;
            return (t <= 0 || t >= nt) ? t : nt - t;
        } else {
            return tile_at(P, seq_of(P, grp), (n + T - 1) / T, t);
        }
    }
    // whether tile index pt names a tile: a bad list entry gives -1
    __device__ __forceinline__ static bool named(int pt) { return ORD != ART_ORDER_LIST || pt >= 0; }
    // positions of a resolved tile
    __device__ __forceinline__ static int rows_in(const TileRef& r) {
        return named(r.t) ? max(0, min(T, r.n - r.t * T)) : 0;
    }

    // r: the tile visited at step t of group grp (r.t is the tile itself)
    __device__ __forceinline__ static void resolve(const Params& P, int grp, int t, TileRef& r) {
        const int b = grp / P.Hkv, g = grp % P.Hkv;
        if constexpr (ORD == ART_ORDER_LIST) {
            const int n = P.ctx_lens[seq_of(P, grp)];
            resolve_from(P, grp, n, t, fetch_blocks(P, grp, n, t), r);
            return;
        }
        r.grp = grp;
        r.n = P.ctx_lens[seq_of(P, grp)];
        r.t = phys(P, grp, r.n, t);
        r.pmask = 0;
        r.err = !named(r.t);
#pragma unroll
        for (int p = 0; p < PAGES; ++p) {
            const int tokp = r.t * T + 16 * p;
            r.prow[p] = 0;
            if (named(r.t) && tokp < r.n) {
                bool ok = true;
                r.prow[p] = row_index(P, b, g, tokp, ok);
                if (ok) r.pmask |= 1 << p;
                else r.err = 1;
            }
        }
    }

    // The block ids of tile t (paged caches): lane p < PAGES loads page p's
    // entry with a vector load, so that it can be issued well before the tile
    // is resolved, and complete with the tile loads issued before it.
    //
    // A caller's tile list (ORD == ART_ORDER_LIST) reads the step table
    // instead: lanes 0..PAGES-1 the pages' block ids, lane PAGES the tile; for
    // a step past the row's tiles lane PAGES holds the step itself.
    __device__ __forceinline__ static int fetch_blocks(const Params& P, int grp, int n, int t) {
        const int lane = lane_id(), sq = seq_of(P, grp);
        if constexpr (ORD == ART_ORDER_LIST) {
            int v = lane == PAGES ? t : 0;
            if (lane <= PAGES && t < (n + T - 1) / T) v = P.steps[((long long)sq * P.nt_max + t) * kStepW + lane];
            return v;
        }
        const int pt = phys(P, grp, n, t);
        const int tokp = pt * T + 16 * lane;
        int blk = 0;
        if (P.block_size && lane < PAGES && named(pt) && tokp < n)
            blk = P.block_table[(long long)sq * P.mbps + (unsigned)tokp / (unsigned)P.block_size];
        return blk;
    }

    // fetch_blocks() into LDS (dst[p] = page p's entry) with LDS-direct loads,
    // so that the ids hold no register while they are in flight; read them
    // (resolve_lds) once the wave's loads have landed
    __device__ __forceinline__ static void fetch_blocks_lds(const Params& P, int grp, int n, int t, int* dst) {
        const int lane = lane_id(), sq = seq_of(P, grp);
        if constexpr (ORD == ART_ORDER_LIST) {
            if (lane <= PAGES && t < (n + T - 1) / T)
                __builtin_amdgcn_global_load_lds(P.steps + ((long long)sq * P.nt_max + t) * kStepW + lane,
                                                 (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
            return;
        }
        const int pt = phys(P, grp, n, t);
        const int tokp = pt * T + 16 * lane;
        if (P.block_size && lane < PAGES && named(pt) && tokp < n)
            __builtin_amdgcn_global_load_lds(P.block_table + (long long)sq * P.mbps + (unsigned)tokp / (unsigned)P.block_size,
                                             (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
    }
    __device__ __forceinline__ static void resolve_lds(const Params& P, int grp, int n, int t, const int* src,
                                                       TileRef& r) {
        const int lane = lane_id();
        const int blkv = lane < PAGES || (ORD == ART_ORDER_LIST && lane == PAGES) ? src[lane] : 0;
        resolve_from(P, grp, n, t, blkv, r);
    }

    // resolve() from the block ids fetch_blocks() returned for tile t: lane
    // p < PAGES works out page p (validity, row index) in one vector pass, and
    // the results are read back as wave-uniform values
    __device__ __forceinline__ static void resolve_from(const Params& P, int grp, int n, int t, int blkv, TileRef& r) {
        const int lane = lane_id();
        const int b = grp / P.Hkv, g = grp % P.Hkv, gc = g >> P.kv_shift;
        r.grp = grp;
        if constexpr (ORD == ART_ORDER_LIST)
            r.t = t < (n + T - 1) / T ? __builtin_amdgcn_readlane(blkv, PAGES) : t;
        else
            r.t = phys(P, grp, n, t);
        r.n = n;
        const int tokp = r.t * T + 16 * lane;
        const bool in = lane < PAGES && named(r.t) && tokp < n;
        bool ok = in;
        long long pr;
        if (P.block_size == 0) {
            pr = ((long long)b * P.hkv_cache + gc) * P.max_ctx + tokp;
        } else {
            ok = in && blkv >= 0 && blkv < P.num_blocks;
            pr = ((long long)blkv * P.hkv_cache + gc) * P.block_size + (unsigned)tokp % (unsigned)P.block_size;
        }
        const uint64_t okm = __ballot(ok), inm = __ballot(in);
        r.pmask = (int)(okm & ((1u << PAGES) - 1));
        r.err = !named(r.t) || ((inm & ~okm) & ((1u << PAGES) - 1)) != 0;
        const int lo = (int)(uint32_t)pr, hi = (int)(pr >> 32);
#pragma unroll
        for (int p = 0; p < PAGES; ++p) {
            const long long v = ((long long)__builtin_amdgcn_readlane(hi, p) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane(lo, p);
            r.prow[p] = ((okm >> p) & 1) ? v : 0;
        }
    }

    // Issue the loads of unit u (pages 2u, 2u+1) of tile r into buffer BUF:
    // exactly OPS unconditional vector-memory instructions.  Pages outside the
    // sequence (or with an invalid block) read the first rows of the cache
    // instead; consume() masks them.
    // WITH_V = false leaves the V rows out (the V skip loads them once the
    // scores are known: issue_v)
    template <int BUF, bool WITH_V = true>
    __device__ __forceinline__ void issue(const Params& P, const TileRef& r, int u) {
        const int lane = lane_id(), r16 = lane & 15, rg = lane >> 4;
        // keep every load of this unit after the previous unit's LDS reads and
        // before the next unit's loads: the waits count instructions in order
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pp = 0; pp < UP; ++pp) {
            const int p = UP * u + pp;
            const long long pr = ((r.pmask >> p) & 1) ? r.prow[p] : 0;
            const char* vbase = static_cast<const char*>(P.v) + pr * ROWB;
            // lane (r16, rg) holds rows 4rg .. 4rg + 3 of the page, the tokens
            // whose scores it computes, head dims 8 r16 .. 8 r16 + 7
            if constexpr (WITH_V) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = 4 * rg + v;
                    vb[BUF][pp][v] = __builtin_nontemporal_load(
                        reinterpret_cast<const vvec*>(vbase + row * ROWB + (ROWB / 16) * r16));
                }
            }
            if constexpr (SCALED) {
                // the value scales of rows 4rg .. 4rg + 3 and the key scales of
                // the score rows (the same rows): one 8-byte load each
                vsr[BUF][pp] = *reinterpret_cast<const u2*>(P.vs + pr + 4 * rg);
                ksr[BUF][pp] = *reinterpret_cast<const u2*>(P.ks + pr + 4 * rg);
            }
            const char* kbase = static_cast<const char*>(P.k) + pr * ROWB;
            char* dst = kl + (BUF * UP + pp) * PAGEB;
#pragma unroll
            for (int i = 0; i < KDMA; ++i) {
                // 1 KB per instruction: LDS chunk (row, c) receives global chunk c ^ (row % CPR)
                const int row = i * (1024 / ROWB) + lane / CPR;
                const int c = (lane % CPR) ^ (row % CPR);
                __builtin_amdgcn_global_load_lds(kbase + row * ROWB + 16 * c,
                                                 (__attribute__((address_space(3))) void*)(dst + 1024 * i),
                                                 16, 0, 2 /* nt */);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // V rows (all four of the lane's rows per page) and, for int8/int4, their
    // value scales: UP * (4 + SCALED) instructions.  K is not loaded (the
    // scores come from elsewhere: consume_given).
    template <int BUF>
    __device__ __forceinline__ void issue_vs(const Params& P, const TileRef& r, int u) {
        const int lane = lane_id(), r16 = lane & 15, rg = lane >> 4;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pp = 0; pp < UP; ++pp) {
            const int p = UP * u + pp;
            const long long pr = ((r.pmask >> p) & 1) ? r.prow[p] : 0;
            const char* vbase = static_cast<const char*>(P.v) + pr * ROWB;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                vb[BUF][pp][v] = __builtin_nontemporal_load(
                    reinterpret_cast<const vvec*>(vbase + (4 * rg + v) * ROWB + (ROWB / 16) * r16));
            if constexpr (SCALED) vsr[BUF][pp] = *reinterpret_cast<const u2*>(P.vs + pr + 4 * rg);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // Fold unit u into the running state from its scores s (the layout
    // scores() returns: token 16pp + 4(lane>>4) + i, head lane & 15, -inf
    // outside the sequence), its V already loaded and landed.
    template <int BUF>
    __device__ __forceinline__ void consume_given(const Params& P, const TileRef& r, int u, const float (&s)[UP][4]) {
        float mu = kNegInf;
#pragma unroll
        for (int pp = 0; pp < UP; ++pp)
#pragma unroll
            for (int i = 0; i < 4; ++i) mu = fmaxf(mu, s[pp][i]);
        mu = fmaxf(mu, __shfl_xor(mu, 16));
        mu = fmaxf(mu, __shfl_xor(mu, 32));
        const float m_new = fmaxf(m_run, mu);
        const float alpha = m_run == kNegInf ? 0.f : exp_fast(m_run - m_new);
        float lsum = 0.f;
        float pw[UP][4];
#pragma unroll
        for (int pp = 0; pp < UP; ++pp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pw[pp][i] = s[pp][i] != kNegInf ? exp_fast(s[pp][i] - m_new) : 0.f;
                lsum += pw[pp][i];
            }
        l_run = fmaf(alpha, l_run, lsum);
        m_run = m_new;
        rescale(alpha);
        const bool full = ((r.pmask >> (UP * u)) & 3) == 3 && r.t * T + 32 * (u + 1) <= r.n;
        if (full) pv_mfma<BUF, false>(P, r, u, pw);
        else pv_mfma<BUF, true>(P, r, u, pw);
    }

    // The V rows of unit u that some head keeps: bit v of keep[pp] is this
    // lane's row 4rg + v of page pp.  A row left out is neither loaded nor
    // dequantised; its registers read as zero.
    template <int BUF>
    __device__ __forceinline__ void issue_v(const Params& P, const TileRef& r, int u, const unsigned (&keep)[UP]) {
        const int lane = lane_id(), r16 = lane & 15, rg = lane >> 4;
#pragma unroll
        for (int pp = 0; pp < UP; ++pp) {
            const int p = UP * u + pp;
            const long long pr = ((r.pmask >> p) & 1) ? r.prow[p] : 0;
            const char* vbase = static_cast<const char*>(P.v) + pr * ROWB;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                vvec x{};
                if ((keep[pp] >> v) & 1)
                    x = __builtin_nontemporal_load(
                        reinterpret_cast<const vvec*>(vbase + (4 * rg + v) * ROWB + (ROWB / 16) * r16));
                vb[BUF][pp][v] = x;
            }
        }
    }

    template <int N>
    __device__ static void wait_vm() {
        static_assert(N < 64, "vmcnt has 6 bits");
        __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    }

    // Scores of unit u (loaded in buffer BUF): s[pp][i] is token 16pp + 4(lane>>4) + i
    // of the unit for head lane & 15 (-inf outside the sequence); returns the
    // unit's max per head (lane & 15), over the whole wave.
    template <int BUF>
    __device__ __forceinline__ float scores(const Params& P, const TileRef& r, int u, float (&s)[UP][4]) {
        const int lane = lane_id(), r16 = lane & 15, rg = lane >> 4;
        float mu = kNegInf;
#pragma unroll
        for (int pp = 0; pp < UP; ++pp) {
            const int p = UP * u + pp;
            const char* kp = kl + (BUF * UP + pp) * PAGEB;
            f4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                bf16x8 a;
                if constexpr (KV == ART_I8) {
                    // 8 bytes: head dims 32st + 8rg .. +7 of row r16
                    const int c = (2 * st + (rg >> 1)) ^ (r16 % CPR);
                    const u2 w = *reinterpret_cast<const u2*>(kp + r16 * ROWB + 16 * c + 8 * (rg & 1));
                    u4 cv;
                    cv.x = bf16_pair(sbyte(w.x, 0), sbyte(w.x, 1));
                    cv.y = bf16_pair(sbyte(w.x, 2), sbyte(w.x, 3));
                    cv.z = bf16_pair(sbyte(w.y, 0), sbyte(w.y, 1));
                    cv.w = bf16_pair(sbyte(w.y, 2), sbyte(w.y, 3));
                    a = __builtin_bit_cast(bf16x8, cv);
                } else if constexpr (KV == ART_I4) {
                    // 4 bytes: head dims 32st + 8rg .. +7 of row r16 (two codes per byte)
                    const int c = st ^ (r16 % CPR);
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(kp + r16 * ROWB + 16 * c + 4 * rg);
                    u4 cv;
                    cv.x = bf16_pair(snib(w, 0), snib(w, 1));
                    cv.y = bf16_pair(snib(w, 2), snib(w, 3));
                    cv.z = bf16_pair(snib(w, 4), snib(w, 5));
                    cv.w = bf16_pair(snib(w, 6), snib(w, 7));
                    a = __builtin_bit_cast(bf16x8, cv);
                } else {
                    const int c = (4 * st + rg) ^ r16;
                    a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u4*>(kp + r16 * ROWB + 16 * c));
                }
                a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[st], a4, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = ((r.pmask >> p) & 1) && r.t * T + 16 * p + 4 * rg + i < r.n;
                const float sc = SCALED ? scale_of(ksr[BUF][pp], i) * P.inv_sqrt_d : P.inv_sqrt_d;
                s[pp][i] = valid ? a4[i] * sc : kNegInf;
                mu = fmaxf(mu, s[pp][i]);
            }
        }
        mu = fmaxf(mu, __shfl_xor(mu, 16));
        mu = fmaxf(mu, __shfl_xor(mu, 32));
        return mu;
    }

    // Fold unit u of tile r (loaded in buffer BUF) into the running state.
    // `pending`: the next unit's loads were issued after this one's.
    template <int BUF>
    __device__ __forceinline__ void consume(const Params& P, const TileRef& r, int u, bool pending) {
        if (pending) consume_after<BUF, 1>(P, r, u);
        else consume_after<BUF, 0>(P, r, u);
    }

    // consume() once at least NY units' loads (NY * OPS instructions) were
    // issued after this unit's: waits until at most that many are outstanding
    // (vector-memory operations complete in issue order), fewer when the count
    // does not fit the counter (a longer wait, never a shorter one)
    template <int BUF, int NY>
    __device__ __forceinline__ void consume_after(const Params& P, const TileRef& r, int u) {
        const int lane = lane_id(), r16 = lane & 15, rg = lane >> 4;
        const int G = P.G;
        constexpr int N = NY * OPS < 63 ? NY * OPS : 63;
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<N>();  // this unit's loads, K in LDS included, have landed
        __builtin_amdgcn_sched_barrier(0);
        float s[UP][4];
        const float mu = scores<BUF>(P, r, u, s);
        const float m_new = fmaxf(m_run, mu);
        const float alpha = m_run == kNegInf ? 0.f : exp_fast(m_run - m_new);
        float lsum = 0.f;
        float pw[UP][4];
#pragma unroll
        for (int pp = 0; pp < UP; ++pp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pw[pp][i] = s[pp][i] != kNegInf ? exp_fast(s[pp][i] - m_new) : 0.f;
                lsum += pw[pp][i];
            }
        l_run = fmaf(alpha, l_run, lsum);
        m_run = m_new;
        rescale(alpha);
        // rows outside the sequence hold whatever the fallback rows hold: zero them
        const bool full = ((r.pmask >> (UP * u)) & 3) == 3 && r.t * T + 32 * (u + 1) <= r.n;
        if (full) pv_mfma<BUF, false>(P, r, u, pw);
        else pv_mfma<BUF, true>(P, r, u, pw);
    }

    // cacc of head h *= the factor alpha holds in lane h (the heads' running
    // max rose); skipped when no head's max changed
    __device__ __forceinline__ void rescale(float alpha) {
        if (__ballot(alpha != 1.f) == 0ull) return;
        const int rg = lane_id() >> 4;
        float ai[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), c));
            if constexpr (GMAX == 8) {
                const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 4 + c));
                ai[c] = rg == 1 ? a1 : a0;
            } else {
                ai[c] = a0;  // lanes of rg > 0 hold no head of the group
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) cacc[j][c] *= ai[c];
    }

    // The whole tile r under the V-skip rule, its K (both units) loaded and
    // its V not yet: the scores of both units give the tile max m; chain(m)
    // returns M, the running max through this tile, for the lane's head (lane
    // & 15); a row j of head h enters P.V only when exp(s_hj - M_h) >= v_skip_eps
    // (tested as s_hj - M_h >= ln v_skip_eps, no exponential), while its weight
    // exp(s_hj - m_h) always enters l.  Only the V rows some head of the group
    // keeps are then loaded (row by row, and a unit with none is not
    // multiplied), and the tile becomes the running state (the state is empty
    // before: a tile at a time).  vrows receives the V rows loaded.  Without
    // DEFER the tile's V rows came with its K and are only masked (vrows 0:
    // counted at issue).  Returns the number of (head, row) pairs left out
    // when the call collects statistics (P.stats), else 0.
    template <bool DEFER, class Chain>
    __device__ __forceinline__ int consume_tile_vskip(const Params& P, const TileRef& r, Chain&& chain,
                                                      unsigned& vrows) {
        const int lane = lane_id(), r16 = lane & 15, rg = lane >> 4;
        const int hin = heads_in(P, r.grp);
        __builtin_amdgcn_sched_barrier(0);
        // the tile's K and scales (and the next block ids); with V coming with
        // K, unit 0's scores start once unit 0 has landed (at most the later
        // unit's OPS instructions outstanding: they complete in issue order)
        if constexpr (DEFER) wait_vm<0>();
        else wait_vm<OPS>();
        __builtin_amdgcn_sched_barrier(0);
        float s0[UP][4], s1[UP][4];
        float mu = scores<0>(P, r, 0, s0);
        if constexpr (!DEFER) {
            __builtin_amdgcn_sched_barrier(0);
            wait_vm<0>();
            __builtin_amdgcn_sched_barrier(0);
        }
        mu = fmaxf(mu, scores<1>(P, r, 1, s1));
        const float M = chain(mu);
        float lsum = 0.f;
        int skipped = 0;
        float pw0[UP][4], pw1[UP][4];
        unsigned keep0[UP] = {}, keep1[UP] = {};
        unsigned rows0 = 0, rows1 = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int pp = 0; pp < UP; ++pp)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sv = u ? s1[pp][i] : s0[pp][i];
                    const bool valid = sv != kNegInf;
                    const float pr = valid ? exp_fast(sv - mu) : 0.f;
                    const bool keep = valid && sv - M >= P.v_skip_ln;
                    lsum += pr;
                    (u ? pw1 : pw0)[pp][i] = keep ? pr : 0.f;
                    // row 16pp + 4rg' + i of the unit is loaded when a head of
                    // lane group rg' keeps it
                    const unsigned long long b = __ballot(keep && r16 < hin);
                    const bool rowk = ((b >> (16 * rg)) & 0xffffull) != 0ull;
                    (u ? keep1 : keep0)[pp] |= (unsigned)rowk << i;
                    const unsigned nk = ((b & 0xffffull) != 0) + (((b >> 16) & 0xffffull) != 0) +
                                        (((b >> 32) & 0xffffull) != 0) + ((b >> 48) != 0);
                    (u ? rows1 : rows0) += nk;
                }
        if constexpr (DEFER) {
            issue_v<0>(P, r, 0, keep0);
            issue_v<1>(P, r, 1, keep1);
        }
        // the statistics' count of left-out pairs, only when the caller asks for it
        if (P.stats) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int pp = 0; pp < UP; ++pp)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float sv = u ? s1[pp][i] : s0[pp][i];
                        skipped += (r16 < hin && sv != kNegInf && !(sv - M >= P.v_skip_ln)) ? 1 : 0;
                    }
            skipped = wave_sum_int(skipped);
        }
        l_run = lsum;
        m_run = mu;
        if constexpr (!DEFER) {
            // every row came in: those outside the sequence hold fallback rows
            vrows = 0;
            const bool full0 = (r.pmask & 3) == 3 && r.t * T + 32 <= r.n;
            const bool full1 = ((r.pmask >> UP) & 3) == 3 && r.t * T + 64 <= r.n;
            if (full0) pv_mfma<0, false>(P, r, 0, pw0);
            else pv_mfma<0, true>(P, r, 0, pw0);
            if (full1) pv_mfma<1, false>(P, r, 1, pw1);
            else pv_mfma<1, true>(P, r, 1, pw1);
            return skipped;
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<0>();  // the kept V rows
        __builtin_amdgcn_sched_barrier(0);
        if (rows0) pv_mfma<0, false>(P, r, 0, pw0);
        if (rows1) pv_mfma<1, false>(P, r, 1, pw1);
        vrows = rows0 + rows1;
        return skipped;
    }

    // Element j (head dim 8 r16 + j) of the lane's V rows k and k + 1 of a
    // unit (k = 4pp + i: token 16pp + 4rg + i) as a bf16 pair, row k low.
    template <int BUF>
    __device__ __forceinline__ uint32_t v_pair(int j, int pp, int i) const {
        if constexpr (KV == ART_I8) {
            // int8 codes are exact in bf16 (at most 8 significant bits)
            const u2 a = vb[BUF][pp][i], b = vb[BUF][pp][i + 1];
            const uint32_t wa = j < 4 ? a.x : a.y, wb = j < 4 ? b.x : b.y;
            return bf16_pair(sbyte(wa, j & 3), sbyte(wb, j & 3));
        } else if constexpr (KV == ART_I4) {
            return bf16_pair(snib(vb[BUF][pp][i], j), snib(vb[BUF][pp][i + 1], j));
        } else {
            const u4 a = vb[BUF][pp][i], b = vb[BUF][pp][i + 1];
            const uint32_t wa = a[j >> 1], wb = b[j >> 1];
            // v_perm_b32 bytes 0-3 come from the second operand, 4-7 from the first
            return __builtin_amdgcn_perm(wb, wa, (j & 1) ? 0x07060302u : 0x05040100u);
        }
    }

    // P.V of unit u on the matrix cores: C[head][dim] += P[head][token] V[token][dim]
    // with v_mfma_f32_16x16x32_bf16, K = the unit's 32 tokens (lane group rg
    // supplies the 8 tokens 16pp + 4rg + i it scored and loaded), M = heads
    // (rows past the group's heads are zero), N = 16 head dims 8n + j per
    // instruction (j = 0..7).  The weights pw (lane (r16, rg): head r16, token
    // 16pp + 4rg + i, times the row's value scale for int8/int4) enter as a
    // bf16 pair hi + lo (hi = bf16(p), lo = bf16(p - hi): 16 significant bits),
    // each against the same V operand.
    template <int BUF, bool MASK>
    __device__ __forceinline__ void pv_mfma(const Params& P, const TileRef& r, int u, const float (&pw)[UP][4]) {
        const int lane = lane_id(), r16 = lane & 15, rg = lane >> 4;
        const bool hv = r16 < P.G;
        bf16x8 ahi, alo;
#pragma unroll
        for (int pp = 0; pp < UP; ++pp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float w = hv ? pw[pp][i] : 0.f;
                if constexpr (SCALED) w *= scale_of(vsr[BUF][pp], i);
                const __bf16 h = (__bf16)w;
                ahi[4 * pp + i] = h;
                alo[4 * pp + i] = (__bf16)(w - (float)h);
            }
        if constexpr (MASK) {
            // a row outside the sequence (or of an invalid block) has weight 0;
            // its V row (a fallback row) must not bring in a NaN or an infinity
#pragma unroll
            for (int pp = 0; pp < UP; ++pp)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool rv = ((r.pmask >> (UP * u + pp)) & 1) && r.t * T + 32 * u + 16 * pp + 4 * rg + i < r.n;
                    if (!rv) vb[BUF][pp][i] = vvec{};
                }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            u4 bw;
#pragma unroll
            for (int q = 0; q < 4; ++q) bw[q] = v_pair<BUF>(j, q >> 1, 2 * (q & 1));
            const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
            cacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, cacc[j], 0, 0, 0);
            cacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, cacc[j], 0, 0, 0);
        }
    }

    // Reduce the running state into the fold mapping and reset it.  The four
    // row groups (lanes l, l^16, l^32, l^48) are summed by a two-step
    // reduce-scatter: after it, lane l holds head 4hb + (l>>4) of each block.
    __device__ __forceinline__ void flush(const Params& P, Out& o) {
        const int lane = lane_id(), rg = lane >> 4;
        const int G = P.G;
        float lt = l_run + __shfl_xor(l_run, 16);
        lt += __shfl_xor(lt, 32);
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            o.m[h] = (h < GMAX && h < G) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_run), h))
                                         : kNegInf;
            o.l[h] = (h < GMAX && h < G) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lt), h)) : 0.f;
        }
        // lane h holds head h: copies for the fold mapping (lane l serves head 4hb + (l >> 4))
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            o.mf[hb] = 4 * hb + rg < G ? __shfl(m_run, 4 * hb + rg) : kNegInf;
            o.lf[hb] = 4 * hb + rg < G ? __shfl(lt, 4 * hb + rg) : 0.f;
        }
        // the accumulators: head 4hb + rg, dims 8n + j (n = lane & 15) sit in
        // component rg of cacc[j] in lane n + 16hb
        const int n = lane & 15;
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float c0 = __shfl(cacc[j][0], n + 16 * hb), c1 = __shfl(cacc[j][1], n + 16 * hb);
                const float c2 = __shfl(cacc[j][2], n + 16 * hb), c3 = __shfl(cacc[j][3], n + 16 * hb);
                o.a[hb][j] = rg == 0 ? c0 : rg == 1 ? c1 : rg == 2 ? c2 : c3;
            }
        reset();
    }
};

// ------------------------------------------------------------------ output of a finished head
__device__ __forceinline__ void write_head_out(const Params& P, int grp, int h, const FoldLanes& fl,
                                               const float (&a8)[8], float L, int err, int U) {
    const long long row = qrow(P, grp, h);
    if (fl.cvalid) {
        float* o = P.out + row * P.D + 8 * fl.cid;
        const float inv = 1.f / L;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = err ? NAN : a8[i] * inv;
    }
    if (fl.cid == 0) P.tiles_used[row] = err ? -1 : U;
}

// ------------------------------------------------------------------ give-up path of every wait
__device__ __forceinline__ void give_up(const Params& P) { cst(P.abort_flag, 1); }
__device__ __forceinline__ bool aborted(const Params& P) { return cld(P.abort_flag) != 0; }

// Wall-clock budget of any single wait (device real-time counter, 100 MHz):
// past it the kernel gives up, so no wait can hang the GPU.
struct Deadline {
    unsigned long long t0;
    __device__ Deadline() : t0(wall_clock64()) {}
    __device__ bool passed() const { return wall_clock64() - t0 > kWaitTicks; }
};

// ------------------------------------------------------------------ ring publication
//
// publish_data() stores a partial into its slot and returns a coherent
// re-read of the last word it stored.  publish_flag() consumes that value
// before storing the tag: vector memory operations of a wave complete in
// issue order, so once the re-read has returned, every slot store before it
// has completed -- and loads issued in between (the next unit's prefetch)
// may still be in flight.
template <int HBM>
__device__ __forceinline__ int publish_data(const Params& P, int grp, int t, const TileOutT<HBM>& o) {
    const int lane = lane_id();
    const FoldLanes fl(P);
    float* slot = P.ring + ((long long)grp * kRing + (t & (kRing - 1))) * P.slot;
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        const int h = hb * 4 + fl.hl;
        if (hb < fl.HB && h < P.G && fl.cvalid) {
            float* a = slot + kSlotHeader + h * P.D + 8 * fl.cid;
#pragma unroll
            for (int j = 0; j < 8; ++j) cst(a + j, o.a[hb][j]);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            if (h < P.G) {
                cst(slot + h, o.m[h]);
                cst(slot + 16 + h, o.l[h]);
            }
        }
        cst(reinterpret_cast<int*>(slot) + 32, o.err);
        cst(reinterpret_cast<int*>(slot) + 33, o.kept);
    }
    return cld(reinterpret_cast<const int*>(slot) + 33);
}

__device__ __forceinline__ void publish_flag(const Params& P, int grp, int t, int token) {
    asm volatile("" ::"v"(token) : "memory");  // wait for the re-read (and so for the slot stores)
    if (lane_id() == 0) cst(&P.ring_tag[(long long)grp * kRing + (t & (kRing - 1))], t + 1);
}

// ------------------------------------------------------------------ fold of ready tiles
//
// (m, l, a) := (m, l, a) (+) (m2, l2, a2): online-softmax merge, left = earlier
__device__ __forceinline__ void sm_merge(float& m, float& l, float (&a)[8], float m2, float l2,
                                         const float (&a2)[8]) {
    const float mn = fmaxf(m, m2);
    if (mn == kNegInf) return;
    const float w1 = m == kNegInf ? 0.f : expf(m - mn);
    const float w2 = m2 == kNegInf ? 0.f : expf(m2 - mn);
    l = fmaf(w1, l, w2 * l2);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = fmaf(w1, a[j], w2 * a2[j]);
    m = mn;
}

// Per-head committed state of the group, kept in registers by the lock holder
// (fold mapping: lane 16*hl + cid, head 4*hb + hl, dims 8*cid .. +7).
template <int HBM>
struct FoldState {
    float M[HBM], L[HBM], pn[HBM], prev[HBM][8], A[HBM][8];
    int streak[HBM], err[HBM], U[HBM];
};

// Decides the tiles f .. f+k-1 (k <= 16) for head block hb, from the committed
// state S.  Writes the output of every head that stops; when `commit`, folds
// the whole window into S (heads that did not stop).  Returns the number of
// heads (of this block, counted in lane 16*hl) still active afterwards.
template <int HBM>
__device__ __forceinline__ int fold_window(const Params& P, int grp, int hb, int f, int k, int nt, bool commit, FoldState<HBM>& S,
                           int& ug) {
    const int lane = lane_id();
    const FoldLanes fl(P);
    const int G = P.G, D = P.D;
    const int i = lane & 15;  // tile of the window (decision lanes)
    const int row0 = lane & ~15;
    const int h = hb * 4 + fl.hl;
    const bool act = h < G && S.U[hb] < 0;
    if (__ballot(act) == 0ull) return 0;
    // probe dims of the committed accumulator, from lane 16*hl (cid 0) of the row
    float Ap[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) Ap[j] = __shfl(S.A[hb][j], row0);
    // tile partials of the window, probe dims only
    const bool tv = act && i < k;
    const float* slot = P.ring + ((long long)grp * kRing + ((f + i) & (kRing - 1))) * P.slot;
    const float mi = tv ? cld(slot + h) : kNegInf;
    const float li = tv ? cld(slot + 16 + h) : 0.f;
    const int ei = tv ? cld(reinterpret_cast<const int*>(slot) + 32) : 0;
    float sa[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sa[j] = tv ? cld(slot + kSlotHeader + h * D + j) : 0.f;
    // inclusive scan over the 16 lanes of the row
    float sm = mi, sl = li;
#pragma unroll
    for (int dd = 1; dd < 16; dd <<= 1) {
        const int src = row0 | ((i >= dd) ? i - dd : i);
        float om = __shfl(sm, src), ol = __shfl(sl, src);
        float oa[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) oa[j] = __shfl(sa[j], src);
        if (i >= dd) {
            sm_merge(om, ol, oa, sm, sl, sa);  // earlier (+) mine
            sm = om; sl = ol;
#pragma unroll
            for (int j = 0; j < 8; ++j) sa[j] = oa[j];
        }
    }
    // seed with the committed state: S_i = S_in (+) scan_i
    float rm = S.M[hb], rl = S.L[hb], ra[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ra[j] = Ap[j];
    sm_merge(rm, rl, ra, sm, sl, sa);
    // probe after tile f+i and its predecessor's
    float x[8], xn2 = 0.f;
    const float invL = 1.f / rl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[j] = ra[j] * invL;
        xn2 = fmaf(x[j], x[j], xn2);
    }
    const float xn = sqrtf(xn2);
    const int srcp = row0 | (i > 0 ? i - 1 : 0);
    float ppn = __shfl(xn, srcp), pp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pp[j] = __shfl(x[j], srcp);
    if (i == 0) {
        ppn = S.pn[hb];
#pragma unroll
        for (int j = 0; j < 8; ++j) pp[j] = S.prev[hb][j];
    }
    bool pass = false;
    if (tv && f + i >= 1) {
        float ds, dd;
        if (xn == 0.f || ppn == 0.f) {
            ds = dd = INFINITY;
        } else {
            ds = fabsf(xn - ppn) / ppn;
            // 1 - cos as half the squared distance of the unit vectors
            const float ix = 1.f / xn, ip = 1.f / ppn;
            float s2 = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float dl = fmaf(x[j], ix, -(pp[j] * ip));
                s2 = fmaf(dl, dl, s2);
            }
            dd = 0.5f * s2;
        }
        pass = P.art && ds < P.eps_scale && dd < P.eps_dir;
    }
    const unsigned pbits = (unsigned)(__ballot(pass) >> row0) & 0xffffu;
    // the stop: streaks of passing tiles, tile 0 never compared
    int st = S.streak[hb], istop = -1;
    for (int q = 0; q < k; ++q) {
        if (f + q >= 1) {
            st = ((pbits >> q) & 1u) ? st + 1 : 0;
            if (st >= P.patience) { istop = q; break; }
        }
    }
    const bool stops = istop >= 0;
    const bool last = f + k >= nt;  // no stop: every tile is used
    const bool update = stops || commit;
    const int ilast = stops ? istop : k - 1;
    const int rowl = row0 | ilast;
    const float M_last = __shfl(rm, rowl), L_last = __shfl(rl, rowl);
    const float xn_last = __shfl(xn, rowl);
    float x_last[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x_last[j] = __shfl(x[j], rowl);
    const unsigned ebits = (unsigned)(__ballot(ei != 0 && i <= ilast) >> row0) & 0xffffu;
    // accumulator over all dims with the tiles up to ilast: loads in two
    // groups of eight tiles, each issued before it is used
    float A[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) A[j] = S.A[hb][j];
    if (update) {
        const float w_in = S.M[hb] == kNegInf ? 0.f : expf(S.M[hb] - M_last);
#pragma unroll
        for (int j = 0; j < 8; ++j) A[j] *= w_in;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        float wq[8], aq[8][8];
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
            const int q = 8 * half + qq;
            const float mq = __shfl(mi, row0 | q);
            const bool use = act && update && q <= ilast && fl.cvalid;
            wq[qq] = use ? expf(mq - M_last) : 0.f;
            const float* sq = P.ring + ((long long)grp * kRing + ((f + q) & (kRing - 1))) * P.slot +
                              kSlotHeader + h * D + 8 * fl.cid;
#pragma unroll
            for (int j = 0; j < 8; ++j) aq[qq][j] = use ? cld(sq + j) : 0.f;
        }
#pragma unroll
        for (int qq = 0; qq < 8; ++qq)
#pragma unroll
            for (int j = 0; j < 8; ++j) A[j] = fmaf(wq[qq], aq[qq][j], A[j]);
    }
    const int err = S.err[hb] | (ebits != 0u);
    const int U = stops ? f + istop + 1 : (commit && last ? nt : -1);
    int still = 0;
    if (act) {
        if (U >= 0) {
            write_head_out(P, grp, h, fl, A, L_last, err, U);
            ug = max(ug, U);
            S.U[hb] = U;
        } else {
            still = fl.cid == 0 ? 1 : 0;
            if (commit) {
                S.M[hb] = M_last; S.L[hb] = L_last; S.streak[hb] = st; S.err[hb] = err; S.pn[hb] = xn_last;
#pragma unroll
                for (int j = 0; j < 8; ++j) { S.prev[hb][j] = x_last[j]; S.A[hb][j] = A[j]; }
            }
        }
    }
    return still;
}

// Decider of one group.  It owns the group's running state (in registers)
// and polls the ring: tiles are decided in windows of up to 16 that start at
// the frontier, a multiple of 16.  For each head, lanes 16*(head%4) + i hold
// tile f+i's partial restricted to the probe dims; an inclusive online-softmax
// scan over the 16 lanes, seeded with the committed state, gives the running
// output after every tile of the window, hence every probe, both stability
// metrics and the streak; the first tile whose streak reaches the patience is
// the head's stop, and the head's output is the committed state merged with
// the tiles up to its stop.  A window is decided again whenever more of its
// tiles are ready (the scan value of lane i depends on lanes 0..i only, so
// every decision is the same whatever the arrival order); the other heads'
// state, over all head dims, is committed only for a complete window (or the
// group's last tiles), so every result is computed in the same order whatever
// the timing: the output is deterministic.  Committing moves the frontier,
// which frees ring slots; once every head has stopped the allocation bound
// drops to the stop, so no later tile is claimed.
template <int HBM>
__device__ __forceinline__ void decide_group(const Params& P, int grp) {
    GroupCtl* C = P.ctl + grp;
    const int lane = lane_id();
    const FoldLanes fl(P);
    const int nt = cld(&C->nt);
    if (nt == 0) return;  // empty or invalid row: written by the init kernel
    FoldState<HBM> S;
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        const int h = hb * 4 + fl.hl;
        S.U[hb] = (hb < fl.HB && h < P.G) ? -1 : 0;
        S.M[hb] = kNegInf; S.L[hb] = 0.f; S.pn[hb] = 0.f; S.streak[hb] = 0; S.err[hb] = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) { S.prev[hb][j] = 0.f; S.A[hb][j] = 0.f; }
    }
    int f = 0;        // committed tiles
    int decided = 0;  // tiles of the window at f already decided
    int ug = 0;       // largest tiles_used of the heads stopped so far
    Deadline dl;
    for (;;) {
        const int tau = f + lane;
        const bool ok =
            tau < nt && cld(&P.ring_tag[(long long)grp * kRing + (tau & (kRing - 1))]) == tau + 1;
        const uint64_t msk = __ballot(ok);
        int kall = (~msk == 0ull) ? 64 : __builtin_ctzll(~msk);
        if (kall <= decided) {
            if (dl.passed() || aborted(P)) {
                if (lane == 0) give_up(P);
                return;
            }
            __builtin_amdgcn_s_sleep(2);
            continue;
        }
        dl = Deadline();
        bool finished = false;
        for (;;) {
            const int kw = min(16, kall);
            const bool commit = kw == 16 || f + kw >= nt;
            int still = 0;
            static_for<0, HBM>([&](auto hbc) {
                constexpr int hb = decltype(hbc)::value;  // a constant: the state stays in registers
                if (hb < fl.HB) still += fold_window<HBM>(P, grp, hb, f, kw, nt, commit, S, ug);
            });
            if (__ballot(still > 0) == 0ull) {
                finished = true;
                break;
            }
            if (!commit) {
                decided = kw;
                break;
            }
            f += kw;
            kall -= kw;
            decided = 0;
            if (kall == 0) break;
        }
        if (finished) {
            // every head has stopped: the group used max(tiles_used) tiles
            int ugw = ug;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) ugw = max(ugw, __shfl_xor(ugw, o));
            if (lane == 0) {
                cst(&C->bound, ugw);
                cst(&C->frontier, ugw);
            }
            return;
        }
        if (lane == 0) cst(&C->frontier, f);
    }
}

// Decider wave d serves groups d, d + deciders, ... one after the other.
template <int HBM>
__device__ __forceinline__ void decider(const Params& P, int d) {
    for (int grp = d; grp < P.NG; grp += P.deciders) {
        if (aborted(P)) return;
        decide_group<HBM>(P, grp);
    }
}

// ------------------------------------------------------------------ tile scheduling
// Claims the next tile of group grp: >= 0 the tile; -1 the group has no tile
// left; -2 its ring is full (claim elsewhere).  A tile t is only claimed while
// t < frontier + kRing, so its ring slot (that of tile t - kRing, already
// folded) is free from the moment it is claimed.
__device__ __forceinline__ int take_tile(const Params& P, int grp) {
    int r = -1;
    if (lane_id() == 0) {
        GroupCtl* C = P.ctl + grp;
        for (int spin = 0; spin < 64; ++spin) {
            const int nx = cld(&C->next);
            if (nx >= cld(&C->bound)) { r = -1; break; }
            if (nx - cld(&C->frontier) >= kRing) { r = -2; break; }
            if (cas(&C->next, nx, nx + 1)) { r = nx; break; }
            r = -2;
        }
    }
    return bcast0(r);
}

// Next group with tiles left (and room in its ring), scanning forward from grp; -1 when none.
__device__ __forceinline__ int next_group(const Params& P, int grp) {
    const int lane = lane_id();
    const Deadline dl;
    for (int spin = 0;; ++spin) {
        if (dl.passed() || aborted(P)) {
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
                const int nx = cld(&C->next), bd = cld(&C->bound), fr = cld(&C->frontier);
                has = nx < bd;
                room = nx - fr < kRing;
            }
            const uint64_t m = __ballot(has && room);
            if (m) return (grp + 1 + base + __builtin_ctzll(m)) % P.NG;
            any_left |= __ballot(has) != 0ull;
        }
        if (!any_left) return -1;
        // every group with tiles left has a full ring: back off (about 1 to 4 us)
        if (spin < 4) __builtin_amdgcn_s_sleep(32);
        else __builtin_amdgcn_s_sleep(127);
    }
}

// Claims a tile, moving on to other groups when grp has none; false when no
// group has tiles left.  May wait for ring space, so a wave calls it only
// while it holds no unpublished tile (an unpublished tile can be the one its
// group's frontier waits for).
__device__ __forceinline__ bool claim(const Params& P, int& grp, int& t) {
    const Deadline dl;
    for (;;) {
        if (aborted(P)) return false;
        if (dl.passed()) {
            if (lane_id() == 0) give_up(P);
            return false;
        }
        t = take_tile(P, grp);
        if (t >= 0) return true;
        grp = next_group(P, grp);
        if (grp < 0) return false;
    }
}

// ------------------------------------------------------------------ kernels
__global__ __launch_bounds__(256) void art_init_kernel(Params P) {
    const int grp = blockIdx.x;
    const int tid = threadIdx.x;
    const int b = grp / P.Hkv, g = grp % P.Hkv;
    const int n = P.ctx_lens[seq_of(P, grp)];
    const bool bad = n < 0 || n > P.cap;
    const int nt = (bad || n == 0) ? 0 : (n + P.T - 1) / P.T;
    GroupCtl* C = P.ctl + grp;
    if (tid == 0) {
        C->next = 0; C->frontier = 0; C->bound = nt; C->nt = nt; C->n = n;
        if (grp == 0) *P.abort_flag = 0;
    }
    for (int i = tid; i < kRing; i += blockDim.x) P.ring_tag[(long long)grp * kRing + i] = 0;
    if (P.vskip)
        for (int i = tid; i < P.nt_max; i += blockDim.x) P.vmax_tag[(long long)grp * P.nt_max + i] = 0;
    // outputs of finished rows now; the others are marked unfinished (-2, NaN)
    // until the fold writes them
    const long long row0 = qrow(P, grp, 0);
    const int Gh = heads_in(P, grp);
    for (int i = tid; i < Gh * P.D; i += blockDim.x)
        P.out[row0 * P.D + i] = (nt == 0 && !bad) ? 0.f : NAN;
    for (int h = tid; h < Gh; h += blockDim.x) P.tiles_used[row0 + h] = nt > 0 ? -2 : (bad ? -1 : 0);
}

// A caller's tile list (ART_ORDER_LIST) turned into a step table for the
// streamed kernels: record (sq, s) holds, for the tile visited at step s of
// sequence sq (tile_at: -1 for a bad list entry), the block id of each of its
// 16-token pages (paged caches) and, last, the tile itself, so that a worker
// finds a step's tile and blocks with one load that it issues a tile ahead,
// as for the ascending order.  Records past a row's tiles are never read.
static_assert(kStepW == 8 && kStepPages == 4, "a step-table record is two 16-byte stores");
__global__ __launch_bounds__(256) void art_steps_kernel(Params P) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long long)(P.NG / P.seq_div) * P.nt_max) return;
    const int sq = (int)(i / P.nt_max), s = (int)(i % P.nt_max);
    const int n = P.ctx_lens[sq];
    if (n < 0 || n > P.cap) return;  // the row reports -1 and no worker reads its records
    const int nt = (n + P.T - 1) / P.T;
    if (s >= nt) return;
    const int pt = tile_at(P, sq, nt, s);
    int rec[kStepW] = {};
    for (int p = 0; p < kStepPages; ++p) {
        const int tok = pt * P.T + 16 * p;
        if (P.block_size && pt >= 0 && tok < n) rec[p] = P.block_table[(long long)sq * P.mbps + tok / P.block_size];
    }
    rec[kStepPages] = pt;
    int4* dst = reinterpret_cast<int4*>(P.steps + i * kStepW);
    dst[0] = make_int4(rec[0], rec[1], rec[2], rec[3]);
    dst[1] = make_int4(rec[4], rec[5], rec[6], rec[7]);
}

__device__ __forceinline__ void count_stats(const Params& P, unsigned long long tiles, unsigned long long rows) {
    if (P.stats && lane_id() == 0) {
        atomicAdd(reinterpret_cast<unsigned long long*>(P.stats + 0), tiles);
        atomicAdd(reinterpret_cast<unsigned long long*>(P.stats + 1), rows);
    }
}

// One tile at a time (generic and matrix-core tiles; the V skip needs this path).
template <class Tile>
__global__ __launch_bounds__(256) void art_persistent_kernel(Params P) {
    extern __shared__ float lds[];
    const int wv = wave_id(), lane = lane_id();
    float* lds_wave = lds + wv * Tile::lds_floats(P);
    const int gw = blockIdx.x * kWavesPerWG + wv;
    if (gw < P.deciders) {
        decider<Tile::HBM>(P, gw);
        return;
    }
    const int worker = gw - P.deciders;
    if (worker >= P.workers) return;
    int grp = worker % P.NG;
    int qgrp = -1;
    Tile tile;
    int t;
    while (claim(P, grp, t)) {
        const int b = grp / P.Hkv, g = grp % P.Hkv;
        if (grp != qgrp) {
            tile.load_q(P, b, g, lds_wave);
            qgrp = grp;
        }
        GroupCtl* C = P.ctl + grp;
        const int n = P.ctx_lens[seq_of(P, grp)];
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
                    if (h < P.G) cst(vm + h, ml[h]);
            drain();
            if (lane == 0) cst(&P.vmax_tag[vbase + t], 1);
            const Deadline dl;
            for (int base = 0; base < t; base += 64) {
                const int tau = base + lane;
                const bool need = tau < t;
                for (;;) {
                    const bool ready = !need || cld(&P.vmax_tag[vbase + tau]) != 0;
                    if (__ballot(!ready) == 0ull) break;
                    if (cld(&C->bound) <= t) return false;
                    if (dl.passed()) {
                        if (lane == 0) give_up(P);
                        return false;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                const float* src = P.vmax + ((long long)vbase + tau) * 16;
#pragma unroll
                for (int h = 0; h < kMaxG; ++h) {
                    if (h < P.G) Mt[h] = fmaxf(Mt[h], wave_max(need ? cld(src + h) : kNegInf));
                }
            }
            return true;
        };
        typename Tile::Out o;
        if (!tile.compute(P, b, g, n, t, hook, o)) continue;
        const int token = publish_data(P, grp, t, o);
        publish_flag(P, grp, t, token);
        count_stats(P, 1ull, (unsigned long long)o.kept);
    }
}

// Streamed matrix-core tiles, one tile per claim.  The wave holds no loaded
// data while it publishes and folds, so the fold's registers never compete
// with a prefetch (the other resident waves keep the memory system busy), and
// the wave holds no unpublished tile when it next claims, so it may wait.
template <class S>
__global__ __launch_bounds__(256, S::MIN_WAVES) void art_stream_kernel(Params P) {
    extern __shared__ float lds[];
    const int wv = wave_id();
    const int gw = blockIdx.x * kWavesPerWG + wv;
    if (gw < P.deciders) {
        decider<S::HBM>(P, gw);
        return;
    }
    const int worker = gw - P.deciders;
    if (worker >= P.workers) return;
    S st;
    st.init(lds + wv * S::lds_floats(P));
    int grp = worker % P.NG;
    int t;
    int qgrp = -1;
    typename S::TileRef C;
    while (claim(P, grp, t)) {
        S::resolve(P, grp, t, C);
        if (C.grp != qgrp) {  // before the tile's loads: consume() counts those in issue order
            st.load_q(P, C.grp);
            qgrp = C.grp;
        }
        st.template issue<0>(P, C, 0);
        st.template issue<1>(P, C, 1);
        st.template consume<0>(P, C, 0, true);
        st.template consume<1>(P, C, 1, false);
        typename S::Out o;
        st.flush(P, o);
        o.err = C.err;
        const int rows = S::named(C.t) ? min(S::T, max(0, C.n - C.t * S::T)) : 0;
        o.kept = rows;
        const int token = publish_data(P, C.grp, t, o);
        publish_flag(P, C.grp, t, token);
        count_stats(P, 1ull, (unsigned long long)rows);
    }
}

// ------------------------------------------------------------------ team kernel (work-groups per group)
//
// A group is served by a primary work-group and, where every work-group of
// the launch fits on the chip at once, up to kMaxHelpers helper work-groups
// on other CUs.  Wave 0 of the primary decides; every other wave is a tile
// worker.  Tiles are assigned statically: over every W consecutive tiles the
// first nA go to the primary's workers in turn and the rest to the helpers'
// workers in turn, so each worker streams its own arithmetic sequence of
// tiles, the loads of the next one issued before the current one is handed
// over.
//
// A primary worker hands each tile's whole partial (per head: the tile's
// softmax max and sum and its accumulator, in the fold mapping) to the
// decider through a ring of LDS slots (data, a wait for LDS, then the slot's
// tag) and never waits for a decision.  A helper hands over only a probe
// record per head (the tile's max and sum, its accumulator on head dims 0..7
// -- the probe dims -- and its error flag) through global memory, as 64-bit
// words whose upper half names the call (epoch) and the lap of the ring slot,
// so that the decider recognises a record word by word and no store has to
// wait for another; a helper keeps each tile's partial until the decider has
// decided the tile, then merges it into its own running state for every head
// that uses it.
//
// The decider takes the tiles in aligned blocks of kBlock: lane i of a
// 16-lane row (one row per head) holds tile f0 + i's record, and an
// inclusive online-softmax scan along the row (DPP row shifts), merged with
// the state committed before the block, gives the probe state after every
// tile of the block.  Lane i's value depends on tiles f0 .. f0 + i only, so
// the tiles of a block are decided as soon as their prefix is complete, with
// the same values however the records trickled in.  Both stability metrics,
// the streak and the stop then follow for every tile in order.  The decider
// merges each primary tile, once decided, into the group's output for the
// heads that use it (in tile order, freeing its slot), publishes per head how
// many tiles are decided -- or tiles_used once the head stops -- for the
// helpers, and once every head has stopped drops the bound, so that no worker
// loads a further tile.  The helpers' running states are merged last, in
// helper order, so the output does not depend on timing.
constexpr int kTeamSlots = 8;   // LDS slots of whole partials, by ordinal among the primary's tiles (a power of two)
constexpr int kBlock = 16;      // tiles the decider scans together
constexpr int kChain = 8;       // LDS slots of the running-max chain (V skip)

// decision word of a head
constexpr int kHdStop = 1 << 30;         // the head stopped; the count is its tiles_used
constexpr int kHdGaveUp = 1 << 29;       // a wait outlasted kWaitTicks: the head reports -2
constexpr int kHdCount = (1 << 29) - 1;  // else the count is the number of tiles decided

// whether tile q enters a head's output under its decision word: 1 yes, 0 no, -1 not decided yet
__device__ __forceinline__ int tile_fate(int w, int q) {
    if (w & kHdStop) return q < (w & kHdCount) ? 1 : 0;
    if (w & kHdGaveUp) return 0;
    return q < (w & kHdCount) ? 1 : -1;
}

template <int HBM>
struct TeamShared {
    int tag[kTeamSlots];  // t + 1 once the slot holds tile t's partial
    int err[kTeamSlots];  // the tile met an invalid block id
    float part[kTeamSlots][HBM * kTeamStateW * 64];  // [head block][max, sum, 8 dims][lane]
    int released;         // the primary's ordinals merged by the decider (their slots may be reused)
    int bound;            // tiles that may still be loaded
    // V skip: the running max through tile t, per head, in slot t % kChain (its tag t + 1 once written)
    int ptag[kChain];
    float pmax[kChain][16];
};

// Control words in LDS, accessed as LDS (a volatile access through a generic
// pointer would become a flat access, which also waits for the wave's
// outstanding global loads).
typedef __attribute__((address_space(3))) volatile int lds_vint;
__device__ __forceinline__ int lds_ld(const int* p) { return *(const lds_vint*)(p); }
__device__ __forceinline__ void lds_st(int* p, int v) { *(lds_vint*)(p) = v; }
// waits for this wave's LDS accesses only (vector-memory loads stay in flight)
__device__ __forceinline__ void wait_lds() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// epoch-stamped control words
__device__ __forceinline__ unsigned long long stamp(unsigned epoch, unsigned v) {
    return ((unsigned long long)epoch << 32) | v;
}
__device__ __forceinline__ int unstamp(unsigned long long w, unsigned epoch, int dflt) {
    return (unsigned)(w >> 32) == epoch ? (int)(unsigned)w : dflt;
}
// tagged data words: (tag << 32) | bits of the value
__device__ __forceinline__ unsigned long long tagw(unsigned tag, float v) {
    return ((unsigned long long)tag << 32) | (unsigned)__float_as_int(v);
}
__device__ __forceinline__ float untag(unsigned long long w) { return __int_as_float((int)(unsigned)w); }
// tag of record ordinal o in a ring of RING slots: the call and the lap of its slot (a slot is
// rewritten only after the decider has taken the previous lap, so a word is
// either of this lap or of the one before)
template <int RING>
__device__ __forceinline__ unsigned rec_tag(unsigned epoch, int o) {
    return epoch * 2u + (unsigned)((o / RING) & 1);
}

// row_shr:D within 16-lane rows; lanes i < D of a row get `old`
template <int D>
__device__ __forceinline__ float row_shr(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x110 + D, 0xf, 0xf, false));
}

// sum of squares of 8 values as a balanced tree (short dependency chain)
__device__ __forceinline__ float sumsq8(const float (&v)[8]) {
    const float a = fmaf(v[1], v[1], v[0] * v[0]), b = fmaf(v[3], v[3], v[2] * v[2]);
    const float c = fmaf(v[5], v[5], v[4] * v[4]), d = fmaf(v[7], v[7], v[6] * v[6]);
    return (a + b) + (c + d);
}

// (m, l, a) := (m, l, a) (+) (m2, l2, a2) with the hardware exponential:
// the decider's merges, which only feed the probe
__device__ __forceinline__ void sm_merge_fast(float& m, float& l, float (&a)[8], float m2, float l2,
                                              const float (&a2)[8]) {
    const float mn = fmaxf(m, m2);
    const float w1 = m == kNegInf ? 0.f : exp_fast(m - mn);
    const float w2 = m2 == kNegInf ? 0.f : exp_fast(m2 - mn);
    l = fmaf(w1, l, w2 * l2);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = fmaf(w1, a[j], w2 * a2[j]);
    m = mn;
}

// The first tile q < kk of a block at which a head's streak of passing tiles
// reaches `patience` (-1 if none), from bit q of p = tile q passes and the
// streak s0 (< patience) carried into the block; sk = the streak after tile
// kk - 1.
__device__ __forceinline__ int first_stop(unsigned p, int kk, int s0, int patience, int& sk) {
    const unsigned valid = (1u << kk) - 1u;  // kk <= 16
    p &= valid;
    const int need0 = patience - s0;        // the leading run continues the carried streak
    const int lead = __builtin_ctz(~p);     // ones from tile 0 on
    int stop = -1;
    if (lead >= need0) {
        stop = need0 - 1;
    } else if (patience <= 16) {
        // bit q of x: tiles q .. q + patience - 1 all pass
        unsigned x = p;
        for (int k = 1; k < patience; ++k) x &= p >> k;
        if (x) stop = __builtin_ctz(x) + patience - 1;
    }
    const unsigned z = ~p & valid;          // failing tiles
    sk = z == 0u ? s0 + kk : kk - 1 - (31 - __builtin_clz(z));
    return stop;
}

// Static assignment of a group's tiles to the workers of its teams.
// Tiles below S0 go to the primary's workers alone, in turn; from S0 on,
// over every W = nA + nH consecutive tiles, the first nA go to the primary's
// workers and the rest to the helpers' (S0 is a multiple of nA, so a primary
// worker's tiles step by nA below S0 and by W above, and its ordinals among
// the primary's tiles by nA throughout).
struct TeamPlan {
    int nA, nH, W, S0;  // primary workers, helper workers (all helpers), period, first shared tile
    __device__ TeamPlan(int nA_, int nH_, int from)
        : nA(nA_), nH(nH_), W(nA_ + nH_), S0(nH_ > 0 ? (from + nA_ - 1) / nA_ * nA_ : 0) {}
    __device__ bool primary(int t) const { return t < S0 || (t - S0) % W < nA; }
    // ordinal of primary tile t among the primary's tiles
    __device__ int ordA(int t) const { return t < S0 ? t : S0 + (t - S0) / W * nA + (t - S0) % W; }
    // ordinal of helper tile t among the helpers' tiles
    __device__ int ordH(int t) const { return (t - S0) / W * nH + (t - S0) % W - nA; }
    // the primary worker's tile after t
    __device__ int nextA(int t) const { return t + (t < S0 ? nA : W); }
};
constexpr int kTeamHelpFrom = 96;  // helpers take no tile below this one (most groups stop before)
constexpr int kTeamHelpLead = 16;  // a helper starts once the decided tiles reach its first tile less this

// A group's words in global memory (team kernel with helpers).
struct TeamGlobal {
    unsigned long long* part;  // [kTeamRingG][HB][kTeamPartW][64]: the helpers' tile partials, tagged
    unsigned long long* ctl;   // [kTeamCtl]
    int slot_words;            // HB * kTeamPartW * 64
    __device__ TeamGlobal(const Params& P, int grp) {
        part = P.team_ring + (long long)grp * group_words(P.G);
        ctl = P.team_ctl + (long long)grp * kTeamCtl;
        slot_words = ((P.G + 3) / 4) * kTeamPartW * 64;
    }
};

// (max, sum, accumulator) per head block in the fold mapping: a tile's
// partial or a running state
template <int HBM>
struct Part {
    float m[HBM], l[HBM], a[HBM][8];
    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            m[hb] = kNegInf;
            l[hb] = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) a[hb][j] = 0.f;
        }
    }
};

// A helper worker: tiles first, first + W, ... of the group.  Each tile's
// whole partial goes to the group's ring in global memory as tagged 64-bit
// words (so no store waits for another), and the primary's decider merges
// it: a helper never waits for a decision, only for a free slot.
template <class S>
__device__ __forceinline__ void team_helper_worker(const Params& P, int grp, int n, int nt, int first,
                                                   const TeamPlan& plan, S& st) {
    constexpr int HBM = S::HBM;
    const int lane = lane_id();
    const TeamGlobal tg(P, grp);
    int t = first;
    if (t >= nt) return;
    // ordinal of tile t among the helpers' tiles; its slot may be written
    // once the decider has released the ordinal a ring before
    int o1 = plan.ordH(first);
    // start once the decided tiles come near this worker's first tile (the
    // group may stop before: then load nothing)
    {
        const Deadline dl;
        for (;;) {
            const int dec = uni(unstamp(cld(tg.ctl + 2), P.epoch, 0));
            const int b0 = uni(unstamp(cld(tg.ctl + 1), P.epoch, nt));
            if (t >= b0) return;
            if (dec >= plan.S0 - kTeamHelpLead) break;
            if (dl.passed()) return;
            __builtin_amdgcn_s_sleep(16);
        }
    }
    // the bound and the released ordinals as last seen, loaded before a
    // tile's loads and taken once those have landed
    int bnd = nt, rel = 0;
    unsigned long long qb = 0, qr = 0;
    auto load_glb = [&]() {
        qb = cld(tg.ctl + 1);
        qr = cld(tg.ctl + 0);
    };
    auto take_glb = [&]() {
        bnd = uni(unstamp(qb, P.epoch, nt));
        rel = uni(unstamp(qr, P.epoch, 0));
    };
    bool gv = false;  // a wait outlasted kWaitTicks
    typename S::TileRef C;
    load_glb();
    st.load_q(P, grp);  // before the tile's loads: consume() counts those in issue order
    S::resolve(P, grp, t, C);
    st.template issue<0>(P, C, 0);
    st.template issue<1>(P, C, 1);
    int blkN = S::fetch_blocks(P, grp, n, t + plan.W);  // block ids of the next tile
    // tiles (and rows) loaded, counted when their loads are issued
    unsigned long long loaded = 1, rows = S::rows_in(C);
    for (;;) {
        st.template consume<0>(P, C, 0, true);
        st.template consume<1>(P, C, 1, false);
        typename S::Out o;
        st.flush(P, o);
        take_glb();
        if (t >= bnd) break;  // past the group's stop: no head uses the tile
        // the next tile's loads first, then the hand-over of this one
        const int tn = t + plan.W;
        const bool haveN = tn < nt && tn < bnd;
        const int cerr = C.err;
        if (haveN) {
            S::resolve_from(P, grp, n, tn, blkN, C);
            load_glb();
            st.template issue<0>(P, C, 0);
            st.template issue<1>(P, C, 1);
            blkN = S::fetch_blocks(P, grp, n, tn + plan.W);
            ++loaded;
            rows += S::rows_in(C);
        }
        // the slot must have been released (the decider releases no further
        // slot once the group is done: then the tile is past the bound)
        if (o1 - kTeamRingG >= rel) {
            const Deadline dl;
            for (;;) {
                __builtin_amdgcn_s_sleep(4);
                rel = uni(unstamp(cld(tg.ctl + 0), P.epoch, 0));
                bnd = uni(unstamp(cld(tg.ctl + 1), P.epoch, nt));
                if (o1 - kTeamRingG < rel || t >= bnd) break;
                if (dl.passed()) {
                    gv = true;
                    break;
                }
            }
            if (gv || t >= bnd) break;
        }
        {
            const unsigned tag = rec_tag<kTeamRingG>(P.epoch, o1);
            unsigned long long* e = tg.part + (long long)(o1 & (kTeamRingG - 1)) * tg.slot_words + lane;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                unsigned long long* w = e + hb * kTeamPartW * 64;
                cst(w, tagw(tag, o.mf[hb]));
                cst(w + 64, tagw(tag, o.lf[hb]));
#pragma unroll
                for (int j = 0; j < 8; ++j) cst(w + 64 * (2 + j), tagw(tag, o.a[hb][j]));
                cst(w + 64 * 10, tagw(tag, __int_as_float(cerr)));
            }
        }
        if (!haveN) break;
        t = tn;
        o1 += plan.nH;
    }
    // loads of a tile fetched past the stop may still be landing (in LDS too)
    __builtin_amdgcn_s_waitcnt(0);
    count_stats(P, loaded, rows);
}

// A primary worker: tiles first, first + W, ... of the group, each handed
// over whole to the decider through the LDS slots.
template <class S, int VSKIP>
__device__ __forceinline__ void team_primary_worker(const Params& P, int grp, int n, int nt, int first,
                                                    const TeamPlan& plan, S& st, TeamShared<S::HBM>* sh) {
    constexpr int HBM = S::HBM;
    const int lane = lane_id();
    int t = first;
    if (t >= nt) return;
    int o1 = first;  // ordinal of tile t among the primary's tiles
    int bnd = nt, rel = 0;
    bool gv = false;  // a wait outlasted kWaitTicks
    typename S::TileRef C;
    st.load_q(P, grp);  // before the tile's loads: consume() counts those in issue order
    S::resolve(P, grp, t, C);
    // (VSKIP 2, the V skip with V loaded late: K only, a tile's V rows are
    // loaded once its scores are known)
    st.template issue<0, VSKIP != 2>(P, C, 0);
    st.template issue<1, VSKIP != 2>(P, C, 1);
    int blkN = S::fetch_blocks(P, grp, n, plan.nextA(t));  // block ids of the next tile
    // tiles (and rows) loaded, counted when their loads are issued (V rows
    // under the V skip: when consumed)
    unsigned long long loaded = 1, rows = VSKIP == 2 ? 0 : S::rows_in(C), skipped = 0;
    for (;;) {
        if constexpr (VSKIP) {
            // the running max through tile t: that through tile t - 1 (from its
            // worker, through LDS) and this tile's
            auto chain = [&](float mu) -> float {
                float M = mu;
                if (t > 0) {
                    // (a tile past the group's stop may wait for one never loaded: it is dropped anyway)
                    const int sp = (t - 1) % kChain;
                    if (lds_ld(&sh->ptag[sp]) != t) {
                        const Deadline dl;
                        while (lds_ld(&sh->ptag[sp]) != t && t < lds_ld(&sh->bound) && !dl.passed())
                            __builtin_amdgcn_s_sleep(1);
                    }
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the value is read after its tag
                    M = fmaxf(M, __int_as_float(lds_ld(reinterpret_cast<const int*>(&sh->pmax[sp][lane & 15]))));
                }
                const int sn = t % kChain;
                if (lane < 16) lds_st(reinterpret_cast<int*>(&sh->pmax[sn][lane]), __float_as_int(M));
                wait_lds();
                if (lane == 0) lds_st(&sh->ptag[sn], t + 1);
                return M;
            };
            unsigned vr = 0;
            skipped += (unsigned)st.template consume_tile_vskip<VSKIP == 2>(P, C, chain, vr);
            rows += vr;
        } else {
            st.template consume<0>(P, C, 0, true);
            st.template consume<1>(P, C, 1, false);
        }
        typename S::Out o;
        st.flush(P, o);
        bnd = uni(lds_ld(&sh->bound));
        if (t >= bnd) break;  // past the group's stop: no head uses the tile
        // the next tile's loads first, then the hand-over of this one
        const int tn = plan.nextA(t);
        const bool haveN = tn < nt && tn < bnd;
        const int cerr = C.err;
        if (haveN) {
            S::resolve_from(P, grp, n, tn, blkN, C);
            st.template issue<0, VSKIP != 2>(P, C, 0);
            st.template issue<1, VSKIP != 2>(P, C, 1);
            blkN = S::fetch_blocks(P, grp, n, plan.nextA(tn));
            ++loaded;
            if constexpr (VSKIP != 2) rows += S::rows_in(C);
        }
        // the slot must have been released (the decider releases no further
        // slot once the group is done: then the tile is past the bound)
        rel = uni(lds_ld(&sh->released));
        if (o1 - kTeamSlots >= rel) {
            const Deadline dl;
            for (;;) {
                __builtin_amdgcn_s_sleep(1);
                rel = uni(lds_ld(&sh->released));
                bnd = uni(lds_ld(&sh->bound));
                if (o1 - kTeamSlots < rel || t >= bnd) break;
                if (dl.passed()) {
                    gv = true;
                    break;
                }
            }
            if (gv || t >= bnd) break;
        }
        {
            const int s = o1 & (kTeamSlots - 1);
            float* e = sh->part[s] + lane;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                e[(hb * kTeamStateW + 0) * 64] = o.mf[hb];
                e[(hb * kTeamStateW + 1) * 64] = o.lf[hb];
#pragma unroll
                for (int j = 0; j < 8; ++j) e[(hb * kTeamStateW + 2 + j) * 64] = o.a[hb][j];
            }
            if (lane == 0) lds_st(&sh->err[s], cerr);
            wait_lds();  // the partial is written before its tag
            if (lane == 0) lds_st(&sh->tag[s], t + 1);
        }
        if (!haveN) break;
        t = tn;
        o1 += plan.nA;
    }
    // loads of a tile fetched past the stop may still be landing (in LDS too)
    __builtin_amdgcn_s_waitcnt(0);
    count_stats(P, loaded, rows);
    if (VSKIP && P.stats && lane == 0) atomicAdd(reinterpret_cast<unsigned long long*>(P.stats + 3), skipped);
}

// The decider's state for a group's heads: the running (max, sum, probe dims)
// committed after the tiles before the current block, the probe after the
// last committed tile, the streak, and per head tiles_used (-1 while active)
// and the error flag; one head per 16-lane row, replicated over the row.
template <int HBM>
struct ProbeState {
    float M[HBM], L[HBM], Pd[HBM][8], X[HBM][8], Xn[HBM];
    int streak[HBM], U[HBM], err[HBM];
    bool hv[HBM];
    __device__ __forceinline__ void init(const FoldLanes& fl, int G) {
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            hv[hb] = hb < fl.HB && hb * 4 + fl.hl < G;
            M[hb] = kNegInf;
            L[hb] = 0.f;
            Xn[hb] = 0.f;
            streak[hb] = 0;
            err[hb] = 0;
            U[hb] = hv[hb] ? -1 : 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                Pd[hb][j] = 0.f;
                X[hb][j] = 0.f;
            }
        }
    }
    // no head left undecided
    __device__ __forceinline__ bool finished() const {
        bool any = false;
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) any |= hv[hb] && U[hb] < 0;
        return __ballot(any) == 0ull;
    }
    // the largest tiles_used over the group's heads
    __device__ __forceinline__ int bound() const {
        int ug = 0;
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb)
            if (hv[hb]) ug = max(ug, U[hb]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ug = max(ug, __shfl_xor(ug, o));
        return ug;
    }
    // decision word of head block hb (this lane's row): tiles_used once
    // stopped, else the tiles decided
    __device__ __forceinline__ int word(int hb, int decided) const {
        return U[hb] >= 0 ? (kHdStop | U[hb]) : decided;
    }
};

// Lane i's probe record: tile f0 + i of the current block (identity until present).
template <int HBM>
struct BlockRecs {
    float m[HBM], l[HBM], p[HBM][8];
    int e[HBM];
    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            m[hb] = kNegInf;
            l[hb] = 0.f;
            e[hb] = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) p[hb][j] = 0.f;
        }
    }
    // from the tagged 64-bit words of a helper's partial ([head block][word][lane],
    // `src` at this row's lane 16*hl); false unless every word carries `tag`
    __device__ __forceinline__ bool load_tagged_part(const unsigned long long* src, const bool (&hv)[HBM],
                                                     unsigned tag) {
        unsigned long long w[HBM][kTeamPartW];
        bool ok = true;
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb)
            if (hv[hb])
#pragma unroll
                for (int j = 0; j < kTeamPartW; ++j) w[hb][j] = cld(src + (hb * kTeamPartW + j) * 64);
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb)
            if (hv[hb])
#pragma unroll
                for (int j = 0; j < kTeamPartW; ++j) ok &= (unsigned)(w[hb][j] >> 32) == tag;
        if (ok) {
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                if (hv[hb]) {
                    m[hb] = untag(w[hb][0]);
                    l[hb] = untag(w[hb][1]);
#pragma unroll
                    for (int j = 0; j < 8; ++j) p[hb][j] = untag(w[hb][2 + j]);
                    e[hb] = __float_as_int(untag(w[hb][10]));
                }
            }
        }
        return ok;
    }
    // from tagged 64-bit words of a record ([word][kTeamRecHeads] apart); false
    // unless every word carries `tag`
    __device__ __forceinline__ bool load_tagged(const unsigned long long* rec, const bool (&hv)[HBM], int hl,
                                                unsigned tag) {
        unsigned long long w[HBM][kTeamRecW];
        bool ok = true;
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb)
            if (hv[hb])
#pragma unroll
                for (int j = 0; j < kTeamRecW; ++j) w[hb][j] = cld(rec + j * kTeamRecHeads + hb * 4 + hl);
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb)
            if (hv[hb])
#pragma unroll
                for (int j = 0; j < kTeamRecW; ++j) ok &= (unsigned)(w[hb][j] >> 32) == tag;
        if (ok) {
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                if (hv[hb]) {
                    m[hb] = untag(w[hb][0]);
                    l[hb] = untag(w[hb][1]);
#pragma unroll
                    for (int j = 0; j < 8; ++j) p[hb][j] = untag(w[hb][2 + j]);
                    e[hb] = (int)(unsigned)w[hb][10];
                }
            }
        }
        return ok;
    }
};

// One pass over block f0 (kmax tiles) whose first kk tiles are present
// (more than at the previous pass): an inclusive online-softmax scan of the
// records along each row, merged with the committed state, gives the probe
// after every tile; both metrics, the streaks and the first stop follow.  A
// head that stops gets tiles_used; when the block is complete (kk == kmax)
// the state after its last tile is committed.  Lane i's values depend on
// tiles f0 .. f0 + i only, so every pass over a block agrees with the others.
template <int HBM>
__device__ __forceinline__ void decide_pass(const Params& P, ProbeState<HBM>& D, const BlockRecs<HBM>& R, int f0,
                                            int kk, int kmax, int nt) {
    const int lane = lane_id(), i = lane & 15, row0 = lane & ~15;
    const int t = f0 + i;
    static_for<0, HBM>([&](auto hbc) {
        constexpr int hb = decltype(hbc)::value;
        const bool act = D.hv[hb] && D.U[hb] < 0;
        if (__ballot(act) == 0ull) return;
        float m = R.m[hb], l = R.l[hb], p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = R.p[hb][j];
        auto step = [&](auto dc) {
            constexpr int d = decltype(dc)::value;
            float om = row_shr<d>(kNegInf, m), ol = row_shr<d>(0.f, l), op[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) op[j] = row_shr<d>(0.f, p[j]);
            sm_merge_fast(om, ol, op, m, l, p);  // the earlier tiles first
            m = om;
            l = ol;
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = op[j];
        };
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 4>{});
        step(std::integral_constant<int, 8>{});
        // the running state after tile t: committed (+) scan
        float sM = D.M[hb], sL = D.L[hb], sP[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sP[j] = D.Pd[hb][j];
        sm_merge_fast(sM, sL, sP, m, l, p);
        // probe: dims 0..7 of the normalised running output; the hardware
        // reciprocal and square root (about 1 ulp)
        const float invL = __builtin_amdgcn_rcpf(sL);
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = sP[j] * invL;
        const float xn = __builtin_amdgcn_sqrtf(sumsq8(x));
        // the previous probe: lane i - 1's, the committed one for lane 0
        const float ppn = row_shr<1>(D.Xn[hb], xn);
        float pp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pp[j] = row_shr<1>(D.X[hb][j], x[j]);
        bool pass = false;
        if (t >= 1) {
            float ds, dd;
            if (xn == 0.f || ppn == 0.f) {
                ds = dd = INFINITY;
            } else {
                const float ix = __builtin_amdgcn_rcpf(xn), ip = __builtin_amdgcn_rcpf(ppn);
                ds = fabsf(xn - ppn) * ip;
                // 1 - cos as half the squared distance of the unit vectors
                float dl2[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) dl2[j] = fmaf(x[j], ix, -(pp[j] * ip));
                dd = 0.5f * sumsq8(dl2);
            }
            pass = ds < P.eps_scale && dd < P.eps_dir;
        }
        const unsigned pbits = (unsigned)(__ballot(pass) >> row0) & 0xffffu;
        const unsigned ebits = (unsigned)(__ballot(R.e[hb] != 0) >> row0) & 0xffffu;
        // the streak from the block start (the same at every pass) to the first stop
        int sk;
        const int istop = first_stop(pbits, kk, D.streak[hb], P.patience, sk);
        if (act) {
            if (istop >= 0) {
                D.U[hb] = f0 + istop + 1;
                D.err[hb] |= (ebits & ((2u << istop) - 1u)) != 0u;
            } else if (kk == kmax) {
                // the block is complete: commit its last tile's state
                const int src = row0 | (kmax - 1);
                D.err[hb] |= (ebits & ((2u << (kmax - 1)) - 1u)) != 0u;
                D.streak[hb] = sk;
                D.M[hb] = __shfl(sM, src);
                D.L[hb] = __shfl(sL, src);
                D.Xn[hb] = __shfl(xn, src);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    D.Pd[hb][j] = __shfl(sP[j], src);
                    D.X[hb][j] = __shfl(x[j], src);
                }
                if (f0 + kmax >= nt) D.U[hb] = nt;  // no stop: every tile is used
            }
        }
    });
}

// The present prefix of the block: tiles whose records every head's row holds.
__device__ __forceinline__ int present_prefix(bool have, int kmax) {
    const unsigned long long b = __ballot(have);
    const unsigned mask = (unsigned)(b & (b >> 16) & (b >> 32) & (b >> 48)) & 0xffffu;
    return min(__builtin_ctz(~mask), kmax);
}

// Decides the group's tiles, block after block, and merges the primary's
// tiles into acc as they are decided; D holds each head's tiles_used (-1 if
// undecided: the wait for a tile outlasted kWaitTicks) and error flag.
template <int HBM, bool HELPERS>
__device__ __forceinline__ void team_decider(const Params& P, int grp, int nt, const TeamPlan& plan,
                                             TeamShared<HBM>* sh, ProbeState<HBM>& D, Part<HBM>& acc,
                                             Part<HBM>& accH, bool publish = false) {
    const int lane = lane_id(), i = lane & 15;
    const FoldLanes fl(P);
    const TeamGlobal tg(P, grp);
    const bool glb = plan.nH > 0;
    const bool pub = glb || publish;  // progress and bound go to global memory (helpers, score workers)
    D.init(fl, heads_in(P, grp));
    acc.clear();
    accH.clear();
    int relA = 0, relH = 0;
    bool finished = false, gave_up = false;
    // merges the decided helper tiles among f0 + qa .. f0 + qb - 1, in order,
    // kHB at a time (their words loaded together); false if a partial did not
    // arrive whole within kWaitTicks
    constexpr int kHB = HBM == 1 ? 4 : 1;
    auto merge_helpers = [&](int f0, int qa, int qb) -> bool {
        int q = qa;
        for (;;) {
            int tl[kHB];
            int cnt = 0;
            static_for<0, kHB>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                while (q < qb && plan.primary(f0 + q)) ++q;
                tl[k] = -1;
                if (q < qb) {
                    tl[k] = f0 + q;
                    ++q;
                    ++cnt;
                }
            });
            if (cnt == 0) return true;
            unsigned long long w[kHB][HBM][kTeamStateW];
            const Deadline dl;
            for (;;) {
                bool ok = true;
                static_for<0, kHB>([&](auto kc) {
                    constexpr int k = decltype(kc)::value;
                    if (tl[k] >= 0) {
                        const int o = plan.ordH(tl[k]);
                        const unsigned tag = rec_tag<kTeamRingG>(P.epoch, o);
                        const unsigned long long* e = tg.part + (long long)(o & (kTeamRingG - 1)) * tg.slot_words + lane;
#pragma unroll
                        for (int hb = 0; hb < HBM; ++hb)
#pragma unroll
                            for (int j = 0; j < kTeamStateW; ++j) {
                                w[k][hb][j] = cld(e + (hb * kTeamPartW + j) * 64);
                                ok &= (unsigned)(w[k][hb][j] >> 32) == tag;
                            }
                    }
                });
                if (__ballot(!ok) == 0ull) break;
                if (dl.passed()) return false;
                __builtin_amdgcn_s_sleep(2);
            }
            static_for<0, kHB>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if (tl[k] >= 0) {
#pragma unroll
                    for (int hb = 0; hb < HBM; ++hb) {
                        if (D.hv[hb] && (D.U[hb] < 0 || tl[k] < D.U[hb])) {
                            float a2[8];
#pragma unroll
                            for (int j = 0; j < 8; ++j) a2[j] = untag(w[k][hb][2 + j]);
                            sm_merge_fast(accH.m[hb], accH.l[hb], accH.a[hb], untag(w[k][hb][0]),
                                          untag(w[k][hb][1]), a2);
                        }
                    }
                    relH = plan.ordH(tl[k]) + 1;
                }
            });
            if (lane == 0) cst(tg.ctl + 0, stamp(P.epoch, (unsigned)relH));  // their slots may be reused
        }
    };
    // merges the decided primary tiles among f0 + q0 .. f0 + q1 - 1, in order
    auto merge_primary = [&](int f0, int q0, int q1) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the slots are read after their tags
        for (int q = q0; q < q1; ++q) {
            const int tq = f0 + q;
            if (!plan.primary(tq)) continue;  // a helper's tile: merged from global memory
            const int oq = plan.ordA(tq);
            const float* e = sh->part[oq & (kTeamSlots - 1)] + lane;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                if (D.hv[hb] && (D.U[hb] < 0 || tq < D.U[hb])) {
                    float a2[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) a2[j] = e[(hb * kTeamStateW + 2 + j) * 64];
                    sm_merge_fast(acc.m[hb], acc.l[hb], acc.a[hb], e[(hb * kTeamStateW) * 64],
                                  e[(hb * kTeamStateW + 1) * 64], a2);
                }
            }
            relA = oq + 1;
        }
        // (a wave's LDS accesses execute in order: the slots are read before they are released)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) lds_st(&sh->released, relA);
    };
    for (int f0 = 0; f0 < nt && !finished && !gave_up; f0 += kBlock) {
        const int kmax = min(kBlock, nt - f0);
        const int t = f0 + i;
        const bool inr = i < kmax;
        const bool prim = plan.primary(t);
        const int ord = prim ? plan.ordA(t) : plan.ordH(t);
        const int sA = ord & (kTeamSlots - 1), sH = ord & (kTeamRingG - 1);
        const unsigned rtag = rec_tag<kTeamRingG>(P.epoch, ord);
        BlockRecs<HBM> R;
        R.clear();
        bool have = !inr;
        int kdone = 0;
        unsigned long long since = wall_clock64();
        for (;;) {
            if (!have) {
                if (prim) {
                    // a wave's LDS accesses execute in order and the worker stores
                    // the data before the tag: data read after the tag is the tile's
                    if (lds_ld(&sh->tag[sA]) == t + 1) {
                        __atomic_signal_fence(__ATOMIC_SEQ_CST);
                        const float* e = sh->part[sA] + 16 * fl.hl;  // lane 16*hl holds the probe dims
                        const int ev = lds_ld(&sh->err[sA]);
#pragma unroll
                        for (int hb = 0; hb < HBM; ++hb) {
                            if (D.hv[hb]) {
                                R.m[hb] = e[(hb * kTeamStateW) * 64];
                                R.l[hb] = e[(hb * kTeamStateW + 1) * 64];
#pragma unroll
                                for (int j = 0; j < 8; ++j) R.p[hb][j] = e[(hb * kTeamStateW + 2 + j) * 64];
                                R.e[hb] = ev;
                            }
                        }
                        __atomic_signal_fence(__ATOMIC_SEQ_CST);
                        have = true;
                    }
                } else if constexpr (HELPERS) {
                    // the probe record: the words of lane 16*hl of the helper's partial
                    have = R.load_tagged_part(tg.part + (long long)sH * tg.slot_words + 16 * fl.hl, D.hv, rtag);
                }
            }
            const int kk = present_prefix(have, kmax);
            if (kk > kdone) {
                since = wall_clock64();
                decide_pass<HBM>(P, D, R, f0, kk, kmax, nt);
                merge_primary(f0, kdone, kk);
                if constexpr (HELPERS) {
                    if (glb && !merge_helpers(f0, kdone, kk)) {
                        gave_up = true;
                        break;
                    }
                }
                kdone = kk;
                finished = D.finished();
                if (pub && lane == 0) cst(tg.ctl + 2, stamp(P.epoch, (unsigned)(f0 + kdone)));  // progress, for helpers
                if (finished) {
                    const int ug = D.bound();
                    if (lane == 0) {
                        lds_st(&sh->bound, ug);
                        if (pub) cst(tg.ctl + 1, stamp(P.epoch, (unsigned)ug));
                    }
                    break;
                }
            }
            if (kdone == kmax) break;
            if (wall_clock64() - since > kWaitTicks) {
                gave_up = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (finished || gave_up) break;
    }
    if (gave_up) {
        // every head reports -2 (a helper's partial may be missing from any of them)
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) D.U[hb] = D.hv[hb] ? -1 : 0;
        if (lane == 0) {
            lds_st(&sh->bound, 0);
            if (pub) cst(tg.ctl + 1, stamp(P.epoch, 0u));
        }
    }
}

// Grid: NG primaries, then P.helpers rounds of NG helpers (helper r of group
// g is work-group (1 + r) * NG + g).
template <class S, int VSKIP>
__global__ __launch_bounds__(S::TEAM * 64) void art_team_kernel(Params P) {
    extern __shared__ float lds[];
    constexpr int HBM = S::HBM, TEAM = S::TEAM;
    const int wv = wave_id(), lane = lane_id();
    const FoldLanes fl(P);
    const int G = P.G;
    const int grp = blockIdx.x % P.NG, team = blockIdx.x / P.NG;
    const int b = grp / P.Hkv, g = grp % P.Hkv;
    const int n = P.ctx_lens[seq_of(P, grp)];
    const bool bad = n < 0 || n > P.cap;
    const int nt = (bad || n == 0) ? 0 : (n + S::T - 1) / S::T;
    if (nt == 0) {
        // empty row: zero output, no tiles; invalid length: NaN, -1
        if (team == 0 && wv == 0) {
            const long long row0 = qrow(P, grp, 0);
            const int Gh = heads_in(P, grp);
            for (int k = lane; k < Gh * P.D; k += 64) P.out[row0 * P.D + k] = bad ? NAN : 0.f;
            for (int h = lane; h < Gh; h += 64) P.tiles_used[row0 + h] = bad ? -1 : 0;
        }
        return;
    }
    const TeamPlan plan(TEAM - 1, P.helpers * TEAM, kTeamHelpFrom);
    const size_t wave_floats = S::lds_floats(P);
    if (team > 0) {
        // a helper: every wave is a worker
        if constexpr (!VSKIP) {
            S st;
            st.init(lds + wv * wave_floats);
            team_helper_worker<S>(P, grp, n, nt, plan.S0 + plan.nA + (team - 1) * TEAM + wv, plan, st);
        }
        return;
    }
    TeamShared<HBM>* sh = reinterpret_cast<TeamShared<HBM>*>(lds + (TEAM - 1) * wave_floats);
    if (wv == 0) {
        if (lane < kTeamSlots) sh->tag[lane] = 0;
        if (lane < kChain) sh->ptag[lane] = 0;
        if (lane == 0) {
            sh->released = 0;
            sh->bound = nt;
        }
    }
    __syncthreads();
    if (wv != 0) {
        S st;
        st.init(lds + (wv - 1) * wave_floats);
        team_primary_worker<S, VSKIP>(P, grp, n, nt, wv - 1, plan, st, sh);
        return;
    }
    // the decider's chain is latency-bound: let its SIMD issue it first
    __builtin_amdgcn_s_setprio(3);
    ProbeState<HBM> D;
    Part<HBM> tot, toth;
    team_decider<HBM, !VSKIP>(P, grp, nt, plan, sh, D, tot, toth);  // (the V skip runs without helpers)
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        const int h = hb * 4 + fl.hl;
        if (!D.hv[hb]) continue;
        if (D.U[hb] < 0) {
            float nan8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) nan8[j] = NAN;
            write_head_out(P, grp, h, fl, nan8, 1.f, 0, -2);
        } else {
            // the primary's tiles, then the helpers' (each merged in tile order)
            sm_merge(tot.m[hb], tot.l[hb], tot.a[hb], toth.m[hb], toth.l[hb], toth.a[hb]);
            write_head_out(P, grp, h, fl, tot.a[hb], tot.l[hb], D.err[hb], D.U[hb]);
        }
    }
}

template <class S>
size_t team_lds_bytes(const Params& p) {
    const size_t primary =
        (size_t)(S::TEAM - 1) * S::lds_floats(p) * sizeof(float) + sizeof(TeamShared<S::HBM>);
    const size_t helper = (size_t)S::TEAM * S::lds_floats(p) * sizeof(float);
    return primary > helper ? primary : helper;
}

// ------------------------------------------------------------------ pair kernel (K and V of a group on two CUs)
//
// A CU's vector-memory pipeline, not HBM, bounds the team kernel: one group
// streams ~45 GB/s on one CU whether its tiles come from HBM or from cache,
// and a tile's 32 one-KB load instructions take most of a worker's cycle.
// The pair kernel gives every group two CUs of one XCD: a score work-group
// loads the K rows (into registers), computes the scores with the matrix
// cores and publishes them per tile (1 KB: 4 heads x 64 tokens); the primary
// work-group loads only the V rows, takes each tile's scores, does the online
// softmax and P.V, and decides as the team kernel does (same decider, same
// LDS slots, same results).  The score workers keep within kPairWindow tiles
// of the decided frontier (the primary's workers run at most kTeamSlots + 7
// tiles ahead of it) and stop at the bound.  A record slot is reused kPairRing
// tiles later, when its tile is decided (kPairRing >= kPairWindow).
constexpr int kPairRing = 32;    // score records per group (a power of two)
constexpr int kPairWindow = 24;  // score workers stay below decided + kPairWindow
constexpr size_t kPairMinLds = 96 * 1024;  // one work-group per CU: the two roles never share a CU

// Scalar load that bypasses the scalar cache (coherent with other CUs' stores).
__device__ __forceinline__ unsigned long long sload_glc(const unsigned long long* p) {
    unsigned long long v;
    asm volatile("s_load_dwordx2 %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}

struct PairRing {
    unsigned long long* flag;  // [kPairRing]: stamp(epoch, t + 1) once slot t % kPairRing holds tile t
    float* rec;                // [kPairRing][256]: lane (h, g) of the primary reads [16 (4g + h) .. +16)
    __device__ PairRing(const Params& P, int grp) {
        unsigned long long* base = P.team_ring + (long long)grp * group_words(P.G);
        flag = base;
        rec = reinterpret_cast<float*>(base + kPairRing);
    }
};

// Score worker: tiles first, first + step, ... of the group.  K rows go to
// registers in the matrix-core operand layout (lane (r, g): row r of a page,
// head dims 32 st + 8 g .. + 7), one v_mfma_f32_16x16x32_bf16 per 32 dims.
template <class S>
__device__ __forceinline__ void pair_score_worker(const Params& P, int grp, int n, int nt, int first, int step,
                                                  S& st) {
    constexpr int KV = S::KVT, ROWB = S::ROWB, T = S::T, PAGES = S::PAGES;
    // vector-memory instructions of one tile's K loads (rows, then scales)
    constexpr int NK = PAGES * 4 + (S::SCALED ? PAGES : 0);
    const int lane = lane_id(), r16 = lane & 15, rg = lane >> 4;
    const TeamGlobal tg(P, grp);
    const PairRing ring(P, grp);
    int t = first;
    if (t >= nt) return;
    st.load_q(P, grp);
    int dec = 0, bnd = nt;
    unsigned long long ktiles = 0;  // K tiles loaded (stats[0])
    typedef typename std::conditional<KV == ART_I4, uint32_t, typename std::conditional<KV == ART_I8, u2, u4>::type>::type kvec;
    kvec kr[PAGES][4];
    float ksc[PAGES][4];
    typename S::TileRef C;
    // the K rows (registers, matrix-core operand layout) and scales of tile r: NK instructions
    auto issue_k = [&](const typename S::TileRef& r) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < PAGES; ++p) {
            const long long pr = ((r.pmask >> p) & 1) ? r.prow[p] : 0;
            const char* kb = static_cast<const char*>(P.k) + pr * ROWB + r16 * ROWB;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (KV == ART_I8) kr[p][q] = __builtin_nontemporal_load(reinterpret_cast<const u2*>(kb + 32 * q + 8 * rg));
                else if constexpr (KV == ART_I4) kr[p][q] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + 16 * q + 4 * rg));
                else kr[p][q] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(kb + 16 * (4 * q + rg)));
            }
            if constexpr (S::SCALED) {
                const u2 w = *reinterpret_cast<const u2*>(P.ks + pr + 4 * rg);
                ksc[p][0] = f16_to_f32(w.x & 0xffff) * P.inv_sqrt_d;
                ksc[p][1] = f16_to_f32(w.x >> 16) * P.inv_sqrt_d;
                ksc[p][2] = f16_to_f32(w.y & 0xffff) * P.inv_sqrt_d;
                ksc[p][3] = f16_to_f32(w.y >> 16) * P.inv_sqrt_d;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto flag = [&](int tt) {
        if (lane == 0) cst(ring.flag + (tt & (kPairRing - 1)), stamp(P.epoch, (unsigned)(tt + 1)));
    };
    S::resolve(P, grp, t, C);
    int blkN = t + step < nt ? S::fetch_blocks(P, grp, n, t + step) : 0;
    issue_k(C);
    for (;;) {
        // scores of tile t (waits for its K)
        float sc[PAGES][4];
#pragma unroll
        for (int p = 0; p < PAGES; ++p) {
            f4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x8 a;
                if constexpr (KV == ART_I8) {
                    const u2 w = kr[p][q];
                    u4 cv;
                    cv.x = bf16_pair(sbyte(w.x, 0), sbyte(w.x, 1));
                    cv.y = bf16_pair(sbyte(w.x, 2), sbyte(w.x, 3));
                    cv.z = bf16_pair(sbyte(w.y, 0), sbyte(w.y, 1));
                    cv.w = bf16_pair(sbyte(w.y, 2), sbyte(w.y, 3));
                    a = __builtin_bit_cast(bf16x8, cv);
                } else if constexpr (KV == ART_I4) {
                    const uint32_t w = kr[p][q];
                    u4 cv;
                    cv.x = bf16_pair(snib(w, 0), snib(w, 1));
                    cv.y = bf16_pair(snib(w, 2), snib(w, 3));
                    cv.z = bf16_pair(snib(w, 4), snib(w, 5));
                    cv.w = bf16_pair(snib(w, 6), snib(w, 7));
                    a = __builtin_bit_cast(bf16x8, cv);
                } else {
                    a = __builtin_bit_cast(bf16x8, kr[p][q]);
                }
                a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, st.qB[q], a4, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = ((C.pmask >> p) & 1) && C.t * T + 16 * p + 4 * rg + i < C.n;
                const float k = S::SCALED ? ksc[p][i] : P.inv_sqrt_d;
                sc[p][i] = valid ? a4[i] * k : kNegInf;
            }
        }
        ++ktiles;
        // the record: lanes of the group's (at most 4) heads write their 16 scores
        if (r16 < 4) {
            float* dst = ring.rec + (t & (kPairRing - 1)) * 256 + 16 * (4 * rg + r16);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u4 v = {__float_as_uint(sc[q][0]), __float_as_uint(sc[q][1]), __float_as_uint(sc[q][2]),
                              __float_as_uint(sc[q][3])};
                asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(dst + 4 * q), "v"(v) : "memory");
            }
        }
        const int tn = t + step;
        bool more = tn < nt && tn < bnd;
        // stay within the window of the decided frontier; stop at the bound
        if (more && tn >= dec + kPairWindow) {
            drain();  // this record has reached memory: flag it before waiting
            flag(t);
            const Deadline dl;
            for (;;) {
                const unsigned long long wb = sload_glc(tg.ctl + 1), wd = sload_glc(tg.ctl + 2);
                bnd = min(nt, unstamp(wb, P.epoch, nt));
                dec = unstamp(wd, P.epoch, 0);
                if (tn >= bnd || tn < dec + kPairWindow) break;
                if (dl.passed()) return;  // the primary gives up on its own
                __builtin_amdgcn_s_sleep(2);
            }
            more = tn < bnd;
            if (!more) break;
            S::resolve_from(P, grp, n, tn, blkN, C);
            blkN = tn + step < nt ? S::fetch_blocks(P, grp, n, tn + step) : 0;
            issue_k(C);
        } else if (more) {
            // the next tile's K goes out behind this record; once only those
            // NK loads may still be in flight the record has reached memory
            S::resolve_from(P, grp, n, tn, blkN, C);
            blkN = tn + step < nt ? S::fetch_blocks(P, grp, n, tn + step) : 0;
            issue_k(C);
            S::template wait_vm<NK>();
            flag(t);
        } else {
            drain();
            flag(t);
            break;
        }
        t = tn;
    }
    __builtin_amdgcn_s_waitcnt(0);
    count_stats(P, ktiles, 0ull);
}

// Primary worker of the pair kernel: tiles first, first + nA, ... ; V rows
// only, the scores from the tile's record; hand-over to the decider as in the
// team kernel.
template <class S>
__device__ __forceinline__ void pair_primary_worker(const Params& P, int grp, int n, int nt, int first,
                                                    const TeamPlan& plan, S& st, TeamShared<S::HBM>* sh,
                                                    float* rec_lds) {
    constexpr int HBM = S::HBM, UP = S::UP;
    const int lane = lane_id(), r16 = lane & 15, rg = lane >> 4;
    const PairRing ring(P, grp);
    int t = first;
    if (t >= nt) return;
    int o1 = first;
    int bnd = nt, rel = 0;
    bool gv = false;
    typename S::TileRef C;
    S::resolve(P, grp, t, C);
    st.template issue_vs<0>(P, C, 0);
    st.template issue_vs<1>(P, C, 1);
    int blkN = S::fetch_blocks(P, grp, n, plan.nextA(t));
    unsigned long long loaded = 1, rows = S::rows_in(C);
    for (;;) {
        // the tile's scores: wait for its record, then copy it into LDS
        const int slot = t & (kPairRing - 1);
        const unsigned long long want = stamp(P.epoch, (unsigned)(t + 1));
        if (sload_glc(ring.flag + slot) != want) {
            const Deadline dl;
            for (;;) {
                __builtin_amdgcn_s_sleep(1);
                if (sload_glc(ring.flag + slot) == want) break;
                bnd = uni(lds_ld(&sh->bound));
                if (t >= bnd) break;
                if (dl.passed()) {
                    gv = true;
                    break;
                }
            }
            if (gv || t >= bnd) break;
        }
        __builtin_amdgcn_global_load_lds(ring.rec + slot * 256 + 4 * lane,
                                         (__attribute__((address_space(3))) void*)rec_lds, 16, 0, 17 /* sc0 sc1 */);
        S::template wait_vm<0>();  // the tile's V, the next block ids and the record
        float s0[UP][4], s1[UP][4];
        {
            const float* e = rec_lds + 16 * (4 * rg + (r16 & 3));
            f4 w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = *reinterpret_cast<const f4*>(e + 4 * q);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s0[0][i] = r16 < 4 ? w[0][i] : kNegInf;
                s0[1][i] = r16 < 4 ? w[1][i] : kNegInf;
                s1[0][i] = r16 < 4 ? w[2][i] : kNegInf;
                s1[1][i] = r16 < 4 ? w[3][i] : kNegInf;
            }
        }
        st.template consume_given<0>(P, C, 0, s0);
        st.template consume_given<1>(P, C, 1, s1);
        typename S::Out o;
        st.flush(P, o);
        bnd = uni(lds_ld(&sh->bound));
        if (t >= bnd) break;
        const int tn = plan.nextA(t);
        const bool haveN = tn < nt && tn < bnd;
        const int cerr = C.err;
        if (haveN) {
            S::resolve_from(P, grp, n, tn, blkN, C);
            st.template issue_vs<0>(P, C, 0);
            st.template issue_vs<1>(P, C, 1);
            blkN = S::fetch_blocks(P, grp, n, plan.nextA(tn));
            ++loaded;
            rows += S::rows_in(C);
        }
        rel = uni(lds_ld(&sh->released));
        if (o1 - kTeamSlots >= rel) {
            const Deadline dl;
            for (;;) {
                __builtin_amdgcn_s_sleep(1);
                rel = uni(lds_ld(&sh->released));
                bnd = uni(lds_ld(&sh->bound));
                if (o1 - kTeamSlots < rel || t >= bnd) break;
                if (dl.passed()) {
                    gv = true;
                    break;
                }
            }
            if (gv || t >= bnd) break;
        }
        {
            const int sl = o1 & (kTeamSlots - 1);
            float* e = sh->part[sl] + lane;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                e[(hb * kTeamStateW + 0) * 64] = o.mf[hb];
                e[(hb * kTeamStateW + 1) * 64] = o.lf[hb];
#pragma unroll
                for (int j = 0; j < 8; ++j) e[(hb * kTeamStateW + 2 + j) * 64] = o.a[hb][j];
            }
            if (lane == 0) lds_st(&sh->err[sl], cerr);
            wait_lds();  // the partial is written before its tag
            if (lane == 0) lds_st(&sh->tag[sl], t + 1);
        }
        if (!haveN) break;
        t = tn;
        o1 += plan.nA;
    }
    __builtin_amdgcn_s_waitcnt(0);
    (void)loaded;  // the K tiles are counted by the score workers
    count_stats(P, 0ull, rows);
}

// Grid: NG primaries, then NG score work-groups (score work-group NG + g
// serves group g; with NG a multiple of 8 both sit on the same XCD).
template <class S>
__global__ __launch_bounds__(S::TEAM * 64) void art_pair_kernel(Params P) {
    extern __shared__ float lds[];
    constexpr int HBM = S::HBM, TEAM = S::TEAM;
    static_assert(HBM == 1, "the pair kernel serves groups of at most 4 query heads");
    const int wv = wave_id(), lane = lane_id();
    const FoldLanes fl(P);
    const int grp = blockIdx.x % P.NG, role = blockIdx.x / P.NG;
    const int n = P.ctx_lens[seq_of(P, grp)];
    const bool bad = n < 0 || n > P.cap;
    const int nt = (bad || n == 0) ? 0 : (n + S::T - 1) / S::T;
    if (nt == 0) {
        if (role == 0 && wv == 0) {
            const long long row0 = qrow(P, grp, 0);
            const int Gh = heads_in(P, grp);
            for (int k = lane; k < Gh * P.D; k += 64) P.out[row0 * P.D + k] = bad ? NAN : 0.f;
            for (int h = lane; h < Gh; h += 64) P.tiles_used[row0 + h] = bad ? -1 : 0;
        }
        return;
    }
    if (role == 1) {
        S st;
        st.init(lds);  // (no LDS use: K stays in registers)
        pair_score_worker<S>(P, grp, n, nt, wv, TEAM, st);
        return;
    }
    const TeamPlan plan(TEAM - 1, 0, kTeamHelpFrom);
    TeamShared<HBM>* sh = reinterpret_cast<TeamShared<HBM>*>(lds + (TEAM - 1) * 256);
    if (wv == 0) {
        if (lane < kTeamSlots) sh->tag[lane] = 0;
        if (lane < kChain) sh->ptag[lane] = 0;
        if (lane == 0) {
            sh->released = 0;
            sh->bound = nt;
        }
    }
    __syncthreads();
    if (wv != 0) {
        S st;
        st.init(lds + (wv - 1) * 256);
        pair_primary_worker<S>(P, grp, n, nt, wv - 1, plan, st, sh, lds + (wv - 1) * 256);
        return;
    }
    __builtin_amdgcn_s_setprio(3);
    ProbeState<HBM> D;
    Part<HBM> tot, toth;
    team_decider<HBM, false>(P, grp, nt, plan, sh, D, tot, toth, true);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        const int h = hb * 4 + fl.hl;
        if (!D.hv[hb]) continue;
        if (D.U[hb] < 0) {
            float nan8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) nan8[j] = NAN;
            write_head_out(P, grp, h, fl, nan8, 1.f, 0, -2);
        } else {
            write_head_out(P, grp, h, fl, tot.a[hb], tot.l[hb], D.err[hb], D.U[hb]);
        }
    }
}

template <class S>
size_t pair_lds_bytes() {
    const size_t need = (size_t)(S::TEAM - 1) * 256 * sizeof(float) + sizeof(TeamShared<S::HBM>);
    return need > kPairMinLds ? need : kPairMinLds;
}

// ------------------------------------------------------------------ pool kernel (workers shared by the groups)
constexpr int kPoolAutoGroups = 64;  // library default: the pool for at most this many groups ...
constexpr int kPoolAutoTiles = 1024;  // ... of at least this many tiles
//
// Every CU runs one persistent work-group.  Wave 0 of work-group g < NG
// decides group g; every other wave is a tile worker that serves whichever
// group needs it.  A worker joins a group (it takes a running-state slot,
// so at most pool_cap workers serve a group), claims the group's tiles one at
// a time from a counter in global memory (a few tiles ahead, so that the
// claim and the block-id lookup of a tile are done before its loads are
// issued), and for each tile publishes a probe record as tagged 64-bit words
// (the same records as the team kernel's helpers, in a ring indexed by tile).
// It merges each of its tiles into its running state once the decider has
// decided the tile, and when the group has no tile left to claim (or has
// stopped) it leaves its running state in its slot and moves to the group
// that has the fewest workers among those with tiles left, so the CUs of
// groups that stop early speed up those that run long.  The decider scans
// the records in aligned blocks like the team kernel's, publishes per-head
// decisions and the bound, and at the end merges the workers' states in slot
// order and writes the output.  Every shared word carries the call's epoch:
// the decider resets each counter to (epoch, 0), and a worker adds to a
// counter only once it has seen it so (the order of stores to different words
// is not relied on).
__device__ __forceinline__ unsigned state_tag(unsigned epoch) { return epoch * 2u; }

// one atomic add for the whole wave (lane 0's), its old value in every lane
__device__ __forceinline__ unsigned long long faa64(unsigned long long* p, unsigned long long v) {
    unsigned long long r = 0;
    if (lane_id() == 0) r = __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return uni64(r);
}
// the same without waiting for it: the low word of the old value in lane 0
// only (read it with uni() once the wave's loads issued before it have landed)
__device__ __forceinline__ int faa64_async(unsigned long long* p, unsigned long long v) {
    int r = 0;
    if (lane_id() == 0) r = (int)(unsigned)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return r;
}
// an atomic add whose old value is not needed
__device__ __forceinline__ void add64(unsigned long long* p, unsigned long long v) {
    if (lane_id() == 0) __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A group's words in global memory (pool kernel).
struct PoolGlobal {
    unsigned long long* rec;     // [kPoolRing][kTeamRecW][kTeamRecHeads]
    unsigned long long* state;   // [kPoolContrib][HB][kTeamStateW][64]
    unsigned long long* ctl;     // [kPoolCtl]
    __device__ PoolGlobal(const Params& P, int grp) {
        rec = P.team_ring + (long long)grp * group_words(P.G);
        state = rec + kPoolRing * kTeamRecW * kTeamRecHeads;
        ctl = P.team_ctl + (long long)grp * kTeamCtl;
    }
};

// tiles of group grp (0 for an empty or invalid row)
__device__ __forceinline__ int group_tiles(const Params& P, int grp, int T) {
    const int n = P.ctx_lens[seq_of(P, grp)];
    return (n <= 0 || n > P.cap) ? 0 : (n + T - 1) / T;
}

template <int HBM>
__device__ __forceinline__ void pool_decider(const Params& P, int grp, int T) {
    const int lane = lane_id(), i = lane & 15;
    const FoldLanes fl(P);
    const int G = P.G;
    const unsigned e = P.epoch;
    const PoolGlobal pg(P, grp);
    const int b = grp / P.Hkv, g = grp % P.Hkv;
    const int n = P.ctx_lens[seq_of(P, grp)];
    const bool bad = n < 0 || n > P.cap;
    const int nt = (bad || n == 0) ? 0 : (n + T - 1) / T;
    // reset the counters (the claim counter last: workers join once they see it reset)
    if (lane == 0) {
        cst(pg.ctl + 0, stamp(e, 0u));
        cst(pg.ctl + 1, stamp(e, (unsigned)nt));
        cst(pg.ctl + 3, stamp(e, 0u));
        cst(pg.ctl + 12, stamp(e, 0u));
        cst(pg.ctl + 2, stamp(e, 0u));
    }
    if (nt == 0) {
        // empty row: zero output, no tiles; invalid length: NaN, -1
        const long long row0 = qrow(P, grp, 0);
        const int Gh = heads_in(P, grp);
        for (int k = lane; k < Gh * P.D; k += 64) P.out[row0 * P.D + k] = bad ? NAN : 0.f;
        for (int h = lane; h < Gh; h += 64) P.tiles_used[row0 + h] = bad ? -1 : 0;
        return;
    }
    ProbeState<HBM> D;
    D.init(fl, heads_in(P, grp));
    bool finished = false, gave_up = false;
    auto publish = [&](int decided) {
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb)
            if (i == 0 && D.hv[hb]) cst(pg.ctl + 4 + hb * 4 + fl.hl, stamp(e, (unsigned)D.word(hb, decided)));
    };
    for (int f0 = 0; f0 < nt && !finished && !gave_up; f0 += kBlock) {
        const int kmax = min(kBlock, nt - f0);
        const int t = f0 + i;
        const unsigned tag = rec_tag<kPoolRing>(e, t);
        const unsigned long long* rec = pg.rec + (long long)(t & (kPoolRing - 1)) * kTeamRecW * kTeamRecHeads;
        BlockRecs<HBM> R;
        R.clear();
        bool have = i >= kmax;
        int kdone = 0;
        unsigned long long since = wall_clock64();
        for (;;) {
            if (!have) have = R.load_tagged(rec, D.hv, fl.hl, tag);
            const int kk = present_prefix(have, kmax);
            if (kk > kdone) {
                since = wall_clock64();
                decide_pass<HBM>(P, D, R, f0, kk, kmax, nt);
                kdone = kk;
                finished = D.finished();
                publish(f0 + kdone);
                if (finished) {
                    const int ug = D.bound();
                    if (lane == 0) cst(pg.ctl + 1, stamp(e, (unsigned)ug));
                    break;
                }
            }
            if (kdone == kmax) break;
            if (wall_clock64() - since > kWaitTicks) {
                gave_up = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (finished || gave_up) break;
        if (lane == 0) cst(pg.ctl + 0, stamp(e, (unsigned)(f0 + kmax)));  // the block's slots may be reused
    }
    if (gave_up) {
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb)
            if (i == 0 && D.hv[hb] && D.U[hb] < 0) cst(pg.ctl + 4 + hb * 4 + fl.hl, stamp(e, (unsigned)kHdGaveUp));
        if (lane == 0) cst(pg.ctl + 1, stamp(e, 0u));
    }
    // the workers' running states, in slot order.  Every worker that claimed a
    // tile joined before it claimed, so the count read now covers them all; a
    // later one finds no tile and its slot is not read.
    const int J = min(unstamp(uni64(cld(pg.ctl + 3)), e, 0), P.pool_cap);
    const unsigned stg = state_tag(e);
    Part<HBM> tot;
    tot.clear();
    bool lost = false;
    constexpr int kB = 4 / HBM;  // states loaded at once
    for (int c0 = 0; c0 < J && !lost; c0 += kB) {
        unsigned long long w[kB][HBM][kTeamStateW];
        const Deadline dl;
        for (;;) {
            bool ok = true;
#pragma unroll
            for (int k = 0; k < kB; ++k) {
                if (c0 + k < J) {
                    const unsigned long long* src = pg.state + (long long)(c0 + k) * HBM * kTeamStateW * 64 + lane;
#pragma unroll
                    for (int hb = 0; hb < HBM; ++hb)
#pragma unroll
                        for (int j = 0; j < kTeamStateW; ++j) {
                            w[k][hb][j] = cld(src + (hb * kTeamStateW + j) * 64);
                            ok &= (unsigned)(w[k][hb][j] >> 32) == stg;
                        }
                }
            }
            if (__ballot(!ok) == 0ull) break;
            if (dl.passed()) {
                lost = true;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
        if (lost) break;
#pragma unroll
        for (int k = 0; k < kB; ++k) {
            if (c0 + k < J) {
#pragma unroll
                for (int hb = 0; hb < HBM; ++hb) {
                    float a2[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) a2[j] = untag(w[k][hb][2 + j]);
                    sm_merge(tot.m[hb], tot.l[hb], tot.a[hb], untag(w[k][hb][0]), untag(w[k][hb][1]), a2);
                }
            }
        }
    }
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        const int h = hb * 4 + fl.hl;
        if (!D.hv[hb]) continue;
        if (lost || D.U[hb] < 0) {
            float nan8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) nan8[j] = NAN;
            write_head_out(P, grp, h, fl, nan8, 1.f, 0, -2);
        } else {
            write_head_out(P, grp, h, fl, tot.a[hb], tot.l[hb], D.err[hb], D.U[hb]);
        }
    }
}

// The group a worker moves to after `cur`: among those with tiles left to
// claim and room for a worker, the one with the fewest workers (ties: the
// nearest after cur, so that workers spread); -1 if none is left.
__device__ __forceinline__ int pool_pick(const Params& P, int cur, int T) {
    const int lane = lane_id();
    const unsigned e = P.epoch;
    unsigned long long best = ~0ull;
    for (int g0 = 0; g0 < P.NG; g0 += 64) {
        const int g = g0 + lane;
        if (g < P.NG) {
            const unsigned long long* ctl = P.team_ctl + (long long)g * kTeamCtl;
            const unsigned long long cw = cld(ctl + 2), bw = cld(ctl + 1), jw = cld(ctl + 3), aw = cld(ctl + 12);
            const int nt = group_tiles(P, g, T);
            bool cand;
            int act = 0;
            if ((unsigned)(cw >> 32) != e) {
                cand = nt > 0;  // not open yet
            } else {
                const int lim = min(nt, unstamp(bw, e, nt));
                cand = (int)(unsigned)cw < lim && unstamp(jw, e, 0) < P.pool_cap;
                act = unstamp(aw, e, 0);
            }
            const unsigned dist = (unsigned)((g - cur - 1 + P.NG) % P.NG);
            const unsigned long long key = ((unsigned long long)act << 32) | dist;
            if (cand && key < best) best = key;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long other = __shfl_xor(best, o);
        best = other < best ? other : best;
    }
    if (best == ~0ull) return -1;
    return (int)(((unsigned)best + cur + 1) % (unsigned)P.NG);
}

// A running state kept in LDS ([head block][m, l, 8 dims][lane]), so that it
// does not hold registers across the tile loop.
template <int HBM>
struct LdsPart {
    float* base;
    __device__ __forceinline__ float& at(int hb, int j) const { return base[(hb * kTeamStateW + j) * 64 + lane_id()]; }
    __device__ __forceinline__ void clear() const {
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            at(hb, 0) = kNegInf;
#pragma unroll
            for (int j = 1; j < kTeamStateW; ++j) at(hb, j) = 0.f;
        }
    }
    // state (+) q for head block hb
    __device__ __forceinline__ void merge(int hb, float qm, float ql, const float (&qa)[8]) const {
        float m = at(hb, 0), l = at(hb, 1), a[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = at(hb, 2 + j);
        sm_merge_fast(m, l, a, qm, ql, qa);
        at(hb, 0) = m;
        at(hb, 1) = l;
#pragma unroll
        for (int j = 0; j < 8; ++j) at(hb, 2 + j) = a[j];
    }
};

// One worker: joins groups and processes their tiles until none is left;
// its running state and a pending tile live in `wsl` (2 * HBM * kTeamStateW
// * 64 floats of LDS), the next tile's block ids in `blk` (S::PAGES ints).
template <class S>
__device__ __forceinline__ void pool_worker(const Params& P, S& st, int widx, float* wsl, int* blk) {
    constexpr int HBM = S::HBM, T = S::T;
    const int lane = lane_id();
    const FoldLanes fl(P);
    const unsigned e = P.epoch;
    unsigned long long loaded = 0, rows = 0;
    int grp = widx % P.NG;
    auto head_ok = [&](int hb) { return hb < fl.HB && hb * 4 + fl.hl < heads_in(P, grp); };
    for (int round = 0;; ++round) {
        if (round > 0) {
            grp = uni(pool_pick(P, grp, T));
            if (grp < 0) break;
        }
        const PoolGlobal pg(P, grp);
        const int n = P.ctx_lens[seq_of(P, grp)];
        const int nt = group_tiles(P, grp, T);
        if (nt == 0) continue;
        // join: once the group's counters are reset, take a state slot
        unsigned long long cw, jw, aw, bw;
        {
            const Deadline dl;
            for (;;) {
                cw = uni64(cld(pg.ctl + 2));
                jw = uni64(cld(pg.ctl + 3));
                aw = uni64(cld(pg.ctl + 12));
                bw = uni64(cld(pg.ctl + 1));
                if ((unsigned)(cw >> 32) == e && (unsigned)(jw >> 32) == e && (unsigned)(aw >> 32) == e) break;
                if (dl.passed()) break;
                __builtin_amdgcn_s_sleep(8);
            }
        }
        if ((unsigned)(cw >> 32) != e || (unsigned)(jw >> 32) != e || (unsigned)(aw >> 32) != e)
            break;  // the group's decider never opened it: give up (the decider reports its heads)
        const int lim0 = min(nt, unstamp(bw, e, nt));
        if ((int)(unsigned)cw >= lim0) continue;  // nothing left to claim
        const int slot = (int)(unsigned)faa64(pg.ctl + 3, 1ull);
        if (slot >= P.pool_cap) continue;  // the group has as many workers as it may have
        add64(pg.ctl + 12, 1ull);
        // the decisions as last seen, loaded before a tile's loads and taken
        // once those have landed; the released tiles are read when needed
        int hw[HBM];
        int bnd = nt, rel = 0;
        unsigned long long qw[HBM], qb = 0;
        auto load_glb = [&]() {
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) qw[hb] = cld(pg.ctl + 4 + min(hb * 4 + fl.hl, kTeamRecHeads - 1));
            qb = cld(pg.ctl + 1);
        };
        auto take_glb = [&]() {
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) hw[hb] = head_ok(hb) ? unstamp(qw[hb], e, 0) : (kHdStop | 0);
            bnd = uni(unstamp(qb, e, nt));
        };
        const LdsPart<HBM> ws{wsl};
        // the tiles awaiting their decision, oldest first: two, as a decision
        // takes about a tile's time to come back through global memory (the
        // second one in LDS, next to the running state)
        const LdsPart<HBM> q1{wsl + HBM * kTeamStateW * 64};
        Part<HBM> q0;
        int t0 = 0, t1 = 0, np = 0;
        ws.clear();
        bool gv = false;
        // merges (or drops) the oldest pending tile once every head has decided it
        auto try_front = [&]() -> bool {
            int fate[HBM];
            bool und = false;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                fate[hb] = tile_fate(hw[hb], t0);
                und |= fate[hb] < 0;
            }
            if (__ballot(und) != 0ull) return false;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb)
                if (fate[hb] > 0) ws.merge(hb, q0.m[hb], q0.l[hb], q0.a[hb]);
            if (np == 2) {
#pragma unroll
                for (int hb = 0; hb < HBM; ++hb) {
                    q0.m[hb] = q1.at(hb, 0);
                    q0.l[hb] = q1.at(hb, 1);
#pragma unroll
                    for (int j = 0; j < 8; ++j) q0.a[hb][j] = q1.at(hb, 2 + j);
                }
            }
            t0 = t1;
            --np;
            return true;
        };
        // merges what is decided; then waits until at most `keep` tiles are pending
        auto retire = [&](int keep) {
            while (np > 0 && try_front()) {
            }
            if (np <= keep) return;
            const Deadline dl;
            for (;;) {
                __builtin_amdgcn_s_sleep(4);
                load_glb();
                take_glb();
                while (np > 0 && try_front()) {
                }
                if (np <= keep) return;
                if (dl.passed()) {
                    gv = true;
                    np = 0;
                    return;
                }
            }
        };
        auto claim = [&]() { return (int)(unsigned)faa64(pg.ctl + 2, 1ull); };
        auto claim_async = [&]() { return faa64_async(pg.ctl + 2, 1ull); };
        // the first tile: claim it and look up its blocks now
        load_glb();
        st.load_q(P, grp);
        int t = claim();
        if (t >= lim0) t = nt;  // nothing needed left
        typename S::TileRef C;
        if (t < nt) {
            const int blk = S::fetch_blocks(P, grp, n, t);
            S::resolve_from(P, grp, n, t, blk, C);
            st.template issue<0>(P, C, 0);
            st.template issue<1>(P, C, 1);
            ++loaded;
            rows += S::rows_in(C);
        }
        // the next one claimed, its blocks in flight; the one after, claimed in flight
        int tN = t < nt ? claim() : nt;
        if (tN < nt) S::fetch_blocks_lds(P, grp, n, tN, blk);
        int tXr = tN < nt ? claim_async() : nt;  // (lane 0)
        while (t < nt) {
            st.template consume<0>(P, C, 0, true);
            st.template consume<1>(P, C, 1, false);
            typename S::Out o;
            st.flush(P, o);
            take_glb();
            const int tX = uni(tXr);  // landed with the tile
            if (t >= bnd) break;  // past the group's stop: no head uses the tile
            retire(1);  // room for this tile
            if (gv) break;
            // the record's slot must have been released (none is, once the
            // group is done: then the tile is past the bound)
            if (t - kPoolRing >= rel) {
                const Deadline dl;
                for (;;) {
                    rel = uni(unstamp(cld(pg.ctl + 0), e, 0));
                    bnd = uni(unstamp(cld(pg.ctl + 1), e, nt));
                    if (t - kPoolRing < rel || t >= bnd) break;
                    if (dl.passed()) {
                        gv = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(4);
                }
                if (gv || t >= bnd) break;
            }
            {
                const unsigned tag = rec_tag<kPoolRing>(e, t);
                unsigned long long* rb = pg.rec + (long long)(t & (kPoolRing - 1)) * kTeamRecW * kTeamRecHeads;
#pragma unroll
                for (int hb = 0; hb < HBM; ++hb) {
                    if (fl.cid == 0 && head_ok(hb)) {
                        unsigned long long* r = rb + hb * 4 + fl.hl;
                        cst(r + 0 * kTeamRecHeads, tagw(tag, o.mf[hb]));
                        cst(r + 1 * kTeamRecHeads, tagw(tag, o.lf[hb]));
#pragma unroll
                        for (int j = 0; j < 8; ++j) cst(r + (2 + j) * kTeamRecHeads, tagw(tag, o.a[hb][j]));
                        cst(r + 10 * kTeamRecHeads, tagw(tag, __int_as_float(C.err)));
                    }
                }
            }
            {
                Part<HBM> qn;
#pragma unroll
                for (int hb = 0; hb < HBM; ++hb) {
                    qn.m[hb] = o.mf[hb];
                    qn.l[hb] = o.lf[hb];
#pragma unroll
                    for (int j = 0; j < 8; ++j) qn.a[hb][j] = o.a[hb][j];
                }
                if (np == 0) {
                    q0 = qn;
                    t0 = t;
                } else {
#pragma unroll
                    for (int hb = 0; hb < HBM; ++hb) {
                        q1.at(hb, 0) = qn.m[hb];
                        q1.at(hb, 1) = qn.l[hb];
#pragma unroll
                        for (int j = 0; j < 8; ++j) q1.at(hb, 2 + j) = qn.a[hb][j];
                    }
                    t1 = t;
                }
                ++np;
            }
            // the next tile's loads
            if (tN >= min(nt, bnd)) break;  // (tX > tN: none of this worker's claims is needed)
            S::resolve_lds(P, grp, n, tN, blk, C);  // (the ids landed with the last tile's loads)
            load_glb();
            st.template issue<0>(P, C, 0);
            st.template issue<1>(P, C, 1);
            ++loaded;
            rows += S::rows_in(C);
            t = tN;
            tN = tX;
            if (tN < nt) S::fetch_blocks_lds(P, grp, n, tN, blk);
            tXr = tN < nt ? claim_async() : nt;
        }
        if (!gv) retire(0);
        __builtin_amdgcn_s_waitcnt(0);  // loads of a dropped tile may still be landing (in LDS too)
        // leave the running state in the slot, then leave the group
        const unsigned stg = state_tag(e);
        unsigned long long* dst = pg.state + (long long)slot * HBM * kTeamStateW * 64 + lane;
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            unsigned long long* w = dst + hb * kTeamStateW * 64;
#pragma unroll
            for (int j = 0; j < kTeamStateW; ++j) cst(w + 64 * j, tagw(stg, ws.at(hb, j)));
        }
        add64(pg.ctl + 12, ~0ull);  // one worker less
        if (gv) break;
    }
    count_stats(P, loaded, rows);
}

// Waves of a pool work-group: as many as are resident on a CU, as long as
// their LDS (tile buffers, running state, a pending tile, block ids) fits.
template <class S>
struct PoolShape {
    static constexpr int WAVE_FLOATS = S::LDS_FLOATS + 2 * S::HBM * kTeamStateW * 64 + 16;
    static constexpr int FIT = (160 * 1024 / 4) / WAVE_FLOATS;
    static constexpr int WAVES = FIT < S::TEAM ? FIT : S::TEAM;
};

// Grid: one work-group per CU, all resident (cooperative launch).
template <class S>
__global__ __launch_bounds__(PoolShape<S>::WAVES * 64) void art_pool_kernel(Params P) {
    extern __shared__ float lds[];
    constexpr int TEAM = PoolShape<S>::WAVES;
    const int wv = wave_id(), wg = blockIdx.x;
    if (wg < P.NG && wv == 0) {
        // the decider's chain is latency-bound: let its SIMD issue it first
        __builtin_amdgcn_s_setprio(3);
        pool_decider<S::HBM>(P, wg, S::T);
        return;
    }
    // workers numbered so that consecutive ones start on consecutive groups
    const int widx = wg < P.NG ? wg * (TEAM - 1) + wv - 1 : P.NG * (TEAM - 1) + (wg - P.NG) * TEAM + wv;
    S st;
    st.init(lds + wv * S::LDS_FLOATS);
    float* mine = lds + TEAM * S::LDS_FLOATS + wv * (2 * S::HBM * kTeamStateW * 64 + 16);
    pool_worker<S>(P, st, widx, mine, reinterpret_cast<int*>(mine + 2 * S::HBM * kTeamStateW * 64));
}

// per wave: tile buffers, then (after all waves' buffers) a running state, a
// pending tile and 16 words for block ids
template <class S>
size_t pool_lds_bytes(const Params&) {
    return (size_t)PoolShape<S>::WAVES * PoolShape<S>::WAVE_FLOATS * sizeof(float);
}

// ------------------------------------------------------------------ XCD engine (ART, streamed tiles)
//
// Work-group i of a grid of one work-group per CU runs on XCD i % 8 (the
// dispatcher deals work-groups round-robin over the XCDs), and the CUs of one
// XCD share an L2.  The engine keeps every group on one XCD: group grp lives on
// XCD grp % 8, its decider runs on that XCD and so do all the workers that
// serve it, so every word the group's waves share crosses one L2 only.
//
//  * Decider work-groups: the first `xp_dec_wgs` work-groups of each XCD run
//    one decider wave per group (the pool kernel's decider: records scanned in
//    aligned 16-tile blocks, per-head decision words, the final merge of the
//    workers' states in slot order).  These CUs load no tiles, so their polls
//    of the records never queue behind a CU's stream of tile loads.
//  * Worker work-groups: `xp_wpc` worker waves per CU.  A worker joins a
//    group of its XCD (the pool kernel's join: a state slot, the claim
//    counter), claims tiles two ahead, and pipelines by unit: the next tile's
//    first unit is issued as soon as the current tile's first unit is consumed,
//    so one or two units are always in flight while it computes.  Decisions are
//    read with scalar loads that bypass the scalar cache (the scalar path does
//    not queue behind the CU's vector loads).  A tile's partial waits in one of
//    kXpPend LDS slots until its decision, then enters the worker's running
//    state or is dropped.  A tile is loaded only while it lies less than
//    `xp_window` tiles past the decided frontier, which bounds the tiles
//    loaded past a stop.  When its group has no tile left to claim, the
//    worker leaves its running state in its slot and joins the group of its
//    XCD with the fewest workers among those with tiles left.
constexpr int kXcd = 8;              // XCDs of the chip: work-group i runs on XCD i % kXcd
constexpr int kXpDeciderWaves = 4;   // decider waves per decider work-group
constexpr int kXpWaves = 4;          // waves per work-group (deciders or workers): one per SIMD, so
                                     // that a wave may hold 512 registers (VGPRs and AGPRs)

// The XCD engine's tile (two tiles of unit buffers: one in flight while the
// other is consumed) and the tiles a worker keeps awaiting their decision.
template <class S>
struct XpShape {
    using T = Stream<S::KVT, S::GM, S::ORDER, 4>;
    static constexpr int HBM = T::HBM;
    static constexpr int PEND = HBM == 1 ? 4 : 2;             // tiles awaiting their decision (registers)
    static constexpr int INTS = 48;                            // block ids (16), control words (32)
    static constexpr int WAVE_FLOATS = T::LDS_FLOATS + INTS;
    static constexpr int FIT = (160 * 1024 / 4) / WAVE_FLOATS;
    static constexpr int MAXW = FIT < kXpWaves ? FIT : kXpWaves;  // worker waves per CU at most
};

// A worker's view of its group's decisions, read with scalar loads that
// bypass the scalar cache (they do not queue behind the CU's outstanding
// vector loads; the loads are waited for inside the same statement): words
// 0..3 and the per-head decision words 4..11 of the group's control block.
// Per lane: hw[hb] = the decision word of the lane's head in head block hb
// (kHdStop | 0 for a lane without a head); bnd = the bound (tiles that may
// still be needed); F = the decided frontier (the smallest count of a head
// still running, nt once every head has stopped); c2, c3 = words 2 and 3.
template <int HBM>
struct XpView {
    int hw[HBM];
    int bnd, F;
    unsigned long long c2, c3;
    __device__ __forceinline__ void read(const unsigned long long* ctl, unsigned e, int nt, int hv, const FoldLanes& fl) {
        typedef unsigned u16s __attribute__((ext_vector_type(16)));
        typedef unsigned u8s __attribute__((ext_vector_type(8)));
        u16s a;
        u8s b;
        asm volatile(
            "s_load_dwordx16 %0, %2, 0x20 glc\n\t"
            "s_load_dwordx8 %1, %2, 0x0 glc\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=s"(a), "=s"(b)
            : "s"(ctl)
            : "memory");
        c2 = ((unsigned long long)b[5] << 32) | b[4];
        c3 = ((unsigned long long)b[7] << 32) | b[6];
        bnd = b[3] == e ? min(nt, (int)b[2]) : nt;
        int f = nt;
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const int w = a[2 * h + 1] == e ? (int)a[2 * h] : 0;
            if (h < hv && !(w & kHdStop)) f = min(f, (w & kHdGaveUp) ? nt : (w & kHdCount));
        }
        F = f;
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            const int h = hb * 4 + fl.hl;
            int w = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) w = h == k ? (a[2 * k + 1] == e ? (int)a[2 * k] : 0) : w;
            hw[hb] = (hb < fl.HB && h < hv) ? w : (kHdStop | 0);
        }
    }
};

// The group a worker of XCD x moves to after `cur`: among the XCD's groups with
// tiles left to claim and room for a worker, the one with the fewest workers
// (ties: the nearest after cur); -1 if none is left.
__device__ __forceinline__ int xp_pick(const Params& P, int cur, int x, int nx, int T) {
    const int lane = lane_id();
    const unsigned e = P.epoch;
    const int kc = (cur - x) / kXcd;
    unsigned long long best = ~0ull;
    for (int k0 = 0; k0 < nx; k0 += 64) {
        const int k = k0 + lane;
        if (k < nx) {
            const int g = x + kXcd * k;
            const unsigned long long* ctl = P.team_ctl + (long long)g * kTeamCtl;
            const unsigned long long cw = cld(ctl + 2), bw = cld(ctl + 1), jw = cld(ctl + 3), aw = cld(ctl + 12);
            const int nt = group_tiles(P, g, T);
            bool cand;
            int act = 0;
            if ((unsigned)(cw >> 32) != e) {
                cand = nt > 0;  // not open yet
            } else {
                const int lim = min(nt, unstamp(bw, e, nt));
                cand = (int)(unsigned)cw < lim && unstamp(jw, e, 0) < P.pool_cap;
                act = unstamp(aw, e, 0);
            }
            const unsigned dist = (unsigned)((k - kc - 1 + nx) % nx);
            const unsigned long long key = ((unsigned long long)act << 32) | dist;
            if (cand && key < best) best = key;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long other = __shfl_xor(best, o);
        best = other < best ? other : best;
    }
    if (best == ~0ull) return -1;
    return x + kXcd * (int)(((unsigned)best + kc + 1) % (unsigned)nx);
}

// Records and decisions of the XCD engine's workers.
//
// A tile's probe record (per head: max, sum, dims 0..7, error flag) is
// stored with one instruction: lane 16*hl + j holds word j of head 4*hb + hl,
// taken from the head's lane 16*hl by lane permutes.
template <int HBM>
__device__ __forceinline__ void xp_store_record(unsigned long long* rb, unsigned tag, const Part<HBM>& o, int err,
                                                const FoldLanes& fl, int hv) {
    const int lane = lane_id(), j = lane & 15, src = lane & ~15;
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        // (every permute runs in all lanes: one evaluated under a condition
        // would read 0 from the source lane where that condition is false)
        const float mv = __shfl(o.m[hb], src), lv = __shfl(o.l[hb], src);
        float v = j == 1 ? lv : mv;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float ak = __shfl(o.a[hb][k], src);
            v = j == 2 + k ? ak : v;
        }
        v = j == 10 ? __int_as_float(err) : v;
        if (j < kTeamRecW && hb < fl.HB && hb * 4 + fl.hl < hv) cst(rb + j * kTeamRecHeads + hb * 4 + fl.hl, tagw(tag, v));
    }
}

// The decisions as loaded by a vector load of the control words (lane i < 16
// holds word i), taken once the load has landed: the bound, the decided
// frontier and each lane's decision words.
template <int HBM>
__device__ __forceinline__ void xp_take(XpView<HBM>& V, unsigned long long q, unsigned e, int nt, int hv,
                                        const FoldLanes& fl) {
    const unsigned lo = (unsigned)q, hi = (unsigned)(q >> 32);
    auto word = [&](int i) -> int {
        const unsigned l = (unsigned)__builtin_amdgcn_readlane((int)lo, i), h = (unsigned)__builtin_amdgcn_readlane((int)hi, i);
        return h == e ? (int)l : -1;
    };
    const int b = word(1);
    V.bnd = b < 0 ? nt : min(nt, b);
    int f = nt;
#pragma unroll
    for (int h = 0; h < 8; ++h) {
        int w = word(4 + h);
        w = w < 0 ? 0 : w;
        if (h < hv && !(w & kHdStop)) f = min(f, (w & kHdGaveUp) ? nt : (w & kHdCount));
    }
    V.F = f;
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        const int h = hb * 4 + fl.hl;
        const int src = 4 + min(h, 7);
        const unsigned l = (unsigned)__shfl((int)lo, src), hh = (unsigned)__shfl((int)hi, src);
        const int w = hh == e ? (int)l : 0;
        V.hw[hb] = (hb < fl.HB && h < hv) ? w : (kHdStop | 0);
    }
}

// One worker of XCD x (index wi among the XCD's workers): joins groups of its
// XCD and processes their tiles until none is left.  Tiles are claimed four
// ahead of the one consumed; tile k's two units are loaded into buffer pair
// k % 2 while tile k - 1 (the other pair) is consumed.  `wint`: 8 LDS ints
// for block ids (LDS-direct loads).
template <class S>
__device__ __forceinline__ void xp_worker(const Params& P, S& st, int x, int wi, int* wint) {
    constexpr int HBM = S::HBM, T = S::T, KP = XpShape<S>::PEND;
    const int lane = lane_id();
    const FoldLanes fl(P);
    const unsigned e = P.epoch;
    const int nx = (P.NG - x + kXcd - 1) / kXcd;  // groups of this XCD: x, x + 8, ...
    if (nx <= 0) return;
    unsigned long long loaded = 0, rows = 0;
    int* blk = wint;        // block ids of the tile whose loads come next but one (LDS-direct)
    int* ctlw = wint + 16;  // the group's control words 0..15 (LDS-direct, coherent)
    int grp = x + kXcd * (wi % nx);
    bool gv = false;  // a wait outlasted kWaitTicks: stop working
    for (int round = 0; !gv; ++round) {
        if (round > 0) {
            grp = uni(xp_pick(P, grp, x, nx, T));
            if (grp < 0) break;
        }
        const PoolGlobal pg(P, grp);
        const int n = P.ctx_lens[seq_of(P, grp)];
        const int nt = group_tiles(P, grp, T);
        if (nt == 0) continue;
        const int hv = heads_in(P, grp);
        // join: once the decider has reset the group's counters, take a state slot
        XpView<HBM> V;
        {
            const Deadline dl;
            for (;;) {
                V.read(pg.ctl, e, nt, hv, fl);
                const unsigned long long aw = uni64(cld(pg.ctl + 12));
                if ((unsigned)(V.c2 >> 32) == e && (unsigned)(V.c3 >> 32) == e && (unsigned)(aw >> 32) == e) break;
                if (dl.passed()) {
                    gv = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
        }
        if (gv) break;  // the group's decider never opened it (it reports its heads)
        if ((int)(unsigned)V.c2 >= V.bnd) continue;  // nothing left to claim
        const int slot = (int)(unsigned)faa64(pg.ctl + 3, 1ull);
        if (slot >= P.pool_cap) continue;  // the group has had as many workers as it may
        add64(pg.ctl + 12, 1ull);
        Part<HBM> run;
        run.clear();
        // tiles awaiting their decision, oldest first: tile ptl[k], partial pq[k]
        Part<HBM> pq[KP];
        int ptl[KP];
        int np = 0;
        // merges (or drops) the oldest pending tile once every head has decided it
        auto try_front = [&]() -> bool {
            const int tp = ptl[0];
            int fate[HBM];
            bool und = false;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                fate[hb] = tile_fate(V.hw[hb], tp);
                und |= fate[hb] < 0;
            }
            if (__ballot(und) != 0ull) return false;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb)
                if (fate[hb] > 0) sm_merge_fast(run.m[hb], run.l[hb], run.a[hb], pq[0].m[hb], pq[0].l[hb], pq[0].a[hb]);
#pragma unroll
            for (int k = 0; k + 1 < KP; ++k) {
                pq[k] = pq[k + 1];
                ptl[k] = ptl[k + 1];
            }
            --np;
            return true;
        };
        auto drain_decided = [&]() {
            while (np > 0 && try_front()) {
            }
        };
        auto refresh = [&]() { V.read(pg.ctl, e, nt, hv, fl); };
        // merges what is decided; then, polling, until at most `keep` tiles are pending
        auto retire = [&](int keep) {
            drain_decided();
            if (np <= keep) return;
            const Deadline dl;
            for (;;) {
                __builtin_amdgcn_s_sleep(2);
                refresh();
                drain_decided();
                if (np <= keep) return;
                if (dl.passed()) {
                    gv = true;
                    np = 0;
                    return;
                }
            }
        };
        // waits (polling) until tile tq may be loaded or is no longer needed:
        // true when it may be loaded
        auto admit = [&](int tq) -> bool {
            if (tq >= V.bnd) return false;
            if (tq < V.F + P.xp_window) return true;
            const Deadline dl;
            for (;;) {
                __builtin_amdgcn_s_sleep(2);
                refresh();
                drain_decided();
                if (tq >= V.bnd) return false;
                if (tq < V.F + P.xp_window) return true;
                if (dl.passed()) {
                    gv = true;
                    return false;
                }
            }
        };
        auto claim = [&]() { return (int)(unsigned)faa64(pg.ctl + 2, 1ull); };
        // every lane takes part (lane 0 adds 1, the others 0), so that no
        // branch around the atomic leaves a result to be merged (and waited
        // for) at once; lane 0's old value is the tile claimed.  A 32-bit add
        // on the count, the low half of the stamped word: the whole result
        // register is used, so none of it is reallocated while the atomic is
        // in flight.
        auto claim_async = [&]() -> int {
            return (int)__hip_atomic_fetch_add(reinterpret_cast<unsigned*>(pg.ctl + 2), lane == 0 ? 1u : 0u,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        // the control words, fetched into LDS (no register waits for them):
        // lane i < 32 loads dword i coherently; read once the load has landed
        auto load_ctl = [&]() {
            if (lane < 32)
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const int*>(pg.ctl) + lane,
                                                 (__attribute__((address_space(3))) void*)ctlw, 4, 0, 16 /* sc1 */);
        };
        auto ctl_word = [&]() -> unsigned long long {
            const int i = lane & 15;
            return ((unsigned long long)(unsigned)lds_ld(ctlw + 2 * i + 1) << 32) | (unsigned)lds_ld(ctlw + 2 * i);
        };
        // pushes a consumed tile's partial (room made first) and stores its record
        auto push = [&](int tq, const typename S::Out& o, int err) {
            retire(KP - 1);
            if (gv) return;
            Part<HBM> pn;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                pn.m[hb] = o.mf[hb];
                pn.l[hb] = o.lf[hb];
#pragma unroll
                for (int j = 0; j < 8; ++j) pn.a[hb][j] = o.a[hb][j];
            }
#pragma unroll
            for (int k = 0; k < KP; ++k)
                if (k == np) {
                    pq[k] = pn;
                    ptl[k] = tq;
                }
            ++np;
            unsigned long long* rb = pg.rec + (long long)(tq & (kPoolRing - 1)) * kTeamRecW * kTeamRecHeads;
            xp_store_record<HBM>(rb, rec_tag<kPoolRing>(e, tq), pn, err, fl, hv);
        };
        // Steady state: tile t in pair A (landed or landing), tile tN in pair B
        // (issued after t), t2's block ids in LDS or on their way, t3 claimed
        // in flight.  A step consumes pair A and issues t2 into it.  When t2
        // is not needed (past the bound: it never becomes needed again) the
        // step issues a dummy tile instead -- rows 0..15 of the cache, held in
        // L2 -- and the loop ends once both pairs hold dummies.  So on every
        // path into a step, t's units, a few single instructions and tN's
        // units were issued in this order: the waits count on at least 3 and
        // 2 units' instructions being younger, and the compiler, seeing the
        // same history on every path, adds no wait of its own.
        typename S::TileRef CA, CB;
        bool realA = false, realB = false;
        auto dummy = [&](typename S::TileRef& r) {
            r.grp = grp;
            r.t = -1;
            r.n = 0;
            r.pmask = 0;
            r.err = 0;
#pragma unroll
            for (int p = 0; p < S::PAGES; ++p) r.prow[p] = 0;
        };
        st.load_q(P, grp);
        int t = claim();
        if (!admit(t)) t = nt;
        int tN = nt, t2 = nt, t3r = nt;
        // A tile past the load window is never waited for while this worker
        // holds a loaded tile whose record is not yet published (the frontier
        // may be waiting for that record): it is deferred -- the pair gets a
        // dummy, the held tile is consumed and published at the next step, and
        // only then does the worker wait for the window.
        auto step = [&](auto pbc, typename S::TileRef& Ccur, bool& realCur, bool realNext) {
            constexpr int PB = decltype(pbc)::value;
            st.template consume_after<2 * PB, 3>(P, Ccur, 0);
            st.template consume_after<2 * PB + 1, 2>(P, Ccur, 1);
            // everything issued before tN's units has landed: t2's block ids,
            // the claim after it and the control words
            typename S::Out o;
            st.flush(P, o);
            xp_take<HBM>(V, ctl_word(), e, nt, hv, fl);
            drain_decided();
            if (realCur && t < V.bnd && !gv) push(t, o, Ccur.err);
            bool issue2 = false;
            if (!gv && t2 < V.bnd) {
                if (t2 < V.F + P.xp_window) issue2 = true;
                else if (!realNext) issue2 = admit(t2);  // nothing unpublished is held: waiting is safe
            }
            const bool defer = !gv && !issue2 && realNext && t2 < V.bnd;
            int t3 = nt;
            if (issue2) {
                t3 = uni(t3r);
                S::resolve_lds(P, grp, n, t2, blk, Ccur);  // (the ids landed with t's loads)
                ++loaded;
                rows += S::rows_in(Ccur);
                if (t3 < V.bnd) S::fetch_blocks_lds(P, grp, n, t3, blk);
                // (claimed whatever happens, so that no select waits for the result;
                // a claim past the bound is never loaded)
                t3r = claim_async();
            } else {
                dummy(Ccur);
            }
            load_ctl();
            st.template issue<2 * PB>(P, Ccur, 0);
            st.template issue<2 * PB + 1>(P, Ccur, 1);
            realCur = issue2;
            t = tN;
            if (issue2) {
                tN = t2;
                t2 = t3 < V.bnd ? t3 : nt;
            } else {
                tN = nt;
                if (!defer) t2 = nt;  // (a deferred t2 keeps its block ids in LDS and its claim)
            }
        };
        if (t < nt) {
            // (one branch holds the prologue and the loop, so that the loop is
            // entered only after both pairs were issued)
            S::resolve_from(P, grp, n, t, S::fetch_blocks(P, grp, n, t), CA);
            st.template issue<0>(P, CA, 0);
            st.template issue<1>(P, CA, 1);
            ++loaded;
            rows += S::rows_in(CA);
            realA = true;
            tN = claim();
            // tile x0 is held unpublished: tN is not waited for (deferred past the window)
            realB = tN < V.bnd && tN < V.F + P.xp_window;
            if (realB) {
                S::resolve_from(P, grp, n, tN, S::fetch_blocks(P, grp, n, tN), CB);
                t2 = claim();
            } else {
                dummy(CB);
                t2 = tN < V.bnd ? tN : nt;  // deferred, or not needed
                tN = nt;
            }
            if (t2 < V.bnd) S::fetch_blocks_lds(P, grp, n, t2, blk);
            t3r = claim_async();  // (lane 0)
            load_ctl();
            st.template issue<2>(P, CB, 0);
            st.template issue<3>(P, CB, 1);
            if (realB) {
                ++loaded;
                rows += S::rows_in(CB);
            }
            for (;;) {
                step(std::integral_constant<int, 0>{}, CA, realA, realB);
                step(std::integral_constant<int, 1>{}, CB, realB, realA);
                if (!realA && !realB) break;
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // loads of a dropped tile may still be landing (in LDS too)
        if (!gv) retire(0);
        // leave the running state in the slot, then leave the group
        const unsigned stg = state_tag(e);
        unsigned long long* dst = pg.state + (long long)slot * HBM * kTeamStateW * 64 + lane;
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            unsigned long long* w = dst + hb * kTeamStateW * 64;
            cst(w, tagw(stg, run.m[hb]));
            cst(w + 64, tagw(stg, run.l[hb]));
#pragma unroll
            for (int j = 0; j < 8; ++j) cst(w + 64 * (2 + j), tagw(stg, run.a[hb][j]));
        }
        add64(pg.ctl + 12, ~0ull);  // one worker less
    }
    count_stats(P, loaded, rows);
}

// Grid: one work-group per CU (all resident: cooperative launch).
template <class S>
__global__ __launch_bounds__(kXpWaves * 64) void art_xp_kernel(Params P) {
    extern __shared__ float lds[];
    using TS = typename XpShape<S>::T;
    constexpr int WF = XpShape<S>::WAVE_FLOATS;
    const int wv = wave_id(), wg = blockIdx.x;
    const int x = wg % kXcd, j = wg / kXcd;
    if (j < P.xp_dec_wgs) {
        const int grp = x + kXcd * (j * kXpDeciderWaves + wv);
        if (grp < P.NG) pool_decider<TS::HBM>(P, grp, TS::T);
        return;
    }
    if (wv >= P.xp_wpc) return;
    const int wi = (j - P.xp_dec_wgs) * P.xp_wpc + wv;
    TS st;
    float* mine = lds + wv * WF;
    st.init(mine);
    xp_worker<TS>(P, st, x, wi, reinterpret_cast<int*>(mine + TS::LDS_FLOATS));
}

// Full mode, one tile at a time: split sp of group grp covers a fixed tile range.
// ------------------------------------------------------------------ round engine
//
// ART mode over every CU, with no hand-over per tile: the visiting steps are
// taken in rounds, one launch each.  In round r every group that still has
// undecided heads loads steps [a_r, a_{r+1}), all at once, over waves[r]
// waves of pw[r] consecutive steps.  For each step a wave leaves (1) that
// tile's own probe record (max, sum and accumulator dims 0..7 per head:
// what the stop rule reads) and (2) its running state through the step (the
// whole accumulator per head).  The last wave of a group to arrive decides
// the round's steps with the block scan the team engine uses, over records
// formed the same way (the same tile partials), so the stops agree with that
// engine's.  A group whose heads are all decided takes no further round; its
// tiles_used are written.  Steps past a group's stop inside its last round
// were loaded for nothing.  A final launch merges, per head, the running
// states of the waves' step ranges below its tiles_used (the range holding
// the stop cut there) and writes the outputs.

struct RoundArgs {
    int r, a0, a1, pw, waves;  // round, its steps [a0, a1), steps per wave, waves per group
};

// a group's decision state between rounds: [HB][kRoundProbeW][64]
__device__ __forceinline__ float* round_state_of(const Params& P, int grp) {
    return P.round_state + (long long)grp * ((P.G + 3) >> 2) * kRoundProbeW * 64;
}

template <int HBM>
__device__ __forceinline__ void round_save(const Params& P, int grp, const ProbeState<HBM>& D) {
    float* cs = round_state_of(P, grp) + lane_id();
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        float* w = cs + hb * kRoundProbeW * 64;
        cst(w + 0 * 64, D.M[hb]);
        cst(w + 1 * 64, D.L[hb]);
        cst(w + 2 * 64, D.Xn[hb]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            cst(w + (3 + j) * 64, D.Pd[hb][j]);
            cst(w + (11 + j) * 64, D.X[hb][j]);
        }
        cst(w + 19 * 64, __int_as_float(D.streak[hb]));
        cst(w + 20 * 64, __int_as_float(D.U[hb]));
        cst(w + 21 * 64, __int_as_float(D.err[hb]));
    }
}

template <int HBM>
__device__ __forceinline__ void round_load(const Params& P, int grp, ProbeState<HBM>& D) {
    const float* cs = round_state_of(P, grp) + lane_id();
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        const float* w = cs + hb * kRoundProbeW * 64;
        D.M[hb] = cld(w + 0 * 64);
        D.L[hb] = cld(w + 1 * 64);
        D.Xn[hb] = cld(w + 2 * 64);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            D.Pd[hb][j] = cld(w + (3 + j) * 64);
            D.X[hb][j] = cld(w + (11 + j) * 64);
        }
        D.streak[hb] = __float_as_int(cld(w + 19 * 64));
        D.U[hb] = __float_as_int(cld(w + 20 * 64));
        D.err[hb] = __float_as_int(cld(w + 21 * 64));
    }
}

// The last wave of group grp to finish round R decides its steps.
template <int HBM>
__device__ __forceinline__ void round_decide(const Params& P, int grp, const RoundArgs& R, int nt, bool bad) {
    const int lane = lane_id(), i = lane & 15;
    const FoldLanes fl(P);
    const int gh = heads_in(P, grp);
    if (nt == 0) {
        // empty row: tiles_used 0; invalid length: -1 (the final launch writes the outputs)
        const long long row0 = qrow(P, grp, 0);
        for (int h = lane; h < gh; h += 64) P.tiles_used[row0 + h] = bad ? -1 : 0;
        return;
    }
    ProbeState<HBM> D;
    D.init(fl, gh);
    if (R.r > 0) round_load<HBM>(P, grp, D);
    const int b = min(R.a1, nt);
    // lane i of each head's row: the probe record of step f0 + i
    auto load = [&](BlockRecs<HBM>& B, int f0) {
        B.clear();
        if (f0 + i < b) {
            const long long rec = (long long)grp * P.nt_max + f0 + i;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                if (D.hv[hb]) {
                    const float* pr = P.round_probe + (rec * P.G + 4 * hb + fl.hl) * kRoundRecW;
                    B.m[hb] = cld(pr + 0);
                    B.l[hb] = cld(pr + 1);
#pragma unroll
                    for (int j = 0; j < 8; ++j) B.p[hb][j] = cld(pr + 2 + j);
                    B.e[hb] = __float_as_int(cld(pr + 10));
                }
            }
        }
    };
    // three blocks of records in flight: blocks f + 16 and f + 32 load while
    // block f is decided
    BlockRecs<HBM> B0, B1, B2;
    load(B0, R.a0);
    load(B1, R.a0 + 16);
    for (int f0 = R.a0; f0 < b; f0 += 48) {
        load(B2, f0 + 32);
        decide_pass<HBM>(P, D, B0, f0, min(16, b - f0), min(16, b - f0), nt);
        if (D.finished() || f0 + 16 >= b) break;
        load(B0, f0 + 48);
        decide_pass<HBM>(P, D, B1, f0 + 16, min(16, b - f0 - 16), min(16, b - f0 - 16), nt);
        if (D.finished() || f0 + 32 >= b) break;
        load(B1, f0 + 64);
        decide_pass<HBM>(P, D, B2, f0 + 32, min(16, b - f0 - 32), min(16, b - f0 - 32), nt);
        if (D.finished()) break;
    }
    if (D.finished()) {
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb)
            if (D.hv[hb] && i == 0) P.tiles_used[qrow(P, grp, 4 * hb + fl.hl)] = D.err[hb] ? -1 : D.U[hb];
        return;  // no further round for this group
    }
    round_save<HBM>(P, grp, D);
    drain();
    if (lane == 0) cst(P.round_ctl + (long long)grp * kRoundCtlW, stamp(P.epoch, (unsigned)(R.r + 1)));
}

// zeroes the groups' control words (arrival counters, round stamps)
__global__ __launch_bounds__(256) void art_round_init_kernel(Params P) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < (long long)P.NG * kRoundCtlW) cst(P.round_ctl + i, 0ull);
}

// two waves per SIMD for the 8-head tile too (its register budget halves: on
// B4 x 40q/8kv at 128K the rounds took 888 us against 1 053 us at one wave)
template <class S>
__global__ __launch_bounds__(256, 2) void art_round_kernel(Params P, RoundArgs R) {
    extern __shared__ float lds[];
    constexpr int HBM = S::HBM;
    const int wv = wave_id(), lane = lane_id();
    const FoldLanes fl(P);
    S st;
    st.init(lds + wv * S::lds_floats(P));
    // the round's items (group, range) = (item / waves, item % waves), taken by
    // the grid's waves in turn: w, w + W, ...
    const long long items = (long long)P.NG * R.waves;
    const long long W = (long long)gridDim.x * kWavesPerWG;
    for (long long item = (long long)blockIdx.x * kWavesPerWG + wv; item < items; item += W) {
        const int grp = (int)(item / R.waves), k = (int)(item % R.waves);
        unsigned long long* ctl = P.round_ctl + (long long)grp * kRoundCtlW;
        // a group takes round r > 0 only if round r - 1 left heads undecided
        if (R.r > 0 && uni64(cld(ctl)) != stamp(P.epoch, (unsigned)R.r)) continue;
        const int n = P.ctx_lens[seq_of(P, grp)];
        const bool bad = n < 0 || n > P.cap;
        const int nt = bad ? 0 : (n + S::T - 1) / S::T;
        const int t0 = R.a0 + k * R.pw;
        const int t1 = min(min(t0 + R.pw, R.a1), nt);
        unsigned long long loaded = 0, rows = 0;
        if (t0 < t1) {
            st.load_q(P, grp);  // before the tile's loads: consume() counts those in issue order
            // (like a team worker: a tile's loads are issued once the previous
            // tile is consumed; the next block ids are loaded a tile ahead)
            typename S::TileRef C;
            S::resolve(P, grp, t0, C);
            st.template issue<0>(P, C, 0);
            st.template issue<1>(P, C, 1);
            int blkN = t0 + 1 < t1 ? S::fetch_blocks(P, grp, n, t0 + 1) : 0;
            Part<HBM> run;  // the running state through the current step
            run.clear();
            for (int t = t0;; ++t) {
                ++loaded;
                rows += S::rows_in(C);
                st.template consume<0>(P, C, 0, true);
                st.template consume<1>(P, C, 1, false);
                typename S::Out o;
                st.flush(P, o);
                const long long rec = (long long)grp * P.nt_max + t;
                float* slot = P.round_rec + rec * P.slot;
#pragma unroll
                for (int hb = 0; hb < HBM; ++hb) {
                    const int h = 4 * hb + fl.hl;
                    if (hb < fl.HB && h < P.G) {
                        // (1) the tile's own probe record (lane (hl, 0) of each head)
                        if (fl.cid == 0) {
                            float* pr = P.round_probe + (rec * P.G + h) * kRoundRecW;
                            cst(pr + 0, o.mf[hb]);
                            cst(pr + 1, o.lf[hb]);
#pragma unroll
                            for (int j = 0; j < 8; ++j) cst(pr + 2 + j, o.a[hb][j]);
                            cst(pr + 10, __int_as_float(C.err));
                        }
                        // (2) the running state through step t (read only by the
                        // final launch: plain stores, seen there after the launch boundary)
                        sm_merge(run.m[hb], run.l[hb], run.a[hb], o.mf[hb], o.lf[hb], o.a[hb]);
                        f4* a = reinterpret_cast<f4*>(slot + kSlotHeader + h * P.D + 8 * fl.cid);
                        a[0] = f4{run.a[hb][0], run.a[hb][1], run.a[hb][2], run.a[hb][3]};
                        a[1] = f4{run.a[hb][4], run.a[hb][5], run.a[hb][6], run.a[hb][7]};
                        if (fl.cid == 0) {
                            slot[h] = run.m[hb];
                            slot[16 + h] = run.l[hb];
                        }
                    }
                }
                if (t + 1 >= t1) break;
                S::resolve_from(P, grp, n, t + 1, blkN, C);
                st.template issue<0>(P, C, 0);
                st.template issue<1>(P, C, 1);
                if (t + 2 < t1) blkN = S::fetch_blocks(P, grp, n, t + 2);
            }
        }
        if (loaded) count_stats(P, loaded, rows);
        drain();  // every record of this item stored before its arrival
        // arrival: one atomic add per item (the call's first launch zeroed the counters)
        int cnt = 0;
        if (lane == 0)
            cnt = (int)__hip_atomic_fetch_add(ctl + 1 + R.r, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
        cnt = bcast0(cnt);
        if (cnt == R.waves) round_decide<HBM>(P, grp, R, nt, bad);
    }
}

// The outputs: per head, the running states of the waves' step ranges below
// its tiles_used (the range holding the stop cut there), merged.  SL
// work-groups of NW waves per group; wave w of slice sl takes ranges
// sl * NW + w, + SL * NW, ... (loaded NB at a time); the waves' states are
// merged in wave order through LDS, and the slices' states (through the
// full-mode partial slots) by the slice that finishes last, in slice order:
// a fixed order, so the output is deterministic.
template <int HBM, int NW, int NB>
__global__ __launch_bounds__(64 * NW) void art_round_combine_kernel(Params P, RoundPlan rp, int SL) {
    __shared__ float part[NW][HBM][64][10];  // per wave, head block, lane: M, L, 8 dims
    const int grp = blockIdx.x / SL, sl = blockIdx.x % SL;
    const int wv = wave_id(), lane = lane_id();
    const FoldLanes fl(P);
    const int gh = heads_in(P, grp);
    int U[HBM];
    int umax = 0;
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        const int h = 4 * hb + fl.hl;
        U[hb] = hb < fl.HB && h < gh ? P.tiles_used[qrow(P, grp, h)] : 0;
        umax = max(umax, U[hb]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) umax = max(umax, __shfl_xor(umax, o));
    umax = uni(umax);
    Part<HBM> acc;
    acc.clear();
    // the ranges of this wave, a batch at a time
    const int me = sl * NW + wv, stride = SL * NW;
    int c = 0, nb = 0;
    int lo[NB] = {}, hi[NB] = {};
    auto flush_batch = [&]() {
        float m2[NB][HBM], l2[NB][HBM], a2[NB][HBM][8];
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                m2[q][hb] = kNegInf;
                l2[q][hb] = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) a2[q][hb][j] = 0.f;
                const int h = 4 * hb + fl.hl;
                if (q < nb && U[hb] > lo[q] && fl.cvalid) {
                    const int last = min(hi[q], U[hb]) - 1;
                    const float* slot = P.round_rec + ((long long)grp * P.nt_max + last) * P.slot;
                    m2[q][hb] = slot[h];
                    l2[q][hb] = slot[16 + h];
                    const f4* a = reinterpret_cast<const f4*>(slot + kSlotHeader + h * P.D + 8 * fl.cid);
                    const f4 x = a[0], y = a[1];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        a2[q][hb][j] = x[j];
                        a2[q][hb][4 + j] = y[j];
                    }
                }
            }
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) sm_merge(acc.m[hb], acc.l[hb], acc.a[hb], m2[q][hb], l2[q][hb], a2[q][hb]);
        nb = 0;
    };
    // range k of round r has index c + k (c: the ranges of the rounds before)
    for (int r = 0; r < rp.R && rp.a[r] < umax; c += rp.waves[r], ++r) {
        for (int k = ((me - c) % stride + stride) % stride; k < rp.waves[r]; k += stride) {
            const int c0 = rp.a[r] + k * rp.pw[r];
            if (c0 >= umax) break;
            const int c1 = min(c0 + rp.pw[r], rp.a[r + 1]);
#pragma unroll
            for (int q = 0; q < NB; ++q)
                if (q == nb) {
                    lo[q] = c0;
                    hi[q] = c1;
                }
            if (++nb == NB) flush_batch();
        }
    }
    if (nb > 0) flush_batch();
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        float* e = part[wv][hb][lane];
        e[0] = acc.m[hb];
        e[1] = acc.l[hb];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[2 + j] = acc.a[hb][j];
    }
    __syncthreads();
    if (wv != 0) return;
    // this slice's state: its waves in order
    Part<HBM> tot;
    tot.clear();
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb)
        for (int w = 0; w < NW; ++w) {
            const float* e = part[w][hb][lane];
            float a2[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) a2[j] = e[2 + j];
            sm_merge(tot.m[hb], tot.l[hb], tot.a[hb], e[0], e[1], a2);
        }
    if (SL > 1) {
        // through slot sl of the group's partials; the last slice merges them all
        // (the full-mode partial layout: max and sum at [h] and [16 + h], the
        // accumulator at kSlotHeader + h * D)
        float* base = P.partials + (long long)grp * P.splits * P.slot;
        float* slot = base + (long long)sl * P.slot;
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            const int h = 4 * hb + fl.hl;
            if (hb >= fl.HB || h >= gh) continue;
            if (fl.cid == 0) {
                cst(slot + h, tot.m[hb]);
                cst(slot + 16 + h, tot.l[hb]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) cst(slot + kSlotHeader + h * P.D + 8 * fl.cid + j, tot.a[hb][j]);
        }
        drain();
        int cnt = 0;
        if (lane == 0)
            cnt = (int)__hip_atomic_fetch_add(P.round_ctl + (long long)grp * kRoundCtlW + kRoundCtlW - 1, 1ull,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
        if (bcast0(cnt) != SL) return;
        tot.clear();
        for (int q = 0; q < SL; ++q) {
            const float* src = base + (long long)q * P.slot;
#pragma unroll
            for (int hb = 0; hb < HBM; ++hb) {
                const int h = 4 * hb + fl.hl;
                if (hb >= fl.HB || h >= gh) continue;
                float a2[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) a2[j] = cld(src + kSlotHeader + h * P.D + 8 * fl.cid + j);
                sm_merge(tot.m[hb], tot.l[hb], tot.a[hb], cld(src + h), cld(src + 16 + h), a2);
            }
        }
    }
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        const int h = 4 * hb + fl.hl;
        if (hb >= fl.HB || h >= gh) continue;
        float A[8], L = tot.l[hb];
#pragma unroll
        for (int j = 0; j < 8; ++j) A[j] = tot.a[hb][j];
        if (U[hb] == 0) {
            // empty row: out = 0
#pragma unroll
            for (int j = 0; j < 8; ++j) A[j] = 0.f;
            L = 1.f;
        }
        write_head_out(P, grp, h, fl, A, L, U[hb] < 0, U[hb]);
    }
}

template <class Tile>
__global__ __launch_bounds__(256) void art_full_kernel(Params P) {
    extern __shared__ float lds[];
    const int wv = wave_id(), lane = lane_id();
    float* lds_wave = lds + wv * Tile::lds_floats(P);
    const int worker = blockIdx.x * kWavesPerWG + wv;
    if (worker >= P.NG * P.splits) return;
    const FoldLanes fl(P);
    const int grp = worker / P.splits, sp = worker % P.splits;
    const int b = grp / P.Hkv, g = grp % P.Hkv;
    const int n = P.ctx_lens[seq_of(P, grp)];
    const bool bad = n < 0 || n > P.cap;
    const int nt = bad ? 0 : (n + P.T - 1) / P.T;
    const int t0 = sp * P.tiles_per_split;
    const int t1 = min(t0 + P.tiles_per_split, nt);
    constexpr int HBM = Tile::HBM;
    float M[HBM], L[HBM], A[HBM][8];
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        M[hb] = kNegInf; L[hb] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) A[hb][j] = 0.f;
    }
    int err = 0, kept_total = 0;
    Tile tile;
    if (t0 < t1) tile.load_q(P, b, g, lds_wave);
    auto hook = [&](const float (&ml)[kMaxG], float (&Mt)[kMaxG]) -> bool {
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) Mt[h] = ml[h];
        return true;
    };
    for (int t = t0; t < t1; ++t) {
        typename Tile::Out o;
        tile.compute(P, b, g, n, t, hook, o);
        err |= o.err;
        kept_total += o.kept;
#pragma unroll
        for (int hb = 0; hb < HBM; ++hb) {
            const int h = hb * 4 + fl.hl;
            // this lane's head: select its tile max and sum from the uniform arrays
            float ml = kNegInf, ll = 0.f;
#pragma unroll
            for (int hh = 0; hh < kMaxG; ++hh)
                if (hh == h) { ml = o.m[hh]; ll = o.l[hh]; }
            if (hb < fl.HB && h < P.G) {
                const float mn = fmaxf(M[hb], ml);
                const bool first = M[hb] == kNegInf;
                const float al = first ? 0.f : expf(M[hb] - mn);
                const float be = expf(ml - mn);
                L[hb] = fmaf(al, L[hb], be * ll);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    A[hb][j] = first ? be * o.a[hb][j] : fmaf(al, A[hb][j], be * o.a[hb][j]);
                M[hb] = mn;
            }
        }
    }
    float* slot = P.partials + ((long long)grp * P.splits + sp) * P.slot;
#pragma unroll
    for (int hb = 0; hb < HBM; ++hb) {
        const int h = hb * 4 + fl.hl;
        if (hb < fl.HB && h < P.G) {
            if (fl.cid == 0) {
                slot[h] = M[hb];
                slot[16 + h] = L[hb];
            }
            if (fl.cvalid) {
                float* a = slot + kSlotHeader + h * P.D + 8 * fl.cid;
#pragma unroll
                for (int j = 0; j < 8; ++j) a[j] = A[hb][j];
            }
        }
    }
    if (lane == 0) {
        reinterpret_cast<int*>(slot)[32] = err;
        reinterpret_cast<int*>(slot)[33] = kept_total;
    }
    if (t1 > t0) count_stats(P, (unsigned long long)(t1 - t0), (unsigned long long)kept_total);
}

// Full mode, streamed: one running state over the whole split range.
template <class S>
__global__ __launch_bounds__(256, S::MIN_WAVES) void art_full_stream_kernel(Params P) {
    extern __shared__ float lds[];
    const int wv = wave_id(), lane = lane_id();
    const int worker = blockIdx.x * kWavesPerWG + wv;
    if (worker >= P.NG * P.splits) return;
    const FoldLanes fl(P);
    const int grp = worker / P.splits, sp = worker % P.splits;
    const int n = P.ctx_lens[seq_of(P, grp)];
    const bool bad = n < 0 || n > P.cap;
    const int nt = bad ? 0 : (n + S::T - 1) / S::T;
    const int t0 = sp * P.tiles_per_split;
    const int t1 = min(t0 + P.tiles_per_split, nt);
    S st;
    st.init(lds + wv * S::lds_floats(P));
    int err = 0, rows = 0;
    typename S::Out o;
    if (t0 < t1) {
        st.load_q(P, grp);
        typename S::TileRef C, N;
        S::resolve(P, grp, t0, C);
        st.template issue<0>(P, C, 0);
        st.template issue<1>(P, C, 1);
        for (int t = t0; t < t1; ++t) {
            const bool more = t + 1 < t1;
            if (more) S::resolve(P, grp, t + 1, N);
            err |= C.err;
            rows += S::named(C.t) ? min(S::T, n - C.t * S::T) : 0;
            st.template consume<0>(P, C, 0, true);
            if (more) st.template issue<0>(P, N, 0);
            st.template consume<1>(P, C, 1, more);
            if (more) st.template issue<1>(P, N, 1);
            C = N;
        }
    }
    st.flush(P, o);
    float* slot = P.partials + ((long long)grp * P.splits + sp) * P.slot;
#pragma unroll
    for (int hb = 0; hb < S::HBM; ++hb) {
        const int h = hb * 4 + fl.hl;
        if (hb < fl.HB && h < P.G && fl.cvalid) {
            float* a = slot + kSlotHeader + h * P.D + 8 * fl.cid;
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] = o.a[hb][j];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            if (h < P.G) {
                slot[h] = o.m[h];
                slot[16 + h] = o.l[h];
            }
        }
        reinterpret_cast<int*>(slot)[32] = err;
        reinterpret_cast<int*>(slot)[33] = rows;
        if (t1 > t0 && P.stats) {
            atomicAdd(reinterpret_cast<unsigned long long*>(P.stats + 0), (unsigned long long)(t1 - t0));
            atomicAdd(reinterpret_cast<unsigned long long*>(P.stats + 1), (unsigned long long)rows);
        }
    }
}

// One work-group of kCombineWaves waves per group merges the splits and
// writes the outputs.  Wave w takes splits w, w + kCombineWaves, ...,
// kCombineBatch of them loaded at once (independent loads, many in flight)
// and merged in split order; the waves' results are then merged in wave
// order through LDS.  The order is fixed: the output is deterministic.
constexpr int kCombineWaves = 4;
constexpr int kCombineBatch = 8;  // splits a wave loads at once

__global__ __launch_bounds__(64 * kCombineWaves) void art_combine_kernel(Params P) {
    __shared__ float part[kCombineWaves][4][64][10];  // per wave, head block, lane: M, L, 8 dims
    __shared__ int perr[kCombineWaves];
    const int grp = blockIdx.x;
    const int wv = wave_id(), lane = lane_id();
    const FoldLanes fl(P);
    const int G = P.G, D = P.D;
    const int b = grp / P.Hkv, g = grp % P.Hkv;
    const int n = P.ctx_lens[seq_of(P, grp)];
    const bool bad = n < 0 || n > P.cap;
    const int nt = bad ? 0 : (n + P.T - 1) / P.T;
    const float* base = P.partials + (long long)grp * P.splits * P.slot;
    int err = 0;
    for (int sp = wv; sp < P.splits; sp += kCombineWaves)
        err |= reinterpret_cast<const int*>(base + (long long)sp * P.slot)[32];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
        const int h = hb * 4 + fl.hl;
        float M = kNegInf, L = 0.f, A[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (hb < fl.HB && h < G) {
            // one pass, kCombineBatch splits loaded at a time and merged in
            // order; splits with no rows (l = 0) take no part
            for (int s0 = wv; s0 < P.splits; s0 += kCombineWaves * kCombineBatch) {
                float m2[kCombineBatch], l2[kCombineBatch], a2[kCombineBatch][8];
#pragma unroll
                for (int q = 0; q < kCombineBatch; ++q) {
                    const int sp = s0 + q * kCombineWaves;
                    m2[q] = kNegInf;
                    l2[q] = 0.f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) a2[q][j] = 0.f;
                    if (sp < P.splits) {
                        const float* slot = base + (long long)sp * P.slot;
                        l2[q] = slot[16 + h];
                        m2[q] = l2[q] > 0.f ? slot[h] : kNegInf;
                        if (fl.cvalid) {
                            const float* a = slot + kSlotHeader + h * D + 8 * fl.cid;
#pragma unroll
                            for (int j = 0; j < 8; ++j) a2[q][j] = a[j];
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < kCombineBatch; ++q) sm_merge(M, L, A, m2[q], l2[q], a2[q]);
            }
        }
        float* e = part[wv][hb][lane];
        e[0] = M;
        e[1] = L;
#pragma unroll
        for (int j = 0; j < 8; ++j) e[2 + j] = A[j];
    }
    if (lane == 0) perr[wv] = err;
    __syncthreads();
    if (wv != 0) return;
    for (int w = 1; w < kCombineWaves; ++w) err |= perr[w];
    if (bad) err = 1;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
        const int h = hb * 4 + fl.hl;
        if (hb >= fl.HB || h >= G) continue;
        float M = kNegInf, L = 0.f, A[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int w = 0; w < kCombineWaves; ++w) {
            const float* e = part[w][hb][lane];
            float a2[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) a2[j] = e[2 + j];
            sm_merge(M, L, A, e[0], e[1], a2);
        }
        if (nt == 0 && !bad) {
            const long long row = (long long)b * P.Hq + (long long)g * G + h;
            if (fl.cvalid)
                for (int j = 0; j < 8; ++j) P.out[row * D + 8 * fl.cid + j] = 0.f;
            if (fl.cid == 0) P.tiles_used[row] = 0;
        } else {
            write_head_out(P, grp, h, fl, A, L, err, nt);
        }
    }
}

// ------------------------------------------------------------------ launches
// Compute units of the current device, queried once per device.
int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev] = cus;
    }
    return cached[dev];
}

// Resident work-groups per CU of `kernel` at this block size and dynamic LDS,
// queried once per (device, kernel, block size, LDS) and kept.
int resident_per_cu(const void* kernel, hipError_t (*query)(int*, const void*, int, size_t), int block,
                    size_t lds) {
    struct Entry {
        const void* kernel;
        int dev, block;
        size_t lds;
        int value;
    };
    static Entry cache[256];
    static int used = 0;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].kernel == kernel && cache[i].dev == dev && cache[i].block == block && cache[i].lds == lds)
            return cache[i].value;
    int v = 0;
    if (query(&v, kernel, block, lds) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    if (used < 256) cache[used++] = Entry{kernel, dev, block, lds, v};
    return v;
}
template <class K>
hipError_t occupancy_of(int* v, const void* kernel, int block, size_t lds) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(v, reinterpret_cast<K>(const_cast<void*>(kernel)), block, lds);
}
template <class K>
int resident(K kernel, int block, size_t lds) {
    return resident_per_cu(reinterpret_cast<const void*>(kernel), &occupancy_of<K>, block, lds);
}

// Persistent grid: the deciders first (the lowest work-groups are dispatched
// first, so they are resident from the start), then the tile workers; without
// a requested worker count, as many as are resident together with them.
template <class K, class Tile>
int launch_persistent(const Params& p0, hipStream_t s, K kernel) {
    Params p = p0;
    const size_t lds = (size_t)kWavesPerWG * Tile::lds_floats(p) * sizeof(float);
    // Deciders wait for workers and workers for deciders (ring space, the V
    // skip's running maxima): every wave of the grid must be resident at
    // once, which only a cooperative launch guarantees.  The worker count is
    // therefore capped at what fits beside the deciders, and the launch is
    // cooperative or fails.
    const int cus = device_cus(), per_cu = resident(kernel, 256, lds);
    if (cus <= 0) return (int)hipErrorInvalidDevice;
    const long long fit = (long long)per_cu * cus * kWavesPerWG - p.deciders;
    if (fit < 1) return (int)hipErrorCooperativeLaunchTooLarge;
    long long w = p.workers > 0 ? p.workers : fit;
    if (w > fit) w = fit;
    if (p.workers == 0) {
        const long long tiles = (long long)p.NG * p.nt_max;
        if (w > tiles) w = tiles;
        if (w > (long long)kMaxWorkersPerGroup * p.NG) w = (long long)kMaxWorkersPerGroup * p.NG;
    }
    p.workers = (int)max(w, 1LL);
    hipLaunchKernelGGL(art_init_kernel, dim3(p.NG), dim3(256), 0, s, p);
    const int blocks = (p.deciders + p.workers + kWavesPerWG - 1) / kWavesPerWG;
    void* args[] = {&p};
    return (int)hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel), dim3(blocks), dim3(256), args,
                                           (unsigned)lds, s);
}

template <class K, class Tile>
int launch_split(const Params& p, hipStream_t s, K kernel) {
    const size_t lds = (size_t)kWavesPerWG * Tile::lds_floats(p) * sizeof(float);
    const int blocks = (p.NG * p.splits + kWavesPerWG - 1) / kWavesPerWG;
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(256), lds, s, p);
    hipLaunchKernelGGL(art_combine_kernel, dim3(p.NG), dim3(64 * kCombineWaves), 0, s, p);
    return (int)hipGetLastError();
}

// Matrix-core tiles serve bf16/int8 caches with head dim 128, bf16 queries,
// at most 8 query heads per KV head and tiles of 16, 32 or 64 tokens; 64-token
// tiles without the V skip are streamed.
bool fast_path(const Params& p) {
    return p.D == 128 && p.q_dtype == ART_BF16 && p.G <= 8 &&
           (((p.kv_dtype == ART_BF16 || p.kv_dtype == ART_I8) && (p.T == 16 || p.T == 32 || p.T == 64)) ||
            (p.kv_dtype == ART_I4 && p.T == 64));
}
// the work-sharing engine serves ART mode
bool sharing(const Params& p) {
    return p.engine == ART_ENGINE_SHARED || (p.engine == ART_ENGINE_AUTO && p.workers > 0);
}
// Streamed 64-token tiles: the team and pool engines (ART; the V skip on the
// team engine), the work-sharing engine (ART without the V skip) and full mode.
bool stream_path(const Params& p, bool art) {
    return fast_path(p) && p.T == 64 && (!p.vskip || (art && !sharing(p)));
}

template <class Tile>
int run_tile(const Params& p, hipStream_t s, bool art) {
    if (art) return launch_persistent<decltype(&art_persistent_kernel<Tile>), Tile>(p, s, &art_persistent_kernel<Tile>);
    return launch_split<decltype(&art_full_kernel<Tile>), Tile>(p, s, &art_full_kernel<Tile>);
}

// The pair kernel where it applies (both roles resident at once, one
// work-group per CU); 0 if launched, else nonzero (the caller falls back).
template <class S>
int launch_pair(const Params& p0, hipStream_t s) {
    if constexpr (S::GM != 4) {
        return 1;
    } else {
        Params p = p0;
        if (p.vskip || p.NG % 8 != 0 || p.NG > kTeamHelpGroups) return 1;
        const int cus = device_cus();
        const size_t lds = pair_lds_bytes<S>();
        const int per_cu = resident(&art_pair_kernel<S>, S::TEAM * 64, lds);
        if (cus <= 0 || per_cu < 1 || 2LL * p.NG > (long long)cus * per_cu) return 1;
        void* args[] = {&p};
        const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&art_pair_kernel<S>),
                                                        dim3(2 * p.NG), dim3(S::TEAM * 64), args, (unsigned)lds, s);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return 1;
        }
        return 0;
    }
}

// Helpers (as many as requested, up to what fits) only where every
// work-group of the grid can be resident at once (cooperative launch); else
// the primaries alone.
template <class S, int VSKIP>
int launch_team(const Params& p0, hipStream_t s) {
    Params p = p0;
    const size_t lds = team_lds_bytes<S>(p);
    p.helpers = 0;
    int cus = 0, per_cu = 0;
    if (!VSKIP && p0.helpers > 0 && p.NG <= kTeamHelpGroups && (cus = device_cus()) > 0 &&
        (per_cu = resident(&art_team_kernel<S, VSKIP>, S::TEAM * 64, lds)) > 0) {
        const long long resident = (long long)per_cu * cus;
        long long h = resident / p.NG - 1;
        if (h > p0.helpers) h = p0.helpers;
        if (h > 0) {
            p.helpers = (int)h;
            void* args[] = {&p};
            const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&art_team_kernel<S, VSKIP>),
                                                            dim3(p.NG * (1 + p.helpers)), dim3(S::TEAM * 64), args,
                                                            (unsigned)lds, s);
            if (e == hipSuccess) return 0;
            (void)hipGetLastError();  // cannot be resident together: primaries alone
            p.helpers = 0;
        }
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL((art_team_kernel<S, VSKIP>), dim3(p.NG), dim3(S::TEAM * 64), lds, s, p);
    return (int)hipGetLastError();
}

// One work-group per resident slot, all resident (cooperative launch), as
// long as each group's decider has a work-group; returns 1 when it did not
// launch (too many groups), so that the team engine runs instead.
template <class S>
int launch_pool(const Params& p0, hipStream_t s) {
    Params p = p0;
    const size_t lds = pool_lds_bytes<S>(p);
    const int cus = device_cus(), per_cu = resident(&art_pool_kernel<S>, PoolShape<S>::WAVES * 64, lds);
    if (cus <= 0 || per_cu < 1) {
        (void)hipGetLastError();
        return 1;
    }
    const long long grid = (long long)per_cu * cus;
    if (p.NG > grid || p.NG > kTeamHelpGroups) return 1;
    p.pool_cap = kPoolContrib;
    void* args[] = {&p};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&art_pool_kernel<S>), dim3((unsigned)grid),
                                                    dim3(PoolShape<S>::WAVES * 64), args, (unsigned)lds, s);
    if (e == hipSuccess) return 0;
    (void)hipGetLastError();
    return 1;
}


constexpr int kRoundCombineCUs = 256;  // work-groups of the round engine's final launch, about
constexpr int kRoundMaxSlices = 8;     // work-groups per group of that launch at most
constexpr int kXpDefaultWindow = 64;  // tiles past the decided frontier a worker may load, by default

// One work-group per CU, all resident (cooperative launch); returns 1 when it
// cannot run (too many groups, a CU count not divisible over the XCDs, or the
// grid would not be resident), so that the team engine runs instead.
template <class S>
int launch_xp(const Params& p0, hipStream_t s) {
    Params p = p0;
    const int cus = device_cus();
    if (cus <= 0 || cus % kXcd || p.NG > kTeamHelpGroups) {
        (void)hipGetLastError();
        return 1;
    }
    const int per_xcd = cus / kXcd;
    const int nx = (p.NG + kXcd - 1) / kXcd;
    p.xp_dec_wgs = (nx + kXpDeciderWaves - 1) / kXpDeciderWaves;
    if (p.xp_dec_wgs >= per_xcd) return 1;
    int wpc = p.xp_wpc_req > 0 ? p.xp_wpc_req : XpShape<S>::MAXW;
    if (wpc > XpShape<S>::MAXW) wpc = XpShape<S>::MAXW;
    if (wpc < 1) return 1;
    p.xp_wpc = wpc;
    p.xp_window = p.xp_window_req > 0 ? p.xp_window_req : kXpDefaultWindow;
    if (p.xp_window > kXpMaxWindow) p.xp_window = kXpMaxWindow;
    p.pool_cap = kPoolContrib;
    // at least half a CU's LDS, so that no CU takes two work-groups
    size_t lds = (size_t)wpc * XpShape<S>::WAVE_FLOATS * sizeof(float);
    if (lds < 82 * 1024) lds = 82 * 1024;
    void* args[] = {&p};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&art_xp_kernel<S>), dim3((unsigned)cus),
                                                    dim3(kXpWaves * 64), args, (unsigned)lds, s);
    if (e == hipSuccess) return 0;
    (void)hipGetLastError();
    return 1;
}

// The round engine: one launch per round, then the outputs; returns 1 when it
// does not apply (its workspace regions were not laid out, or the rows need
// more than kMaxRounds rounds), so that the team engine runs instead.
template <class S>
int launch_round(const Params& p, hipStream_t s) {
    if (!p.round_rec || S::HBM > 2) return 1;
    const RoundPlan rp = round_plan(p.nt_max, p.NG);
    if (rp.R == 0) return 1;
    const size_t lds = (size_t)kWavesPerWG * S::lds_floats(p) * sizeof(float);
    const long long words = (long long)p.NG * kRoundCtlW;
    hipLaunchKernelGGL(art_round_init_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, p);
    // each round: at most as many work-groups as are resident at once, their
    // waves taking the round's items in turn
    const int cus = device_cus(), per_cu = resident(&art_round_kernel<S>, 64 * kWavesPerWG, lds);
    const long long slots = cus > 0 && per_cu > 0 ? (long long)cus * per_cu : 1024;
    for (int r = 0; r < rp.R; ++r) {
        const RoundArgs ra{r, rp.a[r], rp.a[r + 1], rp.pw[r], rp.waves[r]};
        long long blocks = ((long long)p.NG * ra.waves + kWavesPerWG - 1) / kWavesPerWG;
        if (blocks > slots) blocks = slots;
        hipLaunchKernelGGL((art_round_kernel<S>), dim3((unsigned)blocks), dim3(64 * kWavesPerWG), lds, s, p, ra);
    }
    // slices per group: about one work-group per CU over all groups, within
    // the partial slots the workspace holds
    int sl = kRoundCombineCUs / p.NG;
    if (sl > kRoundMaxSlices) sl = kRoundMaxSlices;
    if (sl > p.splits) sl = p.splits;
    if (sl < 1) sl = 1;
    const unsigned grid = (unsigned)((long long)p.NG * sl);
    if constexpr (S::HBM == 1)
        hipLaunchKernelGGL((art_round_combine_kernel<1, 16, 8>), dim3(grid), dim3(64 * 16), 0, s, p, rp, sl);
    else
        hipLaunchKernelGGL((art_round_combine_kernel<2, 8, 4>), dim3(grid), dim3(64 * 8), 0, s, p, rp, sl);
    return (int)hipGetLastError();
}

// engine AUTO takes the rounds on the shapes art::round_auto names
bool round_auto(const Params& p) { return art::round_auto(p.NG, p.G, p.nt_max); }

template <class S>
int run_stream(const Params& p, hipStream_t s, bool art) {
    if constexpr (S::ORDER == ART_ORDER_LIST) {
        const long long recs = (long long)(p.NG / p.seq_div) * p.nt_max;
        if (recs > 0) {
            hipLaunchKernelGGL(art_steps_kernel, dim3((unsigned)((recs + 255) / 256)), dim3(256), 0, s, p);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    if (!art) return launch_split<decltype(&art_full_stream_kernel<S>), S>(p, s, &art_full_stream_kernel<S>);
    if (sharing(p)) return launch_persistent<decltype(&art_stream_kernel<S>), S>(p, s, &art_stream_kernel<S>);
    // The V skip on bf16 caches: a tile's V rows are loaded after its scores,
    // only those some head keeps.  On int8 and int4 caches the tile is bound
    // by its arithmetic rather than its loads, the second round trip costs
    // more than the rows left out save, and the V rows come with the tile's
    // K (the skip leaves out their share of P.V).
    if (p.vskip) return S::KVT == ART_BF16 ? launch_team<S, 2>(p, s) : launch_team<S, 1>(p, s);
    if ((p.engine == ART_ENGINE_ROUND || (p.engine == ART_ENGINE_AUTO && round_auto(p))) && launch_round<S>(p, s) == 0)
        return 0;
    if (p.engine == ART_ENGINE_XCD && launch_xp<S>(p, s) == 0) return 0;
    if (p.engine == ART_ENGINE_PAIR && launch_pair<S>(p, s) == 0) return 0;
    // by default the pool serves few, long groups (where one CU per group
    // would leave most of the chip idle)
    const bool pool = p.engine == ART_ENGINE_POOL ||
                      (p.engine == ART_ENGINE_AUTO && p.NG <= kPoolAutoGroups && p.nt_max >= kPoolAutoTiles);
    if (pool && launch_pool<S>(p, s) == 0) return 0;
    return launch_team<S, 0>(p, s);
}

template <int KV, int GMAX>
int run_fast(const Params& p, hipStream_t s, bool art) {
    if (stream_path(p, art))
        return p.order == ART_ORDER_ASCENDING ? run_stream<Stream<KV, GMAX, ART_ORDER_ASCENDING>>(p, s, art)
               : p.order == ART_ORDER_RECENT  ? run_stream<Stream<KV, GMAX, ART_ORDER_RECENT>>(p, s, art)
                                              : run_stream<Stream<KV, GMAX, ART_ORDER_LIST>>(p, s, art);
    if constexpr (KV == ART_I4) {
        // int4 has only the streamed 64-token tile; the rest runs on the generic tile
        return run_tile<GenericTile<128, ART_I4>>(p, s, art);
    } else {
        if (p.T == 64) return run_tile<FastTile<KV, 4, GMAX>>(p, s, art);
        if (p.T == 32) return run_tile<FastTile<KV, 2, GMAX>>(p, s, art);
        return run_tile<FastTile<KV, 1, GMAX>>(p, s, art);
    }
}

}  // namespace

// The launch code is split into parts by cache format, so that the library
// can be compiled as several translation units in parallel (ART_PART = 0..3,
// one object each); without ART_PART one translation unit holds every part.
#ifndef ART_PART
#define ART_PART -1
#endif
int run_part_bf16(const Params& p, hipStream_t s, bool art);
int run_part_i8(const Params& p, hipStream_t s, bool art);
int run_part_i4(const Params& p, hipStream_t s, bool art);
int run_part_generic(const Params& p, hipStream_t s, bool art);

#if ART_PART < 0 || ART_PART == 1
int run_part_bf16(const Params& p, hipStream_t s, bool art) {
    return p.G <= 4 ? run_fast<ART_BF16, 4>(p, s, art) : run_fast<ART_BF16, 8>(p, s, art);
}
#endif
#if ART_PART < 0 || ART_PART == 2
int run_part_i8(const Params& p, hipStream_t s, bool art) {
    return p.G <= 4 ? run_fast<ART_I8, 4>(p, s, art) : run_fast<ART_I8, 8>(p, s, art);
}
#endif
#if ART_PART < 0 || ART_PART == 3
int run_part_i4(const Params& p, hipStream_t s, bool art) {
    return p.G <= 4 ? run_fast<ART_I4, 4>(p, s, art) : run_fast<ART_I4, 8>(p, s, art);
}
#endif
#if ART_PART < 0 || ART_PART == 0
int run_part_generic(const Params& p, hipStream_t s, bool art) {
    if (p.D == 64) {
        if (p.kv_dtype == ART_F32) return run_tile<GenericTile<64, ART_F32>>(p, s, art);
        if (p.kv_dtype == ART_BF16) return run_tile<GenericTile<64, ART_BF16>>(p, s, art);
        if (p.kv_dtype == ART_I8) return run_tile<GenericTile<64, ART_I8>>(p, s, art);
        return run_tile<GenericTile<64, ART_I4>>(p, s, art);
    }
    if (p.kv_dtype == ART_F32) return run_tile<GenericTile<128, ART_F32>>(p, s, art);
    if (p.kv_dtype == ART_BF16) return run_tile<GenericTile<128, ART_BF16>>(p, s, art);
    if (p.kv_dtype == ART_I8) return run_tile<GenericTile<128, ART_I8>>(p, s, art);
    return run_tile<GenericTile<128, ART_I4>>(p, s, art);
}

namespace {
int run(const Params& p, hipStream_t s, bool art) {
    if (fast_path(p)) {
        if (p.kv_dtype == ART_BF16) return run_part_bf16(p, s, art);
        if (p.kv_dtype == ART_I8) return run_part_i8(p, s, art);
        return run_part_i4(p, s, art);
    }
    return run_part_generic(p, s, art);
}
}  // namespace

int launch_art(const Params& p, void* stream) {
    (void)hipGetLastError();
    if (p.NG == 0) return 0;
    return run(p, static_cast<hipStream_t>(stream), true);
}

int launch_full(const Params& p, void* stream) {
    (void)hipGetLastError();
    if (p.NG == 0) return 0;
    return run(p, static_cast<hipStream_t>(stream), false);
}
#endif

}  // namespace art
