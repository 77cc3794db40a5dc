// Host side of the C ABI (include/art.h): argument validation, workspace
// layout, launch planning.  Never reads device memory, never synchronises.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "art.h"
#include "art_internal.h"

namespace {

thread_local std::string g_last_error;

// Call counter: every call gets its own epoch, which the team kernel stamps on
// the words it shares through the workspace, so that none left by an earlier
// call is taken for one of this call.
std::atomic<unsigned> g_epoch{0};

art_status fail(art_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

// worker waves the full-mode split aims for: 256 CUs x 8 resident waves
constexpr int kTargetWaves = 2048;
constexpr int kMinTilesPerSplit = 4;  // full mode: tiles per split at least (rows permitting)

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool finite_nonneg(float x) { return std::isfinite(x) && x >= 0.f; }

// Validates desc/tile/thresholds and fills the shape part of Params.
art_status check(const art_desc* d, int tile, float eps_scale, float eps_dir, art::Params& p) {
    if (!d) return fail(ART_E_NULL, "desc is NULL");
    if (d->batch < 0) return fail(ART_E_SHAPE, "batch %d < 0", d->batch);
    if (d->num_q_heads < 1 || d->num_kv_heads < 1)
        return fail(ART_E_SHAPE, "head counts must be >= 1 (q %d, kv %d)", d->num_q_heads, d->num_kv_heads);
    if (d->num_q_heads % d->num_kv_heads)
        return fail(ART_E_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d", d->num_q_heads,
                    d->num_kv_heads);
    const int G = d->num_q_heads / d->num_kv_heads;
    if (G > art::kMaxG) return fail(ART_E_SHAPE, "%d query heads per KV head; at most %d supported", G, art::kMaxG);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(ART_E_SHAPE, "head_dim %d; supported: 64, 128", d->head_dim);
    if (d->q_dtype != ART_F32 && d->q_dtype != ART_BF16)
        return fail(ART_E_DTYPE, "q_dtype %d; supported: ART_F32, ART_BF16", d->q_dtype);
    if (d->kv_dtype != ART_F32 && d->kv_dtype != ART_BF16 && d->kv_dtype != ART_I8 && d->kv_dtype != ART_I4)
        return fail(ART_E_DTYPE, "kv_dtype %d unknown", d->kv_dtype);
    if ((d->kv_dtype == ART_I8 || d->kv_dtype == ART_I4) && (!d->k_scale || !d->v_scale))
        return fail(ART_E_NULL, "int8 and int4 caches need k_scale and v_scale");
    if (tile != 16 && tile != 32 && tile != 64 && tile != 128)
        return fail(ART_E_TILE, "tile %d; supported: 16, 32, 64, 128", tile);
    long long cap;
    if (d->block_size) {
        if (d->block_size < 16 || d->block_size % 16)
            return fail(ART_E_SHAPE, "block_size %d must be a positive multiple of 16", d->block_size);
        if (d->batch > 0 && d->max_blocks_per_seq < 1)
            return fail(ART_E_SHAPE, "max_blocks_per_seq %d < 1", d->max_blocks_per_seq);
        if (d->num_blocks < 1) return fail(ART_E_SHAPE, "num_blocks %d < 1", d->num_blocks);
        cap = (long long)d->max_blocks_per_seq * d->block_size;
    } else {
        if (d->max_ctx < 0 || d->max_ctx % 16)
            return fail(ART_E_SHAPE, "max_ctx %d must be a non-negative multiple of 16", d->max_ctx);
        cap = d->max_ctx;
    }
    if (cap > (1LL << 30)) return fail(ART_E_SHAPE, "row capacity %lld tokens too large", cap);
    if (!finite_nonneg(eps_scale) || !finite_nonneg(eps_dir))
        return fail(ART_E_PARAM, "thresholds must be finite and >= 0 (got %g, %g)", eps_scale, eps_dir);
    if (!finite_nonneg(d->v_skip_eps)) return fail(ART_E_PARAM, "v_skip_eps %g must be finite and >= 0", d->v_skip_eps);
    if (d->patience < 1) return fail(ART_E_PARAM, "patience %d < 1", d->patience);
    if (d->max_workers < 0) return fail(ART_E_PARAM, "max_workers %d < 0", d->max_workers);
    if (d->team_helpers < 0 || d->team_helpers > art::kMaxHelpers)
        return fail(ART_E_PARAM, "team_helpers %d not in 0..%d", d->team_helpers, art::kMaxHelpers);
    if (d->engine < ART_ENGINE_AUTO || d->engine > ART_ENGINE_ROUND)
        return fail(ART_E_PARAM, "engine %d not in %d..%d", d->engine, ART_ENGINE_AUTO, ART_ENGINE_ROUND);
    if (d->workers_per_cu < 0) return fail(ART_E_PARAM, "workers_per_cu %d < 0", d->workers_per_cu);
    if (d->window < 0 || d->window > art::kXpMaxWindow)
        return fail(ART_E_PARAM, "window %d not in 0..%d", d->window, art::kXpMaxWindow);
    if (d->per_head_tables != 0 && d->per_head_tables != 1)
        return fail(ART_E_PARAM, "per_head_tables %d not 0 or 1", d->per_head_tables);
    if (d->tile_order < ART_ORDER_ASCENDING || d->tile_order > ART_ORDER_LIST)
        return fail(ART_E_PARAM, "tile_order %d not in %d..%d", d->tile_order, ART_ORDER_ASCENDING, ART_ORDER_LIST);
    if (d->tile_order == ART_ORDER_LIST) {
        if (!d->tile_perm) return fail(ART_E_NULL, "ART_ORDER_LIST needs tile_perm");
        const long long need = (cap + tile - 1) / tile;
        if (d->tile_perm_stride < need)
            return fail(ART_E_SHAPE, "tile_perm_stride %d < %lld tiles a row can hold", d->tile_perm_stride, need);
    }

    p = art::Params{};
    p.B = d->batch; p.Hq = d->num_q_heads; p.Hkv = d->num_kv_heads; p.G = G; p.D = d->head_dim; p.T = tile;
    p.q_dtype = d->q_dtype; p.kv_dtype = d->kv_dtype;
    p.block_size = d->block_size; p.mbps = d->max_blocks_per_seq; p.num_blocks = d->num_blocks;
    p.max_ctx = d->max_ctx;
    p.cap = (int)cap;
    p.nt_max = (int)((cap + tile - 1) / tile);
    p.NG = d->batch * d->num_kv_heads;
    p.hkv_cache = d->num_kv_heads;
    p.kv_shift = 0;
    p.gq = G;
    // Query-head split: decisions are per query head (a group only loads while
    // one of its heads is active), so in ART mode on the streamed 64-token tile
    // a KV head's G = 5..8 or 10..16 query heads run as 2 or 4 groups of at
    // most 4 heads, each reading the KV head's tiles for itself: the 4-head
    // tile runs twice the waves per CU and twice as many CUs work, which
    // outweighs the repeated reads (measured up to two groups per CU).  q, out
    // and tiles_used keep their layout (a group's heads stay contiguous).
    // G = 5 or 7 (and 10, 11, 13..15) split unevenly: groups of ceil(G / 2)
    // (or ceil(G / 4)) heads with a smaller last one; only the team and pool
    // engines track the per-group head count, so an uneven split is not used
    // with the work-sharing engine or helper work-groups.
    {
        const bool art_mode = eps_scale > 0.f && eps_dir > 0.f;
        const bool streamed = d->head_dim == 128 && d->q_dtype == ART_BF16 && tile == 64 &&
                              (d->kv_dtype == ART_BF16 || d->kv_dtype == ART_I8 || d->kv_dtype == ART_I4);
        const bool sharing = d->max_workers > 0 || d->engine == ART_ENGINE_SHARED || d->team_helpers > 0;
        int shift = 0;
        if (G > 4 && G <= 8) shift = 1;
        else if (G > 8 && 3 * ((G + 3) / 4) < G) shift = 2;  // every one of the 4 groups keeps a head
        const int gv = (G + (1 << shift) - 1) >> shift;
        const bool even = (gv << shift) == G;
        // (the round engine loads a KV head's tiles once for all its query heads)
        if (art_mode && streamed && shift > 0 && (even || !sharing) && d->engine != ART_ENGINE_ROUND &&
            (long long)p.NG << shift <= art::kMaxSplitGroups) {
            p.kv_shift = shift;
            p.Hkv <<= shift;
            p.G = gv;
            p.NG <<= shift;
        }
    }
    // the round engine's regions: ART mode on the streamed tile without the
    // V skip, no work-sharing engine or helpers, and engine ROUND, or engine
    // AUTO on the shapes where it takes the rounds
    {
        const bool streamed = d->head_dim == 128 && d->q_dtype == ART_BF16 && tile == 64 &&
                              (d->kv_dtype == ART_BF16 || d->kv_dtype == ART_I8 || d->kv_dtype == ART_I4);
        p.round_ok = eps_scale > 0.f && eps_dir > 0.f && streamed && p.G <= 8 && !(d->v_skip_eps > 0.f) &&
                     d->max_workers == 0 && d->team_helpers == 0 &&
                     (d->engine == ART_ENGINE_ROUND ||
                      (d->engine == ART_ENGINE_AUTO && art::round_auto(p.NG, p.G, p.nt_max)));
    }
    p.seq_div = d->per_head_tables ? (1 << p.kv_shift) : p.Hkv;
    {
        // multiply-high constants for grp / seq_div (round-up method): with
        // s = ceil(log2 seq_div), m = ceil(2^(31+s) / seq_div) < 2^32 and
        // m * seq_div - 2^(31+s) < seq_div <= 2^s, the error term stays below
        // 1 / seq_div for every grp < 2^31
        int sh = 0;
        while ((1LL << sh) < p.seq_div) ++sh;
        const unsigned long long num = 1ULL << (31 + sh);
        p.seq_m = (unsigned)((num + p.seq_div - 1) / p.seq_div);
        p.seq_sh = 31 + sh;
    }
    p.patience = d->patience;
    p.order = d->tile_order;
    p.tile_perm = d->tile_order == ART_ORDER_LIST ? d->tile_perm : nullptr;
    p.perm_stride = d->tile_order == ART_ORDER_LIST ? d->tile_perm_stride : 0;
    p.art = eps_scale > 0.f && eps_dir > 0.f;
    p.vskip = d->v_skip_eps > 0.f;
    p.eps_scale = eps_scale; p.eps_dir = eps_dir; p.v_skip_eps = d->v_skip_eps;
    p.v_skip_ln = p.vskip ? (float)std::log((double)d->v_skip_eps) : -INFINITY;
    p.inv_sqrt_d = 1.f / std::sqrt((float)d->head_dim);
    p.slot = art::kSlotHeader + p.G * d->head_dim;
    // full-mode split plan (part of the workspace layout, so independent of the device)
    const int target = kTargetWaves;
    int splits = p.NG ? (target + p.NG - 1) / p.NG : 1;
    // at least kMinTilesPerSplit tiles per split: a wave of one tile is all
    // latency, and each split adds a partial to the combine
    const int most = (p.nt_max + kMinTilesPerSplit - 1) / kMinTilesPerSplit;
    if (splits > most) splits = most;
    if (splits > p.nt_max) splits = p.nt_max > 0 ? p.nt_max : 1;
    if (splits < 1) splits = 1;
    p.tiles_per_split = p.nt_max > 0 ? (p.nt_max + splits - 1) / splits : 1;
    p.splits = p.nt_max > 0 ? (p.nt_max + p.tiles_per_split - 1) / p.tiles_per_split : 1;
    return ART_OK;
}

}  // namespace

namespace art {

Layout workspace_layout(const Params& p) {
    Layout L{};
    size_t o = 0;
    const size_t NG = (size_t)p.NG, G = (size_t)p.G;
    L.abort_flag = o; o = align256(o + sizeof(int));
    L.ctl = o; o = align256(o + NG * sizeof(GroupCtl));
    L.ring_tag = o; o = align256(o + NG * kRing * sizeof(int));
    L.ring = o; o = align256(o + NG * kRing * (size_t)p.slot * sizeof(float));
    L.vmax_tag = o; o = align256(o + NG * (size_t)p.nt_max * sizeof(int));
    L.vmax = o; o = align256(o + NG * (size_t)p.nt_max * 16 * sizeof(float));
    L.partials = o; o = align256(o + NG * (size_t)p.splits * p.slot * sizeof(float));
    const size_t NT = NG <= (size_t)kTeamHelpGroups ? NG : 0;  // groups that helpers may serve
    L.team_ring = o; o = align256(o + NT * group_words(p.G) * sizeof(unsigned long long));
    L.team_ctl = o; o = align256(o + NT * kTeamCtl * sizeof(unsigned long long));
    const size_t NS = p.order == ART_ORDER_LIST ? (size_t)(p.NG / p.seq_div) * p.nt_max : 0;  // step-table records
    L.steps = o; o = align256(o + NS * kStepW * sizeof(int));
    // round engine: every step's running state and probe record, the groups'
    // decision states and control words
    const RoundPlan rp = p.round_ok ? round_plan(p.nt_max, p.NG) : RoundPlan{};
    const size_t NR = rp.R > 0 ? NG : 0, HB = (G + 3) / 4;
    L.round_rec = o; o = align256(o + NR * (size_t)p.nt_max * p.slot * sizeof(float));
    L.round_probe = o; o = align256(o + NR * (size_t)p.nt_max * G * kRoundRecW * sizeof(float));
    L.round_state = o; o = align256(o + NR * HB * kRoundProbeW * 64 * sizeof(float));
    L.round_ctl = o; o = align256(o + NR * kRoundCtlW * sizeof(unsigned long long));
    L.total = o;
    return L;
}

art_status set_error(art_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

art_status call_workspace_bytes(const art_desc* desc, int tile, float eps_scale, float eps_dir, size_t* need) {
    g_last_error.clear();
    Params p;
    const art_status s = check(desc, tile, eps_scale, eps_dir, p);
    if (s != ART_OK) return s;
    *need = workspace_layout(p).total;
    return ART_OK;
}

}  // namespace art

extern "C" {

const char* art_status_string(int32_t s) {
    switch (s) {
        case ART_OK: return "ok";
        case ART_E_NULL: return "a required pointer is NULL";
        case ART_E_SHAPE: return "inconsistent or unsupported sizes";
        case ART_E_DTYPE: return "unsupported dtype";
        case ART_E_TILE: return "unsupported tile";
        case ART_E_PARAM: return "invalid method parameter";
        case ART_E_WORKSPACE: return "workspace missing, misaligned or too small";
        case ART_E_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* art_last_error(void) { return g_last_error.c_str(); }

int32_t art_abi_version(void) { return ART_ABI_VERSION; }

size_t art_workspace_bytes(const art_desc* desc, int32_t tile) {
    // the layout of full attention and that of ART mode (which may split a
    // KV head's query heads into several groups): enough for either
    art::Params full, art_mode;
    if (check(desc, tile, 0.f, 0.f, full) != ART_OK) return 0;
    if (check(desc, tile, 1.f, 1.f, art_mode) != ART_OK) return 0;
    const size_t a = art::workspace_layout(full).total, b = art::workspace_layout(art_mode).total;
    return a > b ? a : b;
}

art_status art_validate(const art_desc* desc, int32_t tile, float eps_scale, float eps_dir) {
    g_last_error.clear();
    art::Params p;
    art_status s = check(desc, tile, eps_scale, eps_dir, p);
    if (s != ART_OK) return s;
    const size_t need = art::workspace_layout(p).total;
    if (!desc->workspace) return fail(ART_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (reinterpret_cast<uintptr_t>(desc->workspace) & 255)
        return fail(ART_E_WORKSPACE, "workspace not 256-byte aligned");
    if (desc->workspace_bytes < need)
        return fail(ART_E_WORKSPACE, "workspace %zu bytes < %zu needed", desc->workspace_bytes, need);
    return ART_OK;
}

art_status art_decode_attention(const art_desc* desc, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table,
                                const int32_t* ctx_lens, int32_t tile, float eps_scale,
                                float eps_dir, float* out, int32_t* tiles_used, void* stream) {
    art_status s = art_validate(desc, tile, eps_scale, eps_dir);
    if (s != ART_OK) return s;
    art::Params p;
    check(desc, tile, eps_scale, eps_dir, p);
    if (p.B == 0) return ART_OK;
    if (!q || !k_cache || !v_cache || !ctx_lens || !out || !tiles_used)
        return fail(ART_E_NULL, "q, k_cache, v_cache, ctx_lens, out and tiles_used are required");
    if (p.block_size && !block_table) return fail(ART_E_NULL, "paged cache needs block_table");
    p.q = q; p.k = k_cache; p.v = v_cache;
    p.ks = static_cast<const uint16_t*>(desc->k_scale);
    p.vs = static_cast<const uint16_t*>(desc->v_scale);
    p.block_table = block_table; p.ctx_lens = ctx_lens; p.out = out; p.tiles_used = tiles_used;
    p.stats = reinterpret_cast<long long*>(desc->stats);
    // persistent grid (ART mode): one decider wave per group, up to
    // kMaxDeciders, and the requested number of tile workers (0: as many as
    // are resident alongside the deciders, settled at launch)
    p.deciders = p.NG < art::kMaxDeciders ? p.NG : art::kMaxDeciders;
    long long workers = desc->max_workers;
    const long long tiles = (long long)p.NG * p.nt_max;
    if (workers > tiles) workers = tiles > 0 ? tiles : 1;
    // more than kMaxWorkersPerGroup per group only adds waves that poll for
    // claims and slow the deciders (on 32 groups of 2048 tiles: 5 ms with 8
    // per group, 281 ms with 32)
    if (workers > (long long)art::kMaxWorkersPerGroup * p.NG) workers = (long long)art::kMaxWorkersPerGroup * p.NG;
    p.workers = (int)workers;
    p.helpers = desc->team_helpers;
    p.engine = desc->engine;
    p.xp_wpc_req = desc->workers_per_cu;
    p.xp_window_req = desc->window;
    const art::Layout L = art::workspace_layout(p);
    char* ws = static_cast<char*>(desc->workspace);
    p.abort_flag = reinterpret_cast<int*>(ws + L.abort_flag);
    p.ctl = reinterpret_cast<art::GroupCtl*>(ws + L.ctl);
    p.ring_tag = reinterpret_cast<int*>(ws + L.ring_tag);
    p.ring = reinterpret_cast<float*>(ws + L.ring);
    p.vmax_tag = reinterpret_cast<int*>(ws + L.vmax_tag);
    p.vmax = reinterpret_cast<float*>(ws + L.vmax);
    p.partials = reinterpret_cast<float*>(ws + L.partials);
    p.team_ring = reinterpret_cast<unsigned long long*>(ws + L.team_ring);
    p.team_ctl = reinterpret_cast<unsigned long long*>(ws + L.team_ctl);
    p.steps = reinterpret_cast<int*>(ws + L.steps);
    const bool rounds = p.round_ok && L.round_ctl < L.total;
    p.round_rec = rounds ? reinterpret_cast<float*>(ws + L.round_rec) : nullptr;
    p.round_probe = rounds ? reinterpret_cast<float*>(ws + L.round_probe) : nullptr;
    p.round_state = rounds ? reinterpret_cast<float*>(ws + L.round_state) : nullptr;
    p.round_ctl = rounds ? reinterpret_cast<unsigned long long*>(ws + L.round_ctl) : nullptr;
    p.epoch = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    if (p.epoch == 0) p.epoch = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;  // 0 never stamps
    const int rc = (p.art || p.vskip) ? art::launch_art(p, stream) : art::launch_full(p, stream);
    if (rc != 0) return fail(ART_E_HIP, "kernel launch failed: %s", hipGetErrorString((hipError_t)rc));
    return ART_OK;
}

}  // extern "C"
