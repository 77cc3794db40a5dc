/*
 * art.h -- C ABI of the ART decode-attention library for MI355X (gfx950).
 *
 * One decode query per (batch row, query head) attends over that row's KV
 * cache tile by tile with an online softmax, and the traversal stops early
 * once a cheap probe of the running output has stabilised (ART, "Runtime
 * Attention Termination", gist.science technical summary of arXiv
 * 2606.00024, sections 2.1-2.4).  An optional mode leaves out of P.V the V
 * rows whose softmax weight is negligible (puntofijo.es article on skipping
 * V dequantisation in llama.cpp); with bf16 caches on the streamed 64-token
 * tiles (head_dim 128, bf16 queries) a row that no query head of its KV head
 * keeps is not loaded at all.
 *
 * Every pointer passed to art_decode_attention is device memory allocated and
 * owned by the caller; the library keeps none of them after the call returns,
 * allocates nothing and never synchronises.  Work is enqueued on `stream`
 * (a hipStream_t, or NULL for the default stream); results are valid once the
 * stream has reached that point.  Errors are returned as negative status
 * codes, never thrown, printed or aborted on; art_last_error() gives detail.
 */
#ifndef ART_H
#define ART_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ART_ABI_VERSION 9

typedef enum {
    ART_OK = 0,
    ART_E_NULL = -1,        /* a required pointer is NULL                          */
    ART_E_SHAPE = -2,       /* sizes inconsistent or out of the supported range    */
    ART_E_DTYPE = -3,       /* unknown dtype or unsupported q/kv dtype pair        */
    ART_E_TILE = -4,        /* tile not in {16, 32, 64, 128} or not a multiple of
                               the page granule                                    */
    ART_E_PARAM = -5,       /* threshold NaN/negative/infinite, patience < 1, ... */
    ART_E_WORKSPACE = -6,   /* workspace NULL, misaligned or smaller than needed   */
    ART_E_HIP = -7          /* a HIP runtime call (launch) failed                  */
} art_status;

/* ART_I4: signed 4-bit codes, two per byte -- element 2i in the low nibble of
 * byte i, element 2i + 1 in the high nibble -- with the same per-(token, KV
 * head) fp16 scale as ART_I8; a cache row is head_dim / 2 bytes.  This
 * library's own lower-bit format (the pages name quantised caches without
 * specifying their codecs). */
typedef enum { ART_F32 = 0, ART_BF16 = 1, ART_I8 = 2, ART_I4 = 3 } art_dtype;

/* How ART-mode work is spread over the GPU (results agree to rounding; tiles_used
 * is the same whichever runs).  The choice applies to bf16, int8 and int4
 * caches with head_dim 128, bf16 queries and 64-token tiles, at most 8 query
 * heads per KV head (ART mode runs 10 to 16 as groups of at most 4, each
 * reading the KV head's tiles); other shapes always run the work-sharing
 * engine. */
typedef enum {
    ART_ENGINE_AUTO = 0,    /* library default                                         */
    ART_ENGINE_TEAM = 1,    /* one work-group per (row, KV head), plus team_helpers    */
    ART_ENGINE_POOL = 2,    /* waves on every CU move to the groups with work left; no
                               V skip (falls back to TEAM) and at most one group per
                               resident work-group                                     */
    ART_ENGINE_SHARED = 3,  /* work-sharing engine: max_workers waves claim tiles      */
    ART_ENGINE_XCD = 4,     /* one work-group per CU; every (row, KV head) group served
                               by waves of one XCD (chiplet), which move to the groups
                               of that XCD with work left; deciders on CUs that load
                               no tiles; no V skip (falls back to TEAM); at most 512
                               groups                                                  */
    ART_ENGINE_PAIR = 5,    /* two CUs per group on one XCD: one loads K and computes
                               the scores, the other loads V, folds and decides; at
                               most 4 query heads per group, no V skip, the number
                               of groups a multiple of 8 and at most half the CUs
                               (else TEAM)                                             */
    ART_ENGINE_ROUND = 6    /* the steps run in rounds over every CU (one launch per
                               round): round r loads steps [a_r, a_{r+1}) of every
                               group with heads left undecided, all at once, and the
                               last wave of each group decides them; the first
                               round takes 6144 / groups steps (rounded up to 16,
                               within 64..256), each later one as many steps as
                               came before it, at least the first's and at most
                               512.
                               No V skip (falls back to TEAM).  Its
                               workspace keeps every step's running state and probe
                               record (art_workspace_bytes counts them for engine
                               ROUND, and for AUTO on the shapes where AUTO takes
                               it: at most 64 groups of 256-1024 tiles, at most 4
                               query heads per group)                                  */
} art_engine;

/* Order in which a row's tiles are visited (ART summary, section 2.4: the tile
 * sequence may be reordered, e.g. recency- or importance-first, without
 * approximation error; block 0, the attention sink, is evaluated first).  The
 * probe sequence, the patience streak, tiles_used and the V-skip running max
 * follow the visiting steps; every order visits tile 0 first. */
typedef enum {
    ART_ORDER_ASCENDING = 0,  /* tiles 0, 1, ..., n_t - 1                                */
    ART_ORDER_RECENT = 1,     /* tile 0, then the most recent first: n_t - 1, n_t - 2, ..., 1 */
    ART_ORDER_LIST = 2        /* the caller's tile_perm: row b's step s visits tile
                                 tile_perm[b][s]; step 0 must name tile 0 and steps
                                 1..n_t-1 tiles in 1..n_t-1 (a permutation of them;
                                 repeats are not detected)                          */
} art_order;

/*
 * Shape and options of one call.  Layouts are row-major:
 *   q           [batch][num_q_heads][head_dim]           q_dtype (F32 or BF16)
 *   k/v cache   paged:      [num_blocks][num_kv_heads][block_size][head_dim]
 *               contiguous: [batch][num_kv_heads][max_ctx][head_dim]
 *               kv_dtype F32, BF16, I8 or I4 (then k_scale/v_scale are required;
 *               I4 rows hold head_dim / 2 bytes)
 *   k/v scale   fp16 bit patterns, the cache layout without head_dim: one scale
 *               per (token, KV head); the value of an I8 or I4 entry is code * scale
 *   block_table int32 [batch][max_blocks_per_seq] (paged only): logical page p
 *               of row b lives in physical block block_table[b][p]
 *   ctx_lens    int32 [batch]: cached positions of each row (0 allowed)
 *   with per_head_tables = 1 every (row b, KV head g) is a sequence of its own:
 *               ctx_lens [batch][num_kv_heads], block_table
 *               [batch][num_kv_heads][max_blocks_per_seq] (KV head g reads its
 *               slice of the blocks its row lists) and tile_perm
 *               [batch][num_kv_heads][tile_perm_stride]
 *   out         fp32 [batch][num_q_heads][head_dim]
 *   tiles_used  int32 [batch][num_q_heads]
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
typedef struct {
    int32_t batch;               /* >= 0                                              */
    int32_t num_q_heads;         /* >= 1, multiple of num_kv_heads, at most 16 per KV head */
    int32_t num_kv_heads;        /* >= 1                                              */
    int32_t head_dim;            /* 64 or 128                                         */
    int32_t q_dtype;             /* art_dtype: ART_F32 or ART_BF16                    */
    int32_t kv_dtype;            /* art_dtype                                         */
    int32_t block_size;          /* 0 = contiguous cache; else a multiple of 16       */
    int32_t max_blocks_per_seq;  /* paged: row stride of block_table                  */
    int32_t num_blocks;          /* paged: valid block ids are 0..num_blocks-1        */
    int32_t max_ctx;             /* contiguous: row stride in tokens (multiple of 16) */
    int32_t patience;            /* >= 1: consecutive passing tiles needed to stop    */
    float v_skip_eps;            /* 0 = off; else skip V row j when exp(s_j - M_t) <
                                    v_skip_eps, M_t the running max through tile t
                                    (its weight still enters the softmax sum).  bf16
                                    caches, streamed 64-token tiles: rows no head of
                                    the KV head keeps are not loaded.  int8/int4
                                    caches, streamed 64-token tiles: the rows come
                                    with K and a skipped row's weight is zero (the
                                    matrix-core P.V still runs over every row: the
                                    faster arrangement at eps 1e-6).  Other tiles:
                                    only the kept rows are loaded, dequantised and
                                    accumulated                                     */
    const void* k_scale;         /* I8 caches only (device, fp16 bits)                */
    const void* v_scale;
    void* workspace;             /* device scratch, 256-byte aligned, caller-owned    */
    size_t workspace_bytes;      /* >= art_workspace_bytes(desc, tile)                */
    int64_t* stats;              /* optional device int64[4] accumulator, or NULL:
                                    [0] K tiles loaded (in ART mode a KV head's 5-16
                                    query heads may run as several groups of at most
                                    4, each loading the tiles it needs), [1] V rows
                                    loaded (under the V skip on bf16 streamed tiles,
                                    only the rows some head keeps),
                                    [2] reserved (left unchanged; the tiles loaded
                                        past a group's stop are [0] minus the
                                        tiles its heads' tiles_used name),
                                    [3] (query head, position) pairs whose V row was
                                        skipped (v_skip_eps > 0; counted by the
                                        default engine for 64-token tiles only)       */
    int32_t max_workers;         /* 0 = library default; > 0 (engine AUTO or SHARED):
                                    the work-sharing engine with this many waves (at
                                    most 8 per (row, KV head) group are used, and no
                                    more than fit on the device beside its deciders:
                                    the launch is cooperative, every wave resident) */
    int32_t team_helpers;        /* team engine (ART, streamed tiles): helper work-groups
                                    per group on other CUs, 0..3; 0 = none (default).
                                    Used only where every work-group of the launch can
                                    be resident at once; results do not depend on it  */
    int32_t engine;              /* art_engine; ART_ENGINE_AUTO = 0                    */
    int32_t tile_order;          /* art_order; ART_ORDER_ASCENDING = 0                 */
    int32_t tile_perm_stride;    /* ART_ORDER_LIST: row stride of tile_perm, at least
                                    ceil(row capacity / tile)                         */
    const int32_t* tile_perm;    /* ART_ORDER_LIST: device int32 [batch][tile_perm_stride],
                                    caller-owned, read only; else ignored            */
    int32_t per_head_tables;     /* 0: lengths, block tables and tile lists per row;
                                    1: per (row, KV head) -- the positions a per-head
                                    retention or eviction policy kept, in order (ART
                                    summary, section 2.4: ART runs unchanged on top) */
    int32_t workers_per_cu;      /* XCD engine: tile-loading waves per CU, 0 = library
                                    default; capped by what fits in a CU's LDS       */
    int32_t window;              /* XCD engine: a tile is loaded only while it lies less
                                    than this many tiles past the decided frontier
                                    (bounds the tiles loaded past a stop); 0 = library
                                    default; at most 112                             */
} art_desc;

/*
 * art_decode_attention -- ART-terminated decode attention over a KV cache.
 *
 * For every (b, h): the query attends over positions 0..ctx_lens[b]-1 (per-head
 * tables: ctx_lens[b][g]) of its
 * KV head in tiles of `tile` tokens, tile 0 first and then in desc->tile_order,
 * with an online softmax (ART summary, section 2.1).  After each visiting step
 * t the probe is dims 0..7 of the
 * normalised running output; from t = 1 on, d_scale = | |x_t| - |x_{t-1}| | /
 * |x_{t-1}| and d_dir = 1 - cos(x_t, x_{t-1}) (section 2.2).  A tile passes
 * when d_scale < eps_scale and d_dir < eps_dir; after `patience` consecutive
 * passing tiles (section 2.3) the head stops, tiles_used[b][h] = t + 1 and the
 * remaining tiles of that head are never read.  Tile 0 is always evaluated
 * (section 2.4).  Without a stop, tiles_used = ceil(ctx_len / tile).
 * out[b][h] = softmax(q k^T / sqrt(head_dim)) v over the used positions.
 *
 * eps_scale = eps_dir = 0 (or any threshold <= 0) never stops: full attention,
 * run by a kernel without the detector when v_skip_eps is 0.
 * ctx_lens[b] = 0 gives out = 0 and tiles_used = 0.
 *
 * Errors detected on the device, per batch row: ctx_lens[b] < 0 or larger than
 * the cache row capacity, a block id outside [0, num_blocks) inside a
 * visited tile, or a tile_perm entry at a visited step that breaks the rules
 * of ART_ORDER_LIST -> tiles_used = -1 and out = NaN for the affected heads; no
 * out-of-range address is ever dereferenced.  Should a wait between the
 * cooperating waves of a call outlast half a second (the GPU was shared with
 * a starving workload), the heads not yet decided report tiles_used = -2 and
 * out = NaN instead of hanging.
 *
 * Host-side validation happens before anything is enqueued; device memory is
 * never read on the host.  Concurrent calls must use distinct workspaces.
 */
art_status art_decode_attention(const art_desc* desc, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table,
                                const int32_t* ctx_lens, int32_t tile, float eps_scale,
                                float eps_dir, float* out, int32_t* tiles_used, void* stream);

/*
 * art_decode_attention_noalloc -- art_decode_attention for callers that cannot
 * allocate device memory (code under stream capture, serving loops or
 * harnesses that forbid hipMalloc).  Same arguments, results and errors;
 * desc->workspace and desc->workspace_bytes are ignored: the workspace is a
 * fixed array of ART_NOALLOC_SCRATCH_BYTES that the library holds on each
 * device it runs on (from the first call there until the process ends).  The
 * call runs on the current device; `stream` must belong to it.  It allocates
 * nothing and calls no allocating routine.
 *
 * A call whose workspace (art_workspace_bytes for that desc, tile and mode)
 * exceeds ART_NOALLOC_SCRATCH_BYTES returns ART_E_WORKSPACE before anything is
 * touched on the device.  Nothing in the array needs to start at zero: each
 * call initialises the words it reads and stamps the words shared between
 * its waves with a per-call epoch.  Every call on one device shares that
 * device's array, so calls that may run at the same time on one device (on
 * different streams, or from several threads) race and give wrong results:
 * order them on one stream, or use art_decode_attention with a workspace each.
 */
#define ART_NOALLOC_SCRATCH_BYTES (96u << 20)

art_status art_decode_attention_noalloc(const art_desc* desc, const void* q, const void* k_cache,
                                        const void* v_cache, const int32_t* block_table,
                                        const int32_t* ctx_lens, int32_t tile, float eps_scale,
                                        float eps_dir, float* out, int32_t* tiles_used, void* stream);

/* Bytes of workspace a call with this desc and tile needs (0 on an invalid desc). */
size_t art_workspace_bytes(const art_desc* desc, int32_t tile);

/* Host-only validation of everything art_decode_attention checks before
 * launching (pointers in desc are not dereferenced; q/k/v/out pointers are
 * not examined here). */
art_status art_validate(const art_desc* desc, int32_t tile, float eps_scale, float eps_dir);

/* Static description of a status code. */
const char* art_status_string(int32_t status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* art_last_error(void);

/* ART_ABI_VERSION of the loaded library. */
int32_t art_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ART_H */
