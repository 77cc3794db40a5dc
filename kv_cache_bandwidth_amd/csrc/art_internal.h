// Internal declarations shared by the host API (art_api.cpp) and the kernels
// (art_kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "art.h"

namespace art {

constexpr int kRing = 128;        // ring slots per group (tiles in flight ahead of the frontier)
constexpr int kMaxG = 16;         // query heads per KV head
constexpr int kWavesPerWG = 4;    // independent waves per work-group
constexpr int kMaxDeciders = 512; // decider waves at most (one per group up to this many groups)
constexpr int kMaxWorkersPerGroup = 8;  // work-sharing engine: tile workers per group at most
constexpr int kMaxSplitGroups = 1024;   // query-head split up to this many groups (still a gain at 2 per CU)
// team engine, words shared through the workspace (per group)
constexpr int kTeamRingG = 16;    // slots of the helpers' tile partials per group (a power of two)
constexpr int kTeamRecW = 11;     // 64-bit words per (tile, head) record: max, sum, probe dims 0..7, error flag
constexpr int kTeamRecHeads = 8;  // heads per record slot (streamed tiles serve up to 8 query heads per KV head)
constexpr int kTeamStateW = 10;   // values per lane per head block of a partial or running state: m, l, 8 dims
constexpr int kTeamPartW = 11;    // 64-bit words per lane per head block of a helper's tile partial: m, l, 8 dims, error flag
constexpr int kMaxHelpers = 3;    // helper work-groups per group at most
constexpr int kTeamCtl = 16;      // control words: [0] helper slots released, [1] bound, [2] tiles decided
constexpr int kTeamHelpGroups = 512;  // helpers and the pool engine serve launches of at most this many
                                      // groups (the workspace holds their shared words only then)
constexpr int kPoolRing = 128;    // pool engine: record slots per group, by tile index (a power of two)
constexpr int kPoolContrib = 32;  // pool engine: workers per group at most (each leaves its running state)
constexpr int kXpMaxWindow = 112; // XCD engine: the load window at most (records live in a ring of
                                  // kPoolRing slots, released a 16-tile block at a time)
constexpr int kPoolCtl = 16;      // pool engine control words: [0] tiles released, [1] bound, [2] claim counter,
                                  // [3] workers joined, [4..11] per-head decision, [12] workers active
constexpr unsigned long long kWaitTicks = 50000000ull;  // 0.5 s of the 100 MHz device clock:
                                                      // longest any wait may last before the kernel gives up
constexpr int kStepPages = 4;     // 16-token pages of a 64-token tile (entries of a step-table record)
constexpr int kStepW = 8;         // ints per step-table record: kStepPages block ids, the tile, padding
constexpr int kSlotHeader = 48;   // floats before the accumulator block of a partial:
                                  // [0,16) tile max per head, [16,32) tile sum per head,
                                  // [32] error flag (as int), [33] V rows kept (as int)

// Round engine (ART mode, streamed 64-token tiles): the visiting steps run in
// rounds, one launch each; round r takes steps [a[r], a[r+1]) of every group
// still undecided, spread over waves[r] waves per group of pw[r] consecutive
// steps each.  The first rounds take enough steps for about kRoundFirstPW
// steps per wave of a round over all groups (kRoundFirst to kRoundFirstMax),
// later ones as many steps as came before them (at most kRoundMaxSteps): a
// group that stops past the first round has loaded at most twice the steps
// it needs.  (On B8 x 8 KV heads at 32K context, int8, a first round of 96
// steps then doubling took ART 100-101 us and never-firing ART 269 us,
// against 110-111 and 262 us for 128 steps then half again, and 103 and
// 295 us for 96 then half again.)
constexpr int kRoundFirst = 64;          // steps of a round at least (multiple of 16)
constexpr int kRoundFirstMax = 256;      // steps of the first rounds at most (multiple of 16)
constexpr int kRoundFirstPW = 3;         // steps per wave the first rounds aim for
constexpr int kRoundMaxSteps = 512;      // steps of a round at most (multiple of 16)
constexpr int kMaxRounds = 32;           // rounds of a call at most (else the engine does not apply)
constexpr int kRoundWavesTarget = 2048;  // waves of a round over all groups (256 CUs x 8)
constexpr int kRoundMaxPW = 4;           // steps per wave at most
constexpr int kRoundRecW = 12;           // floats of a probe record per (step, head): max, sum,
                                         // accumulator dims 0..7, error flag (as int), padding
constexpr int kRoundProbeW = 22;         // words per lane per head block of a group's decision state
constexpr int kRoundCtlW = 2 + kMaxRounds;  // 64-bit words per group (zeroed by each call): [0] (epoch, next round) once a
                                            // round left heads undecided, [1 + r] arrivals in round r,
                                            // [1 + kMaxRounds] slices of the final launch done

struct RoundPlan {
    int R;                     // rounds (0: the engine does not apply)
    int a[kMaxRounds + 1];     // first step of each round; a[R] = steps of the longest row
    int pw[kMaxRounds];        // steps per wave
    int waves[kMaxRounds];     // waves per group
};

// The rounds of a call with NG groups and rows of at most nt_max tiles.
inline RoundPlan round_plan(int nt_max, int NG) {
    RoundPlan rp{};
    rp.R = 0;
    rp.a[0] = 0;
    long long first = NG > 0 ? ((long long)kRoundFirstPW * kRoundWavesTarget / NG + 15) / 16 * 16 : kRoundFirst;
    if (first < kRoundFirst) first = kRoundFirst;
    if (first > kRoundFirstMax) first = kRoundFirstMax;
    while (rp.a[rp.R] < nt_max) {
        if (rp.R == kMaxRounds) {
            rp.R = 0;
            return rp;
        }
        const int a = rp.a[rp.R];
        int c = (a + 15) / 16 * 16;
        if (c < (int)first) c = (int)first;
        if (c > kRoundMaxSteps) c = kRoundMaxSteps;
        const int b = a + c < nt_max ? a + c : nt_max;
        long long pw = (long long)(b - a) * NG / kRoundWavesTarget;
        if (pw < 1) pw = 1;
        if (pw > kRoundMaxPW) pw = kRoundMaxPW;
        rp.pw[rp.R] = (int)pw;
        rp.waves[rp.R] = (b - a + (int)pw - 1) / (int)pw;
        rp.a[++rp.R] = b;
    }
    return rp;
}

// Engine AUTO takes the rounds for ART without the V skip where they were
// measured faster than one CU per group: few groups (the team engine would
// leave most CUs idle) of 256 to 1024 tiles and at most 4 query heads (on
// B8 x 8 KV heads at 32K context, int8: 100-101 us against 122 us on the
// team engine; with 128 groups, or rows of 2048 tiles, the team and pool
// engines are faster).  Shapes only, so that the workspace layout can follow.
constexpr int kRoundAutoGroups = 64;  // groups at most
inline bool round_auto(int NG, int G, int nt_max) {
    return NG <= kRoundAutoGroups && G <= 4 && nt_max >= 256 && nt_max <= 1024;
}

// Per-group control block; the allocation counter on its own 128-byte line.
struct alignas(128) GroupCtl {
    int next;          // tile allocation counter (atomic)
    int pad0[31];
    int frontier;      // tiles folded into the group's running state (written by its decider)
    int bound;         // tiles that may still be allocated: ceil(n/T), lowered once every head stopped
    int nt;            // tiles of the group
    int n;             // ctx_len of the row
    int pad1[28];
};

struct Params {
    // shape
    int B, Hq, Hkv, G, D, T;
    int q_dtype, kv_dtype;
    int block_size, mbps, num_blocks, max_ctx;
    int cap;            // tokens a row can hold
    int nt_max;         // ceil(cap / T)
    int NG;             // B * Hkv groups
    int hkv_cache;      // KV heads of the cache; Hkv = hkv_cache << kv_shift groups per row
    int kv_shift;       // a KV head's query heads run as 1 << kv_shift groups of G heads each
    int gq;             // query heads per KV head (the last group of a KV head may hold fewer than G)
    int seq_div;        // group grp reads sequence grp / seq_div: Hkv (one per row), or 1 (per-head tables)
    unsigned seq_m;     // grp / seq_div == (grp * seq_m) >> seq_sh for 0 <= grp < 2^31
    int seq_sh;
    // method
    int patience;
    int order;          // art_order: tile i of a row's visiting sequence is tile_at(i)
    const int* tile_perm;  // ART_ORDER_LIST: [B][perm_stride]
    int perm_stride;
    int art;            // stop rule active
    int vskip;          // V-row skip active
    float eps_scale, eps_dir, v_skip_eps, inv_sqrt_d;
    float v_skip_ln;    // ln(v_skip_eps) (-inf without the V skip): exp(x) >= eps  <=>  x >= ln eps
    // inputs / outputs (device)
    const void* q;
    const void* k;
    const void* v;
    const uint16_t* ks;
    const uint16_t* vs;
    const int* block_table;
    const int* ctx_lens;
    float* out;
    int* tiles_used;
    long long* stats;
    // workspace regions (device)
    int* abort_flag;    // set when a wait outlasted kWaitTicks: workers exit, heads stay unfinished
    GroupCtl* ctl;
    int* ring_tag;      // [NG][kRing]
    float* ring;        // [NG][kRing][slot]
    int* vmax_tag;      // [NG][nt_max]
    float* vmax;        // [NG][nt_max][16]
    float* partials;    // [NG][splits][slot]
    unsigned long long* team_ring;  // [NG][group_words(G)]: team engine: the helpers' tile partials
                                    // [kTeamRingG][HB][kTeamPartW][64]; pool engine: records
                                    // [kPoolRing][kTeamRecW][kTeamRecHeads], then worker states
                                    // [kPoolContrib][HB][kTeamStateW][64]; (tag << 32) | value bits
    unsigned long long* team_ctl;   // [NG][kTeamCtl]: (epoch << 32) | value
    int* steps;         // ART_ORDER_LIST: [sequences][nt_max][kStepW] step table (see art_steps_kernel)
    unsigned epoch;     // distinct per call: stale team words of earlier calls never match
    int helpers;        // helper work-groups per group (team kernel)
    int pool_cap;       // pool kernel: workers that may join one group (<= kPoolContrib)
    int engine;         // art_engine requested
    int xp_wpc_req;     // XCD engine: worker waves per CU requested (0 = default)
    int xp_window_req;  // XCD engine: load window requested (0 = default)
    int xp_dec_wgs;     // XCD engine: decider work-groups per XCD (set at launch)
    int xp_wpc;         // XCD engine: worker waves per CU (set at launch)
    int xp_window;      // XCD engine: tiles past the decided frontier a worker may load
    int slot;           // floats per partial: kSlotHeader + G*D
    int round_ok;       // the workspace holds the round engine's regions (set from the call's desc)
    float* round_rec;   // [NG][nt_max][slot]: a wave's running state through each of its steps
    float* round_probe; // [NG][nt_max][G][kRoundRecW]: each step's own probe record
    float* round_state; // [NG][HB][kRoundProbeW][64]: a group's decision state between rounds
    unsigned long long* round_ctl;  // [NG][kRoundCtlW]
    // launch
    int deciders;       // decider waves of the persistent kernel (each owns whole groups)
    int workers;        // tile worker waves of the persistent kernel
    int splits;         // full mode: workers per group
    int tiles_per_split;
};

// 64-bit words per group: the team engine's helper tile partials, or the
// pool engine's records and worker states
constexpr size_t team_words(int G) { return (size_t)kTeamRingG * ((G + 3) / 4) * kTeamPartW * 64; }
constexpr size_t pool_words(int G) {
    return (size_t)kPoolRing * kTeamRecW * kTeamRecHeads + (size_t)kPoolContrib * ((G + 3) / 4) * kTeamStateW * 64;
}
constexpr size_t group_words(int G) { return team_words(G) > pool_words(G) ? team_words(G) : pool_words(G); }

// Workspace layout for a Params (offsets in bytes, all 256-byte aligned).
struct Layout {
    size_t abort_flag, ctl, ring_tag, ring, vmax_tag, vmax, partials, team_ring, team_ctl, steps;
    size_t round_rec, round_probe, round_state, round_ctl;  // round engine (0 bytes unless round_ok)
    size_t total;
};
Layout workspace_layout(const Params& p);

// Host side (art_api.cpp): records a printf-style detail for art_last_error()
// and returns s.
art_status set_error(art_status s, const char* fmt, ...);
// Validates a call's desc, tile and thresholds like art_validate (workspace
// aside) and stores the workspace bytes that exact call needs in *need.
art_status call_workspace_bytes(const art_desc* desc, int tile, float eps_scale, float eps_dir, size_t* need);

// Kernel launches (art_kernels.hip); return a hipError_t value.
int launch_art(const Params& p, void* stream);
int launch_full(const Params& p, void* stream);

}  // namespace art
