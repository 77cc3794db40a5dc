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
constexpr int kTeamRingG = 32;    // global ring slots per group for the tiles of helper teams
constexpr int kTeamSlotLane = 10; // floats per lane per head block in a team slot: m, l, 8 dims
constexpr int kMaxHelpers = 3;    // helper work-groups per group at most (team engine)
constexpr unsigned long long kWaitTicks = 50000000ull;  // 0.5 s of the 100 MHz device clock:
                                                      // longest any wait may last before the kernel gives up
constexpr int kSlotHeader = 48;   // floats before the accumulator block of a partial:
                                  // [0,16) tile max per head, [16,32) tile sum per head,
                                  // [32] error flag (as int), [33] V rows kept (as int)

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
    // method
    int patience;
    int art;            // stop rule active
    int vskip;          // V-row skip active
    float eps_scale, eps_dir, v_skip_eps, inv_sqrt_d;
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
    float* team_ring;   // [NG][kTeamRingG][HB][kTeamSlotLane][64]: tiles of helper teams
    unsigned long long* team_tag;  // [NG][kTeamRingG]: (epoch << 32) | (tile + 1)
    unsigned long long* team_ctl;  // [NG][2]: (epoch << 32) | frontier, (epoch << 32) | bound
    unsigned epoch;     // distinct per call: stale team words of earlier calls never match
    int helpers;        // helper work-groups per group (team kernel)
    int slot;           // floats per partial: kSlotHeader + G*D
    // launch
    int deciders;       // decider waves of the persistent kernel (each owns whole groups)
    int workers;        // tile worker waves of the persistent kernel
    int splits;         // full mode: workers per group
    int tiles_per_split;
};

// Workspace layout for a Params (offsets in bytes, all 256-byte aligned).
struct Layout {
    size_t abort_flag, ctl, ring_tag, ring, vmax_tag, vmax, partials, team_ring, team_tag, team_ctl, total;
};
Layout workspace_layout(const Params& p);

// Kernel launches (art_kernels.hip); return a hipError_t value.
int launch_art(const Params& p, void* stream);
int launch_full(const Params& p, void* stream);

}  // namespace art
