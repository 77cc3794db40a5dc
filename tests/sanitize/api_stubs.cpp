// Host-only stand-ins for the kernel launches, so that the C ABI's host code
// (argument checks, workspace layout, pointer setup) can be built and run
// under AddressSanitizer and UndefinedBehaviorSanitizer on a CPU.  The
// launch stand-in checks that every workspace region the host code laid out
// lies inside the caller's workspace.
#include <cstdio>
#include <cstdlib>

#include <hip/hip_runtime_api.h>

#include "art_internal.h"

namespace {
int check_params(const art::Params& p) {
    const art::Layout L = art::workspace_layout(p);
    const char* base = reinterpret_cast<const char*>(p.abort_flag) - L.abort_flag;
    const char* ends[] = {reinterpret_cast<const char*>(p.ctl), reinterpret_cast<const char*>(p.ring_tag),
                          reinterpret_cast<const char*>(p.ring), reinterpret_cast<const char*>(p.vmax_tag),
                          reinterpret_cast<const char*>(p.vmax), reinterpret_cast<const char*>(p.partials),
                          reinterpret_cast<const char*>(p.team_ring), reinterpret_cast<const char*>(p.team_ctl),
                          reinterpret_cast<const char*>(p.steps)};
    for (const char* e : ends) {
        if (e < base || e > base + L.total) {
            std::fprintf(stderr, "workspace region outside the layout\n");
            std::abort();
        }
    }
    // the round engine's regions, when laid out: each inside the workspace
    // with the extent the kernels index (every step of every group)
    if (p.round_rec) {
        const art::RoundPlan rp = art::round_plan(p.nt_max, p.NG);
        const size_t NG = (size_t)p.NG, HB = (size_t)(p.G + 3) / 4;
        struct Region {
            const char* at;
            size_t bytes;
        } regions[] = {
            {reinterpret_cast<const char*>(p.round_rec), NG * p.nt_max * p.slot * sizeof(float)},
            {reinterpret_cast<const char*>(p.round_probe), NG * p.nt_max * p.G * art::kRoundRecW * sizeof(float)},
            {reinterpret_cast<const char*>(p.round_state), NG * HB * art::kRoundProbeW * 64 * sizeof(float)},
            {reinterpret_cast<const char*>(p.round_ctl), NG * art::kRoundCtlW * sizeof(unsigned long long)},
        };
        for (const Region& r : regions) {
            if (r.at < base || r.at + r.bytes > base + L.total) {
                std::fprintf(stderr, "round engine region outside the layout\n");
                std::abort();
            }
        }
        if (rp.R < 0 || rp.R > art::kMaxRounds || (p.nt_max > 0 && rp.R > 0 && rp.a[rp.R] != p.nt_max)) {
            std::fprintf(stderr, "inconsistent round plan\n");
            std::abort();
        }
        // the final launch's slices use the full-mode partial slots
        if (p.splits < 1) {
            std::fprintf(stderr, "no partial slots for the round engine's final launch\n");
            std::abort();
        }
    }
    if (p.NG < 0 || p.G < 1 || p.G > art::kMaxG || p.nt_max < 0) {
        std::fprintf(stderr, "inconsistent shape in Params\n");
        std::abort();
    }
    return 0;
}
}  // namespace

namespace art {
int launch_art(const Params& p, void*) { return check_params(p); }
int launch_full(const Params& p, void*) { return check_params(p); }
}  // namespace art

const char* hipGetErrorString(hipError_t) { return "stub"; }
