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
