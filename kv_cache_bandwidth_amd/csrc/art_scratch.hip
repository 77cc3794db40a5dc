// art_decode_attention_noalloc: the same call as art_decode_attention, for
// callers that cannot allocate device memory (code under stream capture,
// serving loops that forbid allocation), with the workspace taken from a
// fixed array that the library holds on every device it runs on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "art.h"
#include "art_internal.h"

namespace {

// The call's workspace on every device: control words, tile records and
// partial results of one call.  In host code `scratch` only stands in for the
// symbol; its device address comes from hipGetSymbolAddress.
static_assert(ART_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch holds whole 256-byte lines");
static __device__ __align__(256) unsigned char scratch[ART_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch`, per device, once looked up

// Device address of the current device's scratch (looked up on the first call
// on that device, with that device current), or nullptr with the error set.
void* scratch_on_current_device(art_status* st) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *st = art::set_error(ART_E_HIP, "no current device for the static scratch (%s)",
                             e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *st = art::set_error(ART_E_HIP, "hipGetSymbolAddress of the static scratch failed on device %d: %s", dev,
                                 hipGetErrorString(e));
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" art_status art_decode_attention_noalloc(const art_desc* desc, const void* q, const void* k_cache,
                                                   const void* v_cache, const int32_t* block_table,
                                                   const int32_t* ctx_lens, int32_t tile, float eps_scale,
                                                   float eps_dir, float* out, int32_t* tiles_used,
                                                   void* stream) {
    if (!desc) return art::set_error(ART_E_NULL, "desc is NULL");
    // size check first, on the host alone: a call too large for the scratch
    // is refused before the device is touched
    art_desc d = *desc;
    size_t need = 0;
    art_status v = art::call_workspace_bytes(&d, tile, eps_scale, eps_dir, &need);
    if (v != ART_OK) return v;
    if (need > (size_t)ART_NOALLOC_SCRATCH_BYTES && d.engine == ART_ENGINE_AUTO) {
        // the round engine keeps every step's records; where they do not fit,
        // the team engine (no such records) serves the call
        d.engine = ART_ENGINE_TEAM;
        v = art::call_workspace_bytes(&d, tile, eps_scale, eps_dir, &need);
        if (v != ART_OK) return v;
    }
    if (need > (size_t)ART_NOALLOC_SCRATCH_BYTES)
        return art::set_error(ART_E_WORKSPACE,
                              "the call needs %zu bytes of workspace; the static scratch holds %zu "
                              "(pass a workspace to art_decode_attention instead)",
                              need, (size_t)ART_NOALLOC_SCRATCH_BYTES);
    art_status st = ART_OK;
    void* ws = scratch_on_current_device(&st);
    if (!ws) return st;
    d.workspace = ws;
    d.workspace_bytes = ART_NOALLOC_SCRATCH_BYTES;
    return art_decode_attention(&d, q, k_cache, v_cache, block_table, ctx_lens, tile, eps_scale, eps_dir, out,
                                tiles_used, stream);
}
