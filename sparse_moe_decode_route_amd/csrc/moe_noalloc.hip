// moe_layer_forward_noalloc: moe_layer_forward with its workspace in a
// file-scope device array instead of a caller buffer, for callers that
// cannot allocate device memory (code under stream capture, serving loops,
// harnesses that forbid hipMalloc).  The kernels and results are those of
// moe_layer_forward; only where the workspace lives differs.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "moe_internal.h"

// One copy per device, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol): it uses the device address looked up per device below.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch`, looked up once per
// device with that device current (the caller's current device, which its
// stream belongs to).
moe_status scratch_ptr(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return moe::set_error(MOE_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return moe::set_error(MOE_ERR_UNSUPPORTED, "device ordinal " + std::to_string(dev) +
                                                       " beyond the library's table of " + std::to_string(kMaxDevices));
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return moe::set_error(MOE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward_noalloc(const moe_dims *dims, const moe_layer_weights *w, const void *x, int32_t act,
                                     int32_t n_tokens, float *y, int32_t *topk_idx_out, float *topk_w_out,
                                     void *stream) {
    size_t need = 0;
    moe_status s = moe_workspace_size(dims, n_tokens, &need);
    if (s != MOE_OK) return s;  // moe_last_error() holds the reason
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return moe::set_error(MOE_ERR_WORKSPACE, "moe_layer_forward_noalloc: this call needs a " + std::to_string(need) +
                                                     "-byte workspace; the static scratch holds " +
                                                     std::to_string(MOE_NOALLOC_SCRATCH_BYTES) + " bytes");
    void *ws = nullptr;
    s = scratch_ptr(&ws);
    if (s != MOE_OK) return s;
    return moe_layer_forward(dims, w, x, act, n_tokens, y, topk_idx_out, topk_w_out, ws,
                             (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
