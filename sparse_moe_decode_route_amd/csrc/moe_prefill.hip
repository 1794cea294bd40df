// Prefill path (placeholder until the grouped GEMM lands): reports
// unsupported so callers fail loudly.
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_prefill.h"

namespace moe {

size_t prefill_ws_bytes(int, int, int, int, int, int) { return 0; }
float *prefill_logits_buffer(void *ws, const moe_dims &, int) { return static_cast<float *>(ws); }
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_router_gemm(const void *, int, int, int, int, const uint16_t *, const float *, float *, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace moe
