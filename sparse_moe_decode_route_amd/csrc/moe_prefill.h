// Internal interface of the prefill path (permute, grouped GEMM, combine)
// and of the weight repack.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

struct PrefillArgs {
    int D, F, E, S, K, T, fmt, act;
    size_t expert_bytes;
    const void *x;
    const uint16_t *router;
    const float *bias;
    const uint8_t *experts;
    const float *tscale;
    float *y;
    int32_t *idx_out;
    float *w_out;
    void *ws;
};

size_t prefill_ws_bytes(int D, int F, int E, int S, int K, int T);
float *prefill_logits_buffer(void *ws, const moe_dims &d, int T);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st);
hipError_t launch_repack_q4_1(const uint8_t *canonical, uint8_t *packed, int n_experts, int D, int F, hipStream_t st);

}  // namespace moe
