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
    float *logits_out;        // optional [T, E]
    const int32_t *given_idx; // caller routing [T, K] (router skipped), or nullptr
    const float *given_w;
    int route_only;           // stop after routing (idx_out / w_out / logits_out)
    void *ws;
    hipEvent_t *ev;           // optional start/stop pairs per kernel slot (PREFILL_SLOTS)
};

// Kernel slots of the prefill path, in launch order (timing entry point);
// names of the slots' kernels for tokens of type act (MOE_ACT_*).
constexpr int PREFILL_SLOTS = 7;
// Whether the 4-bit grouped GEMMs run fused in one dispatch (pf_ffn_q4) for
// this format and shape.
bool prefill_fused(int fmt, int D, int F);
// Names of the prefill kernel slots (';'-separated), as timed.
const char *prefill_names(int act, bool fused);

size_t prefill_ws_bytes(int D, int F, int E, int S, int K, int T);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st);
hipError_t launch_repack_q4_1(const uint8_t *canonical, uint8_t *packed, int n_experts, int D, int F, hipStream_t st);

}  // namespace moe
