// Persistent batch-1 stack decode (moe_stack_persist.hip): host/device interface.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int PS_BLOCKS = 256;      // one block per CU
constexpr int PS_SLOT_WORDS = 16;   // 128-byte mailbox slot per block (8-byte words)
constexpr int PS_MAX_LAYERS = 64;   // layers per launch (their pointers travel as kernel arguments, 2 KB)
constexpr int PS_CTRL_WORDS = 64;   // ctrl[0]: abort flag (a wait gave up); rest reserved
// workspace bytes: three mailbox arrays (logits, h, y) and the control words
constexpr size_t PS_WS_BYTES = 3 * (size_t)PS_BLOCKS * PS_SLOT_WORDS * 8 + PS_CTRL_WORDS * 4;

struct PsLayer {
    const uint16_t *router;  // bf16 [E, D]
    const float *bias;       // [E] or nullptr
    const uint8_t *experts;  // device layout, E routed then the shared expert
    const float *tscale;     // NVFP4 tensor scales or nullptr
};

struct PsParams {
    int D, F, E, K;
    int l0;            // global index of the launch's first layer
    int n_layers;      // layers in this launch (<= PS_MAX_LAYERS)
    int last_layer;    // global index of the stack's last layer (its y goes to y)
    int spin;          // polls per wait before a wave gives up
    size_t expert_bytes;
    const float *x0;   // input of layer 0 [D]
    float *y;          // output of the last layer [D], or nullptr
    float *y_trace;    // [layers, D] or nullptr
    int32_t *idx_trace;  // [layers, K] or nullptr
    float *w_trace;      // [layers, K] or nullptr
    unsigned long long *mb_lg, *mb_h, *mb_y;  // mailboxes [PS_BLOCKS][PS_SLOT_WORDS], contiguous in this order
    uint32_t *ctrl;
    PsLayer layer[PS_MAX_LAYERS];
};

// Whether the persistent kernel is built for this shape (and fits one block
// per CU on the current device): shared experts 1, top_k <= 6, n_routed <= 256,
// q4_1 or NVFP4 at d_model 2048, d_ff 512.
bool ps_supported(int fmt, int D, int F, int E, int S, int K);
// Clears the mailboxes and control words (before every call); ev (optional) = start/stop pair.
hipError_t ps_clear_launch(const PsParams &p, hipStream_t st, hipEvent_t *ev);
// One launch of up to PS_MAX_LAYERS layers; ev (optional) = start/stop pair.
hipError_t ps_launch(const PsParams &p, int fmt, hipStream_t st, hipEvent_t *ev);

}  // namespace moe
