// Batch-1 decode with one kernel per layer, each XCD running one active expert
// (moe_decode_xcd.hip): host/device interface.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int XL_XCDS = 8;           // XCDs of the device, blocks go round-robin to them
constexpr int XL_BPX = 32;           // blocks per XCD (one per CU)
constexpr int XL_BLOCKS = XL_XCDS * XL_BPX;
constexpr int XL_WAVES = 8;          // waves per block
constexpr int XL_MAX_LAYERS = 64;    // layers per barrier-counter clear
constexpr int XL_LINE = 32;          // ints per barrier counter (one 128-byte line each)

// Workspace of the path (byte sizes for d_model D, d_ff F, E routed experts).
struct XlWs {
    size_t ypart0, ypart1, lg, hb, bar, total;
};
XlWs xl_ws(int D, int F, int E);

struct XlParams {
    int D, F, E, K;
    int first;             // 1: the layer's input is x0; 0: the previous layer's partials
    uint32_t spin;         // longest barrier wait, in ticks of the 100 MHz real-time counter
    size_t expert_bytes;
    const float *x0;       // [D] (first layer)
    const float *yin;      // [8][D] partial outputs of the previous layer (else)
    float *yout;           // [8][D] this layer's partial outputs
    float *y_prev;         // optional [D]: the previous layer's output (sum of yin), for traces
    const uint16_t *router;
    const float *bias;
    const uint8_t *experts;
    const float *tscale;
    int32_t *idx_out;      // optional [K]
    float *w_out;          // optional [K]
    float *lg;             // [8][E] logits, one row per XCD
    float *hb;             // [8][F] h of each XCD's expert (feature slice)
    int32_t *bar;          // this layer's 2 x 8 barrier counters (XL_LINE ints apart)
    int32_t *err;          // error word (the workspace's batch-1 error word): set when a barrier
                           // wait gave up or crossed an XCD
};

// Whether the path runs this shape on the current device: q4_1 or NVFP4,
// d_model 2048, d_ff 512, 256 routed experts, top-6, one shared expert, and a
// device of 256 compute units that holds the whole grid at once.
bool xl_supported(int fmt, int D, int F, int E, int S, int K);
// Zeroes the barrier counters of XL_MAX_LAYERS layers and (first) the error word.
hipError_t xl_clear_launch(int32_t *bar, int32_t *err, bool clear_err, hipStream_t st, hipEvent_t *ev);
// One layer.
hipError_t xl_layer_launch(const XlParams &p, int fmt, hipStream_t st, hipEvent_t *ev);
// y = sum of the 8 partial outputs in XCD order.
hipError_t xl_reduce_launch(const float *ypart, float *y, int D, hipStream_t st, hipEvent_t *ev);

}  // namespace moe
