// Internal host/device interface of libmoe (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/moe.h"

namespace moe {

// Records msg for moe_last_error() on the calling thread and returns s.
moe_status set_error(moe_status s, const std::string &msg);

constexpr int MAX_DECODE_T = 8;   // batch-1, general and stack decode paths
constexpr int MAX_BN_T = 32;      // small-batch path (regular shapes; the grouped GEMM is faster past 32 tokens)

// Everything a decode-path kernel reads or writes (device pointers).
struct DecodeParams {
    int D, F, E, S, K, T, fmt;
    int amax;            // slots in the active-expert list (shared + routed union bound)
    int route_given;     // 1: idx/w come from the caller (no router, no top-k)
    int want_router;     // phase A computes router logits
    int want_shared;     // phase A computes shared experts' h
    size_t expert_bytes;
    const float *x;      // [T, D] fp32 input, or nullptr when x_prev is used
    const float *x_prev; // previous layer output to RMS-normalise (stacks), or nullptr
    float *xbuf;         // normalised input [T, D] written by phase A when x_prev is set
    const uint16_t *router;
    const float *bias;
    const uint8_t *experts;
    const float *tscale;
    float *logits;       // [T, E]
    int32_t *idx;        // [T, K]
    float *w;            // [T, K]
    int32_t *idx_out;    // optional copies for the caller
    float *w_out;
    int32_t *meta;       // meta[0] = number of active slots
    int32_t *act_expert; // [amax]
    uint32_t *act_mask;  // [amax] token bitmask
    float *act_w;        // [amax, T] combine weight of each token (0 if absent)
    float *h;            // [amax, T, F]
    float *y;            // [T, D]
    // weights of the next layer (stacks), touched during this layer's down
    // projection so that they are on chip when the next layer starts
    const uint8_t *next_router;
    size_t next_router_bytes;
    const uint8_t *next_shared;
    size_t next_shared_bytes;
    int32_t sink_flag;   // always 0: keeps prefetch loads alive
    // optional kernel timing: start/stop event pairs, pair s for the layer's
    // kernel slot s; the kernel is then launched with hipExtLaunchKernelGGL,
    // whose events take the dispatch's own begin and end timestamps
    hipEvent_t *ev;
    int32_t *work;       // small-batch path: gate/up items {slot, token a, token b, expert}
    int32_t *pairs;      // small-batch path: down pairs {slot, token, coef bits, expert}
    int32_t *b1_list;    // batch-1 path: 8 copies (one per XCD) of {expert[8], coef bits[8]}
    int b1_ncopy;        // copies written (gate/up blocks 0 .. b1_ncopy - 1)
};

// Launch `kern(p)` on `st`, timed into event pair `slot` when p.ev is set.
#define MOE_LAUNCH(slot, kern, grid, block, st, p)                                                   \
    do {                                                                                             \
        if ((p).ev)                                                                                  \
            hipExtLaunchKernelGGL(kern, grid, block, 0, st, (p).ev[2 * (slot)], (p).ev[2 * (slot) + 1], 0, p); \
        else                                                                                         \
            hipLaunchKernelGGL(kern, grid, block, 0, st, p);                                         \
    } while (0)

// Kernel slots of one layer, per decode path (names as reported by the timing entry point).
constexpr int MAX_KERNEL_SLOTS = 4;

// Output layer (lm_head): logits [T, V] = x [T, D] . W [V, D]^T.
struct LmHeadArgs {
    const uint8_t *w;       // device layout of W
    const float *tscale;    // NVFP4 tensor scale (1 float), else unused
    const void *x;          // [T, D] fp32 (act 0) or bf16 (act 1)
    float *logits;          // [T, V]
    int V, D, T, act, fmt;
    int n_tiles, n_groups;  // set by the launcher
    hipEvent_t ev0, ev1;    // optional dispatch timing pair
};
hipError_t launch_lm_head(const LmHeadArgs &a, hipStream_t st);
// q4_1 canonical [rows, k] matrix -> code plane [rows, k/2] + scale plane [rows, k/32]
hipError_t launch_repack_q4_1_matrix(const uint8_t *canonical, uint8_t *packed, long long rows, int k,
                                     hipStream_t st);

// Decode attention (one new token per sequence), head size 128.
struct AttnArgs {
    int B, Hq, Hkv, window, max_len;
    int chunk;     // positions per chunk: attn_chunk_size(window, max_len, B, Hq, Hkv)
    int n_chunks;  // chunk slots per (sequence, head): attn_chunk_slots(window, max_len, chunk)
    float rope_base, eps;
    double rope_freq[64];  // base^(-2i/128), i < 64 (host-computed in fp64)
    const float *q, *k_new, *v_new, *q_norm_w, *k_norm_w, *sinks;
    const int32_t *pos;
    uint16_t *k_cache, *v_cache;  // bf16 [B, Hkv, max_len, 128]
    float *out;                   // [B, Hq, 128]
    float *part_m, *part_l;       // workspace [B, Hq, n_chunks]
    float *part_o;                // workspace [B, Hq, n_chunks, 128]
    hipEvent_t *ev;               // optional start/stop pairs for the 2 kernels
};
bool attn_uses_mfma(int window, int Hq, int Hkv);
int attn_chunk_size(int window, int max_len, int B, int Hq, int Hkv);
int attn_chunk_slots(int window, int max_len, int chunk);
hipError_t launch_attn(const AttnArgs &a, hipStream_t st);

hipError_t launch_decode(const DecodeParams &p, hipStream_t st);
// Batch-1 path (three kernels per layer); hipErrorNotSupported if the shape
// is outside what it was built for (the caller then takes launch_decode).
hipError_t launch_decode_b1(const DecodeParams &p, hipStream_t st);
// Small-batch path (1 <= T <= MAX_BN_T, regular shapes: d_model a multiple of 64
// units, d_ff of 16 or 32 units); hipErrorNotSupported otherwise.
hipError_t launch_decode_bn(const DecodeParams &p, hipStream_t st);
hipError_t launch_route_only(const DecodeParams &p, hipStream_t st);
// Whether the small-batch path runs this shape (format, D, F, E, S), routing included.
bool decode_bn_supported(int fmt, int D, int F, int E, int S);
hipError_t launch_bf16_to_f32(const uint16_t *in, float *out, int n, hipStream_t st);
}  // namespace moe
