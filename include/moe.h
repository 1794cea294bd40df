/*
 * moe.h - C ABI of libmoe, the MI355X (gfx950) sparse mixture-of-experts FFN
 * layer for token decode and prefill.
 *
 * What the layer computes is set by the Flint 40B-A2.5B pages:
 *   - "Recursive Flint 40B-A2.5B" (orcarouter.ai blog), section "The
 *     architecture is a memory-bandwidth argument", sparsity bullet: each
 *     MoE layer has 256 routed experts, 6 are chosen per token, and one
 *     shared expert is always active; decode is bound by moving weights, so
 *     only the chosen experts' weights are read.
 *   - same page, sections "What shipped" and "The quantisation recipe is
 *     the most transferable part": weights ship as 4-bit q4_1 and NVFP4.
 * Readings taken where the pages are open (gating, activation, layouts):
 *   logits l = x Wr^T (+ bias); p = softmax(l) over all routed experts;
 *   S = top_k experts by (logit descending, index ascending);
 *   w_i = p_i / sum_{j in S} p_j;
 *   expert(x) = Wd (silu(Wg x) * (Wu x)),  silu(z) = z / (1 + e^-z);
 *   y = sum_shared expert(x) + sum_{i in S} w_i expert_i(x).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless marked (host).  The caller owns
 *     every buffer; the library never allocates or frees device memory.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue
 *     work and return without synchronising the host.
 *   - Arguments are checked on the host before anything is enqueued; a
 *     failed check returns a negative status, enqueues nothing, and leaves a
 *     message for moe_last_error().  A launch failure returns
 *     MOE_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Device pointers must be 16-byte aligned (256 recommended).
 *   - Dims: d_model and d_ff multiples of 32 in [32, 8192]; 1 <= top_k <= 8;
 *     top_k <= n_routed <= 256;
 *     0 <= n_shared <= 4.
 *   - Matrices use the [out, in] (nn.Linear) convention; quantisation
 *     blocks run along the input dimension.  Experts are numbered
 *     0..n_routed-1 (routed) then n_routed.. (shared).
 *   - Results do not depend on run-to-run scheduling: no floating-point
 *     atomics; every sum has a fixed order.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* bad dims, NULL pointer, n_tokens out of range */
    MOE_ERR_UNSUPPORTED = -2, /* format/activation combination not built */
    MOE_ERR_WORKSPACE = -3,   /* ws NULL or smaller than moe_workspace_size() */
    MOE_ERR_ALIGNMENT = -4,   /* a device pointer not 16-byte aligned */
    MOE_ERR_HIP = -5          /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_W_BF16 = 0, MOE_W_Q4_1 = 1, MOE_W_NVFP4 = 2 } moe_wfmt;
typedef enum { MOE_ACT_F32 = 0, MOE_ACT_BF16 = 1 } moe_act;

/* (host) layer shape and weight format */
typedef struct {
    int32_t d_model;  /* hidden size D */
    int32_t d_ff;     /* expert intermediate size F */
    int32_t n_routed; /* routed experts E */
    int32_t n_shared; /* always-active experts */
    int32_t top_k;    /* experts chosen per token */
    int32_t wfmt;     /* moe_wfmt */
} moe_dims;

/* (host) struct of device pointers for one layer */
typedef struct {
    const void *router;        /* bf16 [n_routed, d_model] */
    const float *router_bias;  /* fp32 [n_routed] or NULL */
    const void *experts;       /* n_routed + n_shared experts in the device layout
                                  written by moe_repack_weights */
    const float *tensor_scale; /* NVFP4: fp32 [(n_routed + n_shared) * 3]
                                  (gate, up, down per expert); otherwise NULL */
} moe_layer_weights;

/*
 * Canonical expert layout (input of moe_repack_weights), per expert the
 * matrices gate [F, D], up [F, D], down [D, F] back to back:
 *   bf16:  row-major 16-bit values.
 *   q4_1:  rows x (K/32) blocks of 20 bytes {fp16 d, fp16 m, u8 q[16]};
 *          element j in the low nibble of q[j], element j+16 in the high
 *          nibble; value = d*q + m.
 *   NVFP4: nibbles [rows, K/2] (element 2i low nibble, 2i+1 high nibble of
 *          byte i), then E4M3 block-16 scales [rows, K/16]; value =
 *          e2m1(q) * e4m3(scale) * tensor_scale.
 * The device layout has the same size (moe_packed_expert_bytes).  For q4_1
 * each matrix becomes a code plane [rows, K/2] followed by a scale plane
 * [rows, K/32] of {fp16 d, fp16 m}; bf16 and NVFP4 are unchanged.
 */

/* (host) bytes of one expert (gate + up + down), canonical or device
   layout; 0 if dims are invalid. */
size_t moe_packed_expert_bytes(const moe_dims *dims);

/* (host) workspace bytes needed by moe_expert_ffn_q4 / moe_layer_forward /
   moe_stack_decode / moe_layer_forward_prefill for n_tokens tokens. */
moe_status moe_workspace_size(const moe_dims *dims, int32_t n_tokens, size_t *bytes);

/* Convert n_experts experts from the canonical layout to the device layout.
   canonical and packed are device buffers of n_experts *
   moe_packed_expert_bytes() bytes and must not overlap. */
moe_status moe_repack_weights(const moe_dims *dims, const void *canonical, void *packed, int32_t n_experts,
                              void *stream);

/*
 * Router and selection.  "Recursive Flint 40B-A2.5B" (orcarouter.ai blog),
 * section "The architecture is a memory-bandwidth argument", sparsity
 * bullet: every MoE layer routes each token to 6 of its 256 routed experts
 * (the softmax gate and the renormalisation are readings; the pages name only
 * the counts).  For each token:
 * logits = x Wr^T (+ bias) in fp32; softmax over n_routed; the top_k
 * experts by (logit descending, index ascending); renormalised weights.
 *   x          [n_tokens, d_model], fp32 (act = MOE_ACT_F32) or bf16
 *   router     bf16 [n_routed, d_model]; router_bias fp32 [n_routed] or NULL
 *   topk_idx   out int32 [n_tokens, top_k], slots in selection order
 *   topk_w     out fp32 [n_tokens, top_k], summing to 1 per token
 *   logits_out out fp32 [n_tokens, n_routed], or NULL
 *   ws, ws_bytes workspace of at least moe_workspace_size(dims, n_tokens)
 * 1 <= n_tokens <= 65536.
 */
moe_status moe_route_topk(const moe_dims *dims, const void *x, int32_t act, int32_t n_tokens, const void *router,
                          const float *router_bias, int32_t *topk_idx, float *topk_w, float *logits_out, void *ws,
                          size_t ws_bytes, void *stream);

/*
 * Expert FFN over given routing.  Same page and section as moe_route_topk:
 * besides the routed experts one shared expert is always active, and decode
 * time goes to moving the chosen experts' weights, so only those are read;
 * section "The quantisation recipe is the most transferable part": the
 * weights are 4-bit (q4_1, NVFP4).  For each token
 * y = sum_shared expert_s(x) + sum_i topk_w[i] * expert_{topk_idx[i]}(x),
 * reading from HBM only the chosen experts' 4-bit (or bf16) weights, each
 * distinct expert once per call (repeated reads by further tokens are served
 * by the caches).
 * 1 <= n_tokens <= 65536: up to 8 tokens (up to 32 when the small-batch
 * kernels fit the shape, see moe_layer_forward) take the decode GEMV path,
 * more take the grouped GEMM of moe_layer_forward_prefill.
 *   experts      device layout; tensor_scale as in moe_layer_weights
 *   topk_idx     int32 [n_tokens, top_k], normally in [0, n_routed) and
 *                distinct per token
 *   topk_w       fp32 [n_tokens, top_k]
 *   y            out fp32 [n_tokens, d_model]
 *   ws, ws_bytes workspace of at least moe_workspace_size(dims, n_tokens)
 * Indices outside [0, n_routed) select nothing (their slot contributes 0).
 * A repeated index contributes once per slot, as the sum above says: the
 * expert is applied once with the sum of its slots' weights (added in slot
 * order).
 */
moe_status moe_expert_ffn_q4(const moe_dims *dims, const void *x, int32_t act, int32_t n_tokens,
                             const void *experts, const float *tensor_scale, const int32_t *topk_idx,
                             const float *topk_w, float *y, void *ws, size_t ws_bytes, void *stream);

/*
 * Whole layer: route + expert FFN, as defined by moe_route_topk and
 * moe_expert_ffn_q4 (same page and section).  n_tokens <= 8 takes a decode path
 * (GEMV kernels that stream only the chosen experts' weights; an expert chosen
 * by several tokens comes from HBM once, its other reads from cache), and so
 * does n_tokens <= 32
 * when the small-batch kernels fit the shape (d_model 2048 or 4096 with
 * 4-bit weights, 512 or 1024 with bf16; d_ff of 16 or 32 blocks, a multiple
 * of 64; at least one shared expert); larger n_tokens take the prefill path
 * (moe_layer_forward_prefill).  topk_idx_out / topk_w_out may be
 * NULL.  1 <= n_tokens <= 65536.
 */
moe_status moe_layer_forward(const moe_dims *dims, const moe_layer_weights *w, const void *x, int32_t act,
                             int32_t n_tokens, float *y, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                             size_t ws_bytes, void *stream);

/*
 * moe_layer_forward without a caller workspace, for callers that cannot
 * allocate device memory: code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (less ws and ws_bytes),
 * kernels and results as moe_layer_forward.  The workspace is a static
 * device array of MOE_NOALLOC_SCRATCH_BYTES bytes, one copy per device, held
 * until the process ends; its address is looked up on the first call on each
 * device (the current device).  The call allocates nothing.  A call whose
 * moe_workspace_size() exceeds the array returns MOE_ERR_WORKSPACE with
 * nothing enqueued (at d_model 2048, d_ff 512, 256 + 1 experts, top-6 every
 * call of up to 339 tokens fits: the decode paths up to 32 tokens, the
 * grouped-GEMM path from 33 to 339).  Every call on a device shares that
 * device's array, which keeps the last call's contents: calls that overlap in
 * time on one device (different streams or threads) race and give undefined
 * results; calls ordered on one stream are safe.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
moe_status moe_layer_forward_noalloc(const moe_dims *dims, const moe_layer_weights *w, const void *x, int32_t act,
                                     int32_t n_tokens, float *y, int32_t *topk_idx_out, float *topk_w_out,
                                     void *stream);

/*
 * Prefill path for any n_tokens: route all tokens, permute
 * (token, slot) pairs by expert (histogram, scan, scatter), run the experts
 * as a grouped GEMM on the matrix cores (fp16 operands, fp32 accumulate),
 * and combine each token's slots in a fixed order.
 */
moe_status moe_layer_forward_prefill(const moe_dims *dims, const moe_layer_weights *w, const void *x,
                                     int32_t act, int32_t n_tokens, float *y, int32_t *topk_idx_out,
                                     float *topk_w_out, void *ws, size_t ws_bytes, void *stream);

/*
 * A stack of decode layers.  Same page and section: 47 of the model's 49
 * layers are MoE layers (also the layer table of the 648news.com page, section
 * "MoE structure and recommended settings"); the RMS normalisation between
 * layers, with unit gain and no residual, is a reading for independent
 * synthetic layers.  x_0 = x0 (fp32 [n_tokens, d_model]),
 * y_l = layer_l(x_l), x_{l+1} = y_l / sqrt(mean(y_l^2) + 1e-6) per token;
 * y receives y_{n_layers-1}.  layers is a host array of n_layers structs.
 * y_trace fp32 [n_layers, n_tokens, d_model] and idx_trace int32
 * [n_layers, n_tokens, top_k] receive every layer's output and selection, or
 * are NULL.  1 <= n_tokens <= 8.
 */
moe_status moe_stack_decode(const moe_dims *dims, int32_t n_layers, const moe_layer_weights *layers,
                            const float *x0, int32_t n_tokens, float *y, float *y_trace, int32_t *idx_trace,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Measurement variant of moe_stack_decode (no y_trace): the same kernels,
 * each launched with a start/stop event pair that takes the dispatch's own
 * begin and end timestamps, so the durations match a kernel trace.  The
 * pages time whole-model decode only (tokens/s on the two named machines);
 * this call gives the per-kernel split of the decode step that those
 * figures are made of.  Blocks the calling thread until the stack is done.
 * The launches are enqueued behind a one-wave kernel that holds the stream
 * until the host has enqueued all of them (at most 0.2 s), so that they run
 * back to back as in a graph replay instead of each after an idle gap;
 * timed calls of one process are serialised.  Results are those of
 * moe_stack_decode, bit for bit.
 *   kernel_us  (host) float [4]: mean duration in microseconds of each
 *              kernel slot of a layer, averaged over the layers that ran it
 *              (-1 for a slot that never ran).
 *   n_kernels  (host) receives the number of slots used (3 on the batch-1
 *              and small-batch paths, 4 on the general path,
 *              2 on the persistent path: the persistent kernel's time per
 *              layer, and the clearing kernel's per call).
 *   names      (host, optional) receives the slots' kernel names separated
 *              by ';' (truncated to names_cap bytes, NUL-terminated).
 * Creates and destroys 8 * n_layers HIP events (n_layers <= 4096); not for
 * use under stream capture.
 */
moe_status moe_stack_decode_timed(const moe_dims *dims, int32_t n_layers, const moe_layer_weights *layers,
                                  const float *x0, int32_t n_tokens, float *y, int32_t *idx_trace, void *ws,
                                  size_t ws_bytes, float *kernel_us, int32_t *n_kernels, char *names,
                                  size_t names_cap, void *stream);

/*
 * Measurement variant of moe_layer_forward_prefill (no routing outputs): the
 * same kernels, each launched with a start/stop event pair on its dispatch,
 * held back and then run back to back as in moe_stack_decode_timed.
 * Blocks the calling thread until the layer is done.
 *   kernel_us  (host) float [7]: duration in microseconds of each kernel, in
 *              launch order (router logits, top-k, scan, scatter, gate/up
 *              GEMM, down GEMM, combine); -1 for a kernel that did not run.
 *              q4_1 (and NVFP4 with d_model and d_ff multiples of 64) runs
 *              both GEMMs in one kernel, named "pf_ffn" in the gate/up slot;
 *              the down GEMM's slot then reports -1.
 *   n_kernels  (host) receives 7.
 *   names      (host, optional) receives the kernel names separated by ';'.
 * Creates and destroys 14 HIP events; not for use under stream capture.
 */
moe_status moe_layer_forward_prefill_timed(const moe_dims *dims, const moe_layer_weights *w, const void *x,
                                           int32_t act, int32_t n_tokens, float *y, void *ws, size_t ws_bytes,
                                           float *kernel_us, int32_t *n_kernels, char *names, size_t names_cap,
                                           void *stream);

/*
 * Output layer (lm_head) at decode.  "Recursive Flint 40B-A2.5B"
 * (orcarouter.ai blog), section "The quantisation recipe is the most
 * transferable part": the output layer is quantised to 4 bits, since with
 * 2.5 B active parameters it is a large share of the weights every decoded
 * token reads.  For each token t and vocabulary row v:
 *   logits[t, v] = sum_k x[t, k] * W[v, k]     (fp32 accumulation)
 * W is [vocab, d_model] in the formats of the experts (moe_wfmt; quantisation
 * blocks along d_model): canonical layout as for one expert matrix, device
 * layout as written by moe_lm_head_repack.  Limits: 1 <= vocab <=
 * MOE_LM_HEAD_MAX_VOCAB; d_model a multiple of 32 in [32,
 * MOE_LM_HEAD_MAX_D]; 1 <= n_tokens <= MOE_LM_HEAD_MAX_TOKENS.
 */
#define MOE_LM_HEAD_MAX_VOCAB 16777216
#define MOE_LM_HEAD_MAX_D 4096
#define MOE_LM_HEAD_MAX_TOKENS 8

/* (host) bytes of W (canonical or device layout); 0 if the shape or format
   is invalid. */
size_t moe_lm_head_bytes(int32_t vocab, int32_t d_model, int32_t wfmt);

/* Convert W from the canonical layout to the device layout (q4_1: code plane
   [vocab, d_model/2] then scale plane [vocab, d_model/32] of {fp16 d, fp16 m};
   bf16 and NVFP4: a copy).  canonical and packed are device buffers of
   moe_lm_head_bytes() bytes and must not overlap. */
moe_status moe_lm_head_repack(int32_t vocab, int32_t d_model, int32_t wfmt, const void *canonical, void *packed,
                              void *stream);

/*
 *   weights      W in the device layout
 *   tensor_scale NVFP4: fp32 [1] (4-byte aligned), the matrix's tensor scale;
 *                otherwise ignored (may be NULL)
 *   x            [n_tokens, d_model], fp32 (act = MOE_ACT_F32) or bf16
 *   logits       out fp32 [n_tokens, vocab]; must not overlap an input
 * Every row of W is read once per call (tokens beyond four per pass re-read
 * it, mostly from L2).  Each logit is a fixed-order sum.
 */
moe_status moe_lm_head(int32_t vocab, int32_t d_model, int32_t wfmt, const void *weights, const float *tensor_scale,
                       const void *x, int32_t act, int32_t n_tokens, float *logits, void *stream);

/* Measurement variant of moe_lm_head: the same kernel launched with a
   start/stop event pair on its dispatch; *kernel_us (host) receives its
   duration in microseconds.  Blocks the calling thread until it is done;
   not for use under stream capture. */
moe_status moe_lm_head_timed(int32_t vocab, int32_t d_model, int32_t wfmt, const void *weights,
                             const float *tensor_scale, const void *x, int32_t act, int32_t n_tokens, float *logits,
                             float *kernel_us, void *stream);

/*
 * Decode attention, the step before the MoE FFN in every layer.
 * "Recursive Flint 40B-A2.5B" (orcarouter.ai blog), section "The
 * architecture is a memory-bandwidth argument", attention and
 * positional-encoding bullets: 32 query heads share 4 key/value heads of
 * size 128; sliding-window layers see the current token and the 512 before
 * it and use rotary embeddings, full-attention layers see every earlier
 * token and use none; queries and keys are RMS-normalised per head, and
 * each head has a learned attention sink.  One new token per sequence b at
 * position P = pos[b]:
 *   qh = rope(rmsnorm(q[b,h]) * q_norm_w), kh likewise with k_norm_w
 *     (rmsnorm over the 128 values with norm_eps; rope only when window > 0:
 *     pairs (i, i + 64) turned by P * rope_base^(-2i/128));
 *   the caches receive bf16(kh) and bf16(v_new) at P;
 *   query head h reads key/value head h / (n_q_heads / n_kv_heads) at the
 *   positions j in [max(0, P - window + 1), P] (every j <= P when window = 0):
 *   s_j = qh . K[j] / sqrt(128),
 *   out[b,h] = sum_j e^(s_j) V[j] / (sum_j e^(s_j) + e^(sinks[h])).
 * Every sum has a fixed order.
 */
typedef struct {
    int32_t n_q_heads;  /* query heads; a multiple of n_kv_heads, group of 1, 2, 4 or 8 */
    int32_t n_kv_heads; /* key/value heads */
    int32_t head_dim;   /* must be 128 */
    int32_t window;     /* > 0: sliding window of this many positions, rotary embeddings; 0: full, none */
    float rope_base;    /* rotary base (used when window > 0), > 0 */
    float norm_eps;     /* RMSNorm epsilon, >= 0 */
} moe_attn_dims;

/* (host) workspace bytes moe_attn_decode needs for n_seqs sequences of
   caches of max_len positions. */
moe_status moe_attn_workspace_size(const moe_attn_dims *dims, int32_t n_seqs, int32_t max_len, size_t *bytes);

/* (host) the chunk plan moe_attn_decode uses for these sizes: *chunk
   positions per block of the first kernel, and *slots chunk partials per
   (sequence, query head) in the workspace (the combine kernel merges the
   slots a position range touches).  Sliding windows take 64-position
   chunks with groups of 8 query heads (the matrix-core kernel) and 32
   otherwise; full layers the smallest power of two in [64, 1024] that keeps a
   call near 512 blocks with groups of 8 query heads (the matrix-core
   kernel) and near 1024 blocks otherwise.  Same argument checks as
   moe_attn_workspace_size. */
moe_status moe_attn_chunk_plan(const moe_attn_dims *dims, int32_t n_seqs, int32_t max_len, int32_t *chunk,
                               int32_t *slots);

/*
 *   q          fp32 [n_seqs, n_q_heads, 128], the new tokens' query projections
 *   k_new      fp32 [n_seqs, n_kv_heads, 128]; v_new likewise
 *   q_norm_w   fp32 [128]; k_norm_w fp32 [128]; sinks fp32 [n_q_heads]
 *   pos        int32 [n_seqs] (device): the new token's position; positions
 *              0 .. P - 1 of the caches hold earlier tokens
 *   k_cache    bf16 [n_seqs, n_kv_heads, max_len, 128], read and written at
 *              P; v_cache likewise
 *   out        fp32 [n_seqs, n_q_heads, 128]
 *   ws         workspace of moe_attn_workspace_size() bytes
 * 1 <= n_seqs <= 4096, 1 <= max_len <= 16777216.  A position outside
 * [0, max_len) leaves that sequence's caches untouched and gives NaN
 * outputs.  Buffers must not overlap.
 */
moe_status moe_attn_decode(const moe_attn_dims *dims, int32_t n_seqs, int32_t max_len, const float *q,
                           const float *k_new, const float *v_new, const float *q_norm_w, const float *k_norm_w,
                           const float *sinks, const int32_t *pos, uint16_t *k_cache, uint16_t *v_cache, float *out,
                           void *ws, size_t ws_bytes, void *stream);

/* Measurement variant: the same two kernels, each launched with a
   start/stop event pair on its dispatch, held back and then run back to
   back as in moe_stack_decode_timed; kernel_us (host) float [2]
   receives their durations (chunks, combine) in microseconds.
   Blocks the calling thread; not for use under stream capture. */
moe_status moe_attn_decode_timed(const moe_attn_dims *dims, int32_t n_seqs, int32_t max_len, const float *q,
                                 const float *k_new, const float *v_new, const float *q_norm_w,
                                 const float *k_norm_w, const float *sinks, const int32_t *pos, uint16_t *k_cache,
                                 uint16_t *v_cache, float *out, void *ws, size_t ws_bytes, float *kernel_us,
                                 void *stream);

/*
 * (host) Batch-1 decode path of moe_layer_forward and moe_stack_decode,
 * process-wide, for calls made after it returns:
 *   MOE_PATH_KERNELS     (default) three kernels per layer;
 *   MOE_PATH_PERSISTENT  the persistent kernel where it is built for the
 *                        shape (q4_1 or NVFP4, d_model 2048, d_ff 512, one
 *                        shared expert, top_k <= 6, n_routed <= 256, one block
 *                        per CU fitting on 256 CUs), else three kernels.
 * The persistent kernel runs every layer of a stack in one dispatch (one per
 * 64 layers) after a small clearing kernel: one block per CU, the layer's
 * three global dependencies (logits, h, y) exchanged through mailboxes in the
 * workspace, and the next layer's router row and shared expert loaded while
 * the current layer runs.  On MI355X it is slower than three kernels per
 * layer (the exchanges cost more than kernel boundaries), hence not the
 * default.  Its waits are bounded: a wait that gives up ends the call with
 * NaN outputs and an error that moe_decode_check reports.
 *   MOE_PATH_XCD         one kernel per layer where built for the shape (q4_1
 *                        or NVFP4, d_model 2048, d_ff 512, 256 routed experts,
 *                        top-6, one shared expert, a device of 256 CUs in 8
 *                        XCDs), else three kernels.  Each XCD runs one active
 *                        expert (XCD j < 6 the routed expert of rank j, which
 *                        it selects from logits it computes itself; XCDs 6
 *                        and 7 half of the shared expert each) and writes a
 *                        partial output; the next layer's kernel adds the 8
 *                        partials.  Its exchanges stay inside one XCD (its
 *                        L2): barriers of the XCD's 32 blocks, bounded, and
 *                        checked against the blocks' XCC ids; a barrier that
 *                        gives up or sees another XCC ends the call with NaN
 *                        outputs and an error that moe_decode_check reports.
 */
#define MOE_PATH_KERNELS 0
#define MOE_PATH_PERSISTENT 1
#define MOE_PATH_XCD 2
moe_status moe_set_decode_path(int32_t path);

/*
 * (host) Whether the last batch-1 call that used this workspace on the
 * persistent kernel (or the one-kernel-per-layer path) finished its waits:
 * MOE_OK, or MOE_ERR_HIP when a wait gave up (its outputs are NaN).  Copies the workspace's error word and
 * synchronises `stream`.  Calls on other paths leave the word untouched.
 */
moe_status moe_decode_check(const moe_dims *dims, int32_t n_tokens, const void *ws, size_t ws_bytes,
                            void *stream);

/* (host) static description of a status code. */
const char *moe_status_string(moe_status s);

/* (host) detail of the last non-OK status on the calling thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
