// C ABI of libmoe: argument checks on the host, workspace layout, and the
// enqueueing of the decode, prefill and stack paths.  Nothing here touches
// the device before every check has passed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "moe_internal.h"
#include "moe_xcd.h"
#include "moe_persist.h"
#include "moe_prefill.h"

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const std::string &msg) {
    g_err = msg;
    return s;
}

moe_status ok() {
    g_err.clear();
    return MOE_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t mat_bytes(int fmt, size_t rows, size_t k) {
    if (fmt == MOE_W_BF16) return rows * k * 2;
    if (fmt == MOE_W_Q4_1) return rows * (k / 32) * 20;
    return rows * (k / 2) + rows * (k / 16);
}

moe_status check_dims(const moe_dims *d) {
    if (!d) return fail(MOE_ERR_INVALID_ARG, "dims is NULL");
    if (d->wfmt != MOE_W_BF16 && d->wfmt != MOE_W_Q4_1 && d->wfmt != MOE_W_NVFP4)
        return fail(MOE_ERR_UNSUPPORTED, "unknown weight format " + std::to_string(d->wfmt));
    if (d->d_model < 32 || d->d_model > 8192 || d->d_model % 32)
        return fail(MOE_ERR_INVALID_ARG, "d_model must be a multiple of 32 in [32, 8192]");
    if (d->d_ff < 32 || d->d_ff > 8192 || d->d_ff % 32)
        return fail(MOE_ERR_INVALID_ARG, "d_ff must be a multiple of 32 in [32, 8192]");
    if (d->n_routed < 1 || d->n_routed > 256) return fail(MOE_ERR_INVALID_ARG, "n_routed must be in [1, 256]");
    if (d->top_k < 1 || d->top_k > 8 || d->top_k > d->n_routed)
        return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, min(8, n_routed)]");
    if (d->n_shared < 0 || d->n_shared > 4) return fail(MOE_ERR_INVALID_ARG, "n_shared must be in [0, 4]");
    return MOE_OK;
}

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// Whether n_tokens runs on a decode path: up to 8 tokens always, up to 32 on
// the small-batch path when the shape fits it.
bool decode_tokens(const moe_dims &d, int T) {
    if (T <= moe::MAX_DECODE_T) return true;
    return T <= moe::MAX_BN_T && d.n_shared >= 1 &&
           moe::decode_bn_supported(d.wfmt, d.d_model, d.d_ff, d.n_routed, d.n_shared);
}

// Decode-path workspace (n_tokens <= 32).
struct DecodeWs {
    size_t logits, idx, w, xbuf, xconv, meta, act_expert, act_mask, act_w, h, ybuf0, ybuf1, work, pairs, b1_list, ps,
        xl, total;
    int amax;
};

DecodeWs decode_ws(const moe_dims &d, int T) {
    DecodeWs L{};
    L.amax = std::min(d.n_routed, T * d.top_k) + d.n_shared;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o += align_up(bytes);
        return at;
    };
    L.logits = take((size_t)T * d.n_routed * 4);
    L.idx = take((size_t)T * d.top_k * 4);
    L.w = take((size_t)T * d.top_k * 4);
    L.xbuf = take((size_t)T * d.d_model * 4);
    L.xconv = take((size_t)T * d.d_model * 4);
    L.meta = take(256);
    L.act_expert = take((size_t)L.amax * 4);
    L.act_mask = take((size_t)L.amax * 4);
    L.act_w = take((size_t)L.amax * T * 4);
    L.h = take((size_t)L.amax * T * d.d_ff * 4);
    L.ybuf0 = take((size_t)T * d.d_model * 4);
    L.ybuf1 = take((size_t)T * d.d_model * 4);
    L.work = take((size_t)(d.n_shared * ((T + 1) / 2) + T * d.top_k) * 16);
    L.pairs = take((size_t)(d.n_shared * T + T * d.top_k) * 16);
    L.b1_list = take(8 * 16 * 4);
    L.ps = take(moe::PS_WS_BYTES);
    L.xl = take(moe::xl_ws(d.d_model, d.d_ff, d.n_routed).total);
    L.total = o;
    return L;
}

template <typename T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

moe::DecodeParams base_params(const moe_dims &d, int T, void *ws, const DecodeWs &L) {
    moe::DecodeParams p{};
    p.D = d.d_model;
    p.F = d.d_ff;
    p.E = d.n_routed;
    p.S = d.n_shared;
    p.K = d.top_k;
    p.T = T;
    p.fmt = d.wfmt;
    p.amax = L.amax;
    p.expert_bytes = moe_packed_expert_bytes(&d);
    p.logits = at<float>(ws, L.logits);
    p.idx = at<int32_t>(ws, L.idx);
    p.w = at<float>(ws, L.w);
    p.xbuf = at<float>(ws, L.xbuf);
    p.meta = at<int32_t>(ws, L.meta);
    p.act_expert = at<int32_t>(ws, L.act_expert);
    p.act_mask = at<uint32_t>(ws, L.act_mask);
    p.act_w = at<float>(ws, L.act_w);
    p.h = at<float>(ws, L.h);
    p.work = at<int32_t>(ws, L.work);
    p.pairs = at<int32_t>(ws, L.pairs);
    p.b1_list = at<int32_t>(ws, L.b1_list);
    return p;
}

moe_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return ok();
}

moe_status check_ptr(const void *p, const char *name, bool required = true) {
    if (!p) return required ? fail(MOE_ERR_INVALID_ARG, std::string(name) + " is NULL") : MOE_OK;
    if (!aligned16(p)) return fail(MOE_ERR_ALIGNMENT, std::string(name) + " is not 16-byte aligned");
    return MOE_OK;
}

#define MOE_TRY(expr)                   \
    do {                                \
        moe_status _s = (expr);         \
        if (_s != MOE_OK) return _s;    \
    } while (0)

moe_status check_ws(const moe_dims *d, int T, const void *ws, size_t ws_bytes) {
    size_t need = 0;
    MOE_TRY(moe_workspace_size(d, T, &need));
    if (!ws || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes, got " +
                                           std::to_string(ws ? ws_bytes : 0));
    return check_ptr(ws, "ws");
}

// fp32 view of the decode input (bf16 inputs are widened into ws first).
moe_status decode_input(const moe_dims &d, const void *x, int act, int T, void *ws, const DecodeWs &L,
                        hipStream_t st, const float **out) {
    if (act == MOE_ACT_F32) {
        *out = static_cast<const float *>(x);
        return MOE_OK;
    }
    float *xc = at<float>(ws, L.xconv);
    MOE_TRY(hip_status(moe::launch_bf16_to_f32(static_cast<const uint16_t *>(x), xc, T * d.d_model, st),
                       "bf16 widening launch"));
    *out = xc;
    return MOE_OK;
}

// The batch-1 path when the shape fits it, the general decode path otherwise.
moe::PrefillArgs prefill_args(const moe_dims &d, const void *x, int act, int T, void *ws) {
    moe::PrefillArgs a{};
    a.D = d.d_model;
    a.F = d.d_ff;
    a.E = d.n_routed;
    a.S = d.n_shared;
    a.K = d.top_k;
    a.T = T;
    a.fmt = d.wfmt;
    a.act = act;
    a.expert_bytes = moe_packed_expert_bytes(&d);
    a.x = x;
    a.ws = ws;
    return a;
}

// The batch-1 path, else the small-batch path, else the general one (any
// shape).  *path (optional) receives 1, 3 or 2 respectively.  Each launcher
// checks its shape before enqueueing anything.
hipError_t launch_any(const moe::DecodeParams &p, hipStream_t st, int *path = nullptr) {
    hipError_t e = moe::launch_decode_b1(p, st);
    if (path) *path = 1;
    if (e != hipErrorNotSupported) return e;
    e = moe::launch_decode_bn(p, st);
    if (path) *path = 3;
    if (e != hipErrorNotSupported) return e;
    if (path) *path = 2;
    return moe::launch_decode(p, st);
}

// Kernel names of one layer's slots, per path (slot order of MOE_LAUNCH).
const char *const kB1Names = "b1_route;b1_topk_gateup;b1_down";
const char *const kGenericNames = "phase_a_kernel;select_kernel;gateup_kernel;down_kernel";
const char *const kBnNames = "bn_router;bn_gateup;bn_down";
const char *const kPsNames = "ps_stack;ps_clear";
const char *const kXlNames = "xl_layer;xl_reduce;xl_clear";

// Process-wide choice of the batch-1 decode path (moe_set_decode_path).
int g_decode_path = MOE_PATH_KERNELS;

// Whether batch-1 calls of this shape take the persistent kernel.
bool use_persistent(const moe_dims &d, int T) {
    return T == 1 && g_decode_path == MOE_PATH_PERSISTENT &&
           moe::ps_supported(d.wfmt, d.d_model, d.d_ff, d.n_routed, d.n_shared, d.top_k);
}

// Whether batch-1 calls of this shape take one kernel per layer with one
// expert per XCD.
bool use_xcd(const moe_dims &d, int T) {
    return T == 1 && g_decode_path == MOE_PATH_XCD &&
           moe::xl_supported(d.wfmt, d.d_model, d.d_ff, d.n_routed, d.n_shared, d.top_k);
}

// The batch-1 path with one kernel per layer and one expert per XCD over
// n_layers layers (host array), x0 fp32 [D]: a clear of the barrier counters
// per XL_MAX_LAYERS layers, one kernel per layer (each adds the previous
// layer's 8 partial outputs), and a final sum of the last layer's partials.
// ev (optional): per layer MAX_KERNEL_SLOTS start/stop pairs; pair 0 times the
// layer's kernel, pair 1 (last layer) the final sum, pair 2 a clear.
moe_status xcd_impl(const moe_dims &d, int n_layers, const moe_layer_weights *layers, const float *x0, float *y,
                    float *y_trace, int32_t *idx_trace, float *w_out, void *ws, const DecodeWs &L, hipStream_t st,
                    hipEvent_t *ev) {
    const moe::XlWs X = moe::xl_ws(d.d_model, d.d_ff, d.n_routed);
    char *base = static_cast<char *>(ws) + L.xl;
    float *part[2] = {reinterpret_cast<float *>(base + X.ypart0), reinterpret_cast<float *>(base + X.ypart1)};
    int32_t *bar = reinterpret_cast<int32_t *>(base + X.bar);
    // the error word is the persistent path's (ctrl[0]), so that
    // moe_decode_check reports the last batch-1 call of either path
    int32_t *err = at<int32_t>(ws, L.ps + 3 * (size_t)moe::PS_BLOCKS * moe::PS_SLOT_WORDS * 8);
    const size_t D = (size_t)d.d_model;
    moe::XlParams p{};
    p.D = d.d_model;
    p.F = d.d_ff;
    p.E = d.n_routed;
    p.K = d.top_k;
    p.expert_bytes = moe_packed_expert_bytes(&d);
    p.x0 = x0;
    // longest barrier wait: 20 ms of the 100 MHz real-time counter; the
    // environment variable MOE_XCD_SPIN_TICKS lowers it so that tests can drive
    // the give-up path with every kernel still ending normally
    p.spin = 2000000u;
    if (const char *e = getenv("MOE_XCD_SPIN_TICKS")) p.spin = (uint32_t)std::max(0, std::min((int)p.spin, atoi(e)));
    p.lg = reinterpret_cast<float *>(base + X.lg);
    p.hb = reinterpret_cast<float *>(base + X.hb);
    p.err = err;
    for (int l = 0; l < n_layers; l++) {
        hipEvent_t *lev = ev ? ev + (size_t)l * 2 * moe::MAX_KERNEL_SLOTS : nullptr;
        if (l % moe::XL_MAX_LAYERS == 0)
            MOE_TRY(hip_status(moe::xl_clear_launch(bar, err, l == 0, st, lev ? lev + 4 : nullptr), "clear launch"));
        const moe_layer_weights &w = layers[l];
        p.first = l == 0;
        p.yin = l == 0 ? nullptr : part[(l - 1) & 1];
        p.yout = part[l & 1];
        p.y_prev = (l > 0 && y_trace) ? y_trace + (size_t)(l - 1) * D : nullptr;
        p.router = static_cast<const uint16_t *>(w.router);
        p.bias = w.router_bias;
        p.experts = static_cast<const uint8_t *>(w.experts);
        p.tscale = d.wfmt == MOE_W_NVFP4 ? w.tensor_scale : nullptr;
        p.idx_out = idx_trace ? idx_trace + (size_t)l * d.top_k : nullptr;
        p.w_out = n_layers == 1 ? w_out : nullptr;
        p.bar = bar + (size_t)(l % moe::XL_MAX_LAYERS) * 2 * moe::XL_XCDS * moe::XL_LINE;
        MOE_TRY(hip_status(moe::xl_layer_launch(p, d.wfmt, st, lev), "layer launch"));
    }
    hipEvent_t *last = ev ? ev + (size_t)(n_layers - 1) * 2 * moe::MAX_KERNEL_SLOTS + 2 : nullptr;
    MOE_TRY(hip_status(moe::xl_reduce_launch(part[(n_layers - 1) & 1], y, d.d_model, st, last), "sum launch"));
    if (y_trace)
        MOE_TRY(hip_status(hipMemcpyAsync(y_trace + (size_t)(n_layers - 1) * D, y, D * 4, hipMemcpyDeviceToDevice, st),
                           "trace copy"));
    return ok();
}

// The persistent batch-1 path over n_layers layers (host array), x0 fp32
// [D]: clear the mailboxes, then one launch per PS_MAX_LAYERS layers.  ev:
// optional start/stop pairs, pair 0 for the clear and pair 1 + c for launch c.
moe_status persistent_impl(const moe_dims &d, int n_layers, const moe_layer_weights *layers, const float *x0,
                           float *y, float *y_trace, int32_t *idx_trace, float *w_trace, void *ws,
                           const DecodeWs &L, hipStream_t st, hipEvent_t *ev) {
    moe::PsParams p{};
    p.D = d.d_model;
    p.F = d.d_ff;
    p.E = d.n_routed;
    p.K = d.top_k;
    p.last_layer = n_layers - 1;
    p.expert_bytes = moe_packed_expert_bytes(&d);
    p.x0 = x0;
    p.y = y;
    p.y_trace = y_trace;
    p.idx_trace = idx_trace;
    p.w_trace = w_trace;
    // polls per wait before giving up: 2^18 (about 0.1 s); the environment
    // variable MOE_PERSISTENT_SPIN_LIMIT lowers it so that tests can drive the
    // give-up path with every kernel still ending normally
    p.spin = 1 << 18;
    if (const char *e = getenv("MOE_PERSISTENT_SPIN_LIMIT")) p.spin = std::max(0, std::min(p.spin, atoi(e)));
    const size_t nslot = (size_t)moe::PS_BLOCKS * moe::PS_SLOT_WORDS;
    p.mb_lg = at<unsigned long long>(ws, L.ps);
    p.mb_h = p.mb_lg + nslot;
    p.mb_y = p.mb_h + nslot;
    p.ctrl = reinterpret_cast<uint32_t *>(p.mb_y + nslot);
    MOE_TRY(hip_status(moe::ps_clear_launch(p, st, ev), "persistent clear launch"));
    for (int c = 0, l0 = 0; l0 < n_layers; c++, l0 += moe::PS_MAX_LAYERS) {
        p.l0 = l0;
        p.n_layers = std::min(moe::PS_MAX_LAYERS, n_layers - l0);
        for (int i = 0; i < p.n_layers; i++) {
            const moe_layer_weights &w = layers[l0 + i];
            p.layer[i] = moe::PsLayer{static_cast<const uint16_t *>(w.router), w.router_bias,
                                      static_cast<const uint8_t *>(w.experts),
                                      d.wfmt == MOE_W_NVFP4 ? w.tensor_scale : nullptr};
        }
        MOE_TRY(hip_status(moe::ps_launch(p, d.wfmt, st, ev ? ev + 2 * (1 + c) : nullptr), "persistent launch"));
    }
    return ok();
}

// ---- launch gate of the timed entry points ----
// The host enqueues event-bracketed launches more slowly than the GPU runs
// them; left alone, every timed kernel would start after an idle gap that a
// graph replay of the same launches does not have.  A one-wave kernel holds
// the stream until the host has enqueued every timed launch behind it, so
// that they then run back to back.  Its wait is bounded: it ends by itself
// after GATE_MAX_TICKS of the 100 MHz real-time counter (0.2 s), so a store
// that never arrives only delays the timed kernels.

constexpr uint64_t GATE_MAX_TICKS = 20000000ull;

__global__ void __launch_bounds__(64) hold_stream(uint32_t *flag, uint32_t seq, uint64_t max_ticks) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while ((int32_t)(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) - seq) < 0 &&
           __builtin_amdgcn_s_memrealtime() - t0 < max_ticks)
        __builtin_amdgcn_s_sleep(16);
}

// One gated timing call at a time per process: the flag word (pinned,
// host-coherent, kept until the process ends) only ever grows.
std::mutex g_gate_mu;
uint32_t *g_gate_host = nullptr;
uint32_t *g_gate_dev = nullptr;
uint32_t g_gate_seq = 0;

class StreamGate {
  public:
    // Enqueues the hold on st; without a flag word (allocation refused) the
    // timed launches run ungated.
    explicit StreamGate(hipStream_t st) : lk_(g_gate_mu) {
        if (!g_gate_host) {
            void *h = nullptr, *dptr = nullptr;
            if (hipHostMalloc(&h, 256, hipHostMallocCoherent | hipHostMallocMapped) != hipSuccess) {
                (void)hipGetLastError();
                return;
            }
            if (hipHostGetDevicePointer(&dptr, h, 0) != hipSuccess) {
                (void)hipGetLastError();
                (void)hipHostFree(h);
                return;
            }
            g_gate_host = static_cast<uint32_t *>(h);
            g_gate_dev = static_cast<uint32_t *>(dptr);
            __atomic_store_n(g_gate_host, g_gate_seq, __ATOMIC_RELEASE);
        }
        seq_ = ++g_gate_seq;
        hipLaunchKernelGGL(hold_stream, dim3(1), dim3(64), 0, st, g_gate_dev, seq_, GATE_MAX_TICKS);
        if (hipGetLastError() != hipSuccess) seq_ = 0;
    }
    // Lets the held stream run (idempotent).
    void release() {
        if (seq_) __atomic_store_n(g_gate_host, seq_, __ATOMIC_RELEASE);
        seq_ = 0;
    }
    ~StreamGate() { release(); }

  private:
    std::lock_guard<std::mutex> lk_;
    uint32_t seq_ = 0;
};

}  // namespace

moe_status moe::set_error(moe_status s, const std::string &msg) { return fail(s, msg); }

extern "C" {

size_t moe_packed_expert_bytes(const moe_dims *d) {
    if (check_dims(d) != MOE_OK) return 0;
    return 2 * mat_bytes(d->wfmt, d->d_ff, d->d_model) + mat_bytes(d->wfmt, d->d_model, d->d_ff);
}

moe_status moe_workspace_size(const moe_dims *d, int32_t n_tokens, size_t *bytes) {
    MOE_TRY(check_dims(d));
    if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    if (n_tokens < 1 || n_tokens > 65536) return fail(MOE_ERR_INVALID_ARG, "n_tokens must be in [1, 65536]");
    size_t need = 0;
    if (decode_tokens(*d, n_tokens)) need = decode_ws(*d, n_tokens).total;
    need = std::max(need, moe::prefill_ws_bytes(d->d_model, d->d_ff, d->n_routed, d->n_shared, d->top_k, n_tokens));
    *bytes = need;
    return ok();
}

moe_status moe_repack_weights(const moe_dims *d, const void *canonical, void *packed, int32_t n_experts,
                              void *stream) {
    MOE_TRY(check_dims(d));
    MOE_TRY(check_ptr(canonical, "canonical"));
    MOE_TRY(check_ptr(packed, "packed"));
    if (n_experts < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts must be >= 1");
    const size_t eb = moe_packed_expert_bytes(d);
    const char *c0 = static_cast<const char *>(canonical), *p0 = static_cast<const char *>(packed);
    if (c0 < p0 + eb * n_experts && p0 < c0 + eb * n_experts)
        return fail(MOE_ERR_INVALID_ARG, "canonical and packed overlap");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (d->wfmt != MOE_W_Q4_1)
        return hip_status(hipMemcpyAsync(packed, canonical, eb * n_experts, hipMemcpyDeviceToDevice, st),
                          "repack copy");
    return hip_status(moe::launch_repack_q4_1(static_cast<const uint8_t *>(canonical), static_cast<uint8_t *>(packed),
                                              n_experts, d->d_model, d->d_ff, st),
                      "repack launch");
}

moe_status moe_route_topk(const moe_dims *d, const void *x, int32_t act, int32_t n_tokens, const void *router,
                          const float *router_bias, int32_t *topk_idx, float *topk_w, float *logits_out, void *ws,
                          size_t ws_bytes, void *stream) {
    MOE_TRY(check_dims(d));
    if (act != MOE_ACT_F32 && act != MOE_ACT_BF16) return fail(MOE_ERR_UNSUPPORTED, "unknown activation type");
    if (n_tokens < 1 || n_tokens > 65536) return fail(MOE_ERR_INVALID_ARG, "n_tokens must be in [1, 65536]");
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(router, "router"));
    MOE_TRY(check_ptr(router_bias, "router_bias", false));
    MOE_TRY(check_ptr(topk_idx, "topk_idx"));
    MOE_TRY(check_ptr(topk_w, "topk_w"));
    MOE_TRY(check_ptr(logits_out, "logits_out", false));
    MOE_TRY(check_ws(d, n_tokens, ws, ws_bytes));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (n_tokens > moe::MAX_DECODE_T) {  // many tokens: the prefill router (MFMA) with its top-k
        moe::PrefillArgs a = prefill_args(*d, x, act, n_tokens, ws);
        a.router = static_cast<const uint16_t *>(router);
        a.bias = router_bias;
        a.idx_out = topk_idx;
        a.w_out = topk_w;
        a.logits_out = logits_out;
        a.route_only = 1;
        return hip_status(moe::launch_prefill(a, st), "prefill route launch");
    }
    const DecodeWs L = decode_ws(*d, n_tokens);
    moe::DecodeParams p = base_params(*d, n_tokens, ws, L);
    MOE_TRY(decode_input(*d, x, act, n_tokens, ws, L, st, &p.x));
    p.router = static_cast<const uint16_t *>(router);
    p.bias = router_bias;
    if (logits_out) p.logits = logits_out;
    p.idx_out = topk_idx;
    p.w_out = topk_w;
    p.want_router = 1;
    p.want_shared = 0;
    return hip_status(moe::launch_route_only(p, st), "route launch");
}

moe_status moe_expert_ffn_q4(const moe_dims *d, const void *x, int32_t act, int32_t n_tokens, const void *experts,
                             const float *tensor_scale, const int32_t *topk_idx, const float *topk_w, float *y,
                             void *ws, size_t ws_bytes, void *stream) {
    MOE_TRY(check_dims(d));
    if (act != MOE_ACT_F32 && act != MOE_ACT_BF16) return fail(MOE_ERR_UNSUPPORTED, "unknown activation type");
    if (n_tokens < 1 || n_tokens > 65536) return fail(MOE_ERR_INVALID_ARG, "n_tokens must be in [1, 65536]");
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(experts, "experts"));
    MOE_TRY(check_ptr(tensor_scale, "tensor_scale", d->wfmt == MOE_W_NVFP4));
    MOE_TRY(check_ptr(topk_idx, "topk_idx"));
    MOE_TRY(check_ptr(topk_w, "topk_w"));
    MOE_TRY(check_ptr(y, "y"));
    MOE_TRY(check_ws(d, n_tokens, ws, ws_bytes));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (n_tokens > moe::MAX_DECODE_T) {  // many tokens: grouped GEMM over the given routing
        moe::PrefillArgs a = prefill_args(*d, x, act, n_tokens, ws);
        a.experts = static_cast<const uint8_t *>(experts);
        a.tscale = d->wfmt == MOE_W_NVFP4 ? tensor_scale : nullptr;
        a.given_idx = topk_idx;
        a.given_w = topk_w;
        a.y = y;
        return hip_status(moe::launch_prefill(a, st), "prefill expert FFN launch");
    }
    const DecodeWs L = decode_ws(*d, n_tokens);
    moe::DecodeParams p = base_params(*d, n_tokens, ws, L);
    MOE_TRY(decode_input(*d, x, act, n_tokens, ws, L, st, &p.x));
    p.experts = static_cast<const uint8_t *>(experts);
    p.tscale = d->wfmt == MOE_W_NVFP4 ? tensor_scale : nullptr;
    p.route_given = 1;
    p.idx = const_cast<int32_t *>(topk_idx);
    p.w = const_cast<float *>(topk_w);
    p.want_router = 0;
    p.want_shared = 1;
    p.y = y;
    return hip_status(moe::launch_decode(p, st), "expert FFN launch");
}

static moe_status check_layer(const moe_dims *d, const moe_layer_weights *w) {
    if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
    MOE_TRY(check_ptr(w->router, "router"));
    MOE_TRY(check_ptr(w->router_bias, "router_bias", false));
    MOE_TRY(check_ptr(w->experts, "experts"));
    MOE_TRY(check_ptr(w->tensor_scale, "tensor_scale", d->wfmt == MOE_W_NVFP4));
    return MOE_OK;
}

moe_status moe_layer_forward(const moe_dims *d, const moe_layer_weights *w, const void *x, int32_t act,
                             int32_t n_tokens, float *y, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                             size_t ws_bytes, void *stream) {
    MOE_TRY(check_dims(d));
    if (!decode_tokens(*d, n_tokens))
        return moe_layer_forward_prefill(d, w, x, act, n_tokens, y, topk_idx_out, topk_w_out, ws, ws_bytes, stream);
    if (act != MOE_ACT_F32 && act != MOE_ACT_BF16) return fail(MOE_ERR_UNSUPPORTED, "unknown activation type");
    if (n_tokens < 1) return fail(MOE_ERR_INVALID_ARG, "n_tokens must be >= 1");
    MOE_TRY(check_layer(d, w));
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(y, "y"));
    MOE_TRY(check_ptr(topk_idx_out, "topk_idx_out", false));
    MOE_TRY(check_ptr(topk_w_out, "topk_w_out", false));
    MOE_TRY(check_ws(d, n_tokens, ws, ws_bytes));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const DecodeWs L = decode_ws(*d, n_tokens);
    moe::DecodeParams p = base_params(*d, n_tokens, ws, L);
    MOE_TRY(decode_input(*d, x, act, n_tokens, ws, L, st, &p.x));
    p.router = static_cast<const uint16_t *>(w->router);
    p.bias = w->router_bias;
    p.experts = static_cast<const uint8_t *>(w->experts);
    p.tscale = d->wfmt == MOE_W_NVFP4 ? w->tensor_scale : nullptr;
    p.idx_out = topk_idx_out;
    p.w_out = topk_w_out;
    p.want_router = 1;
    p.want_shared = 1;
    p.y = y;
    if (use_persistent(*d, n_tokens))
        return persistent_impl(*d, 1, w, p.x, y, nullptr, topk_idx_out, topk_w_out, ws, L, st, nullptr);
    if (use_xcd(*d, n_tokens)) return xcd_impl(*d, 1, w, p.x, y, nullptr, topk_idx_out, topk_w_out, ws, L, st, nullptr);
    return hip_status(launch_any(p, st), "layer launch");
}

static moe_status prefill_check(const moe_dims *d, const moe_layer_weights *w, const void *x, int32_t act,
                                int32_t n_tokens, float *y, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                                size_t ws_bytes) {
    MOE_TRY(check_dims(d));
    if (act != MOE_ACT_F32 && act != MOE_ACT_BF16) return fail(MOE_ERR_UNSUPPORTED, "unknown activation type");
    if (n_tokens < 1 || n_tokens > 65536) return fail(MOE_ERR_INVALID_ARG, "n_tokens must be in [1, 65536]");
    if (d->wfmt != MOE_W_Q4_1 && d->wfmt != MOE_W_NVFP4 && d->wfmt != MOE_W_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "prefill format");
    MOE_TRY(check_layer(d, w));
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(y, "y"));
    MOE_TRY(check_ptr(topk_idx_out, "topk_idx_out", false));
    MOE_TRY(check_ptr(topk_w_out, "topk_w_out", false));
    return check_ws(d, n_tokens, ws, ws_bytes);
}

static moe_status prefill_impl(const moe_dims *d, const moe_layer_weights *w, const void *x, int32_t act,
                               int32_t n_tokens, float *y, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                               size_t ws_bytes, hipStream_t st, hipEvent_t *ev) {
    MOE_TRY(prefill_check(d, w, x, act, n_tokens, y, topk_idx_out, topk_w_out, ws, ws_bytes));
    moe::PrefillArgs a = prefill_args(*d, x, act, n_tokens, ws);
    a.router = static_cast<const uint16_t *>(w->router);
    a.bias = w->router_bias;
    a.experts = static_cast<const uint8_t *>(w->experts);
    a.tscale = d->wfmt == MOE_W_NVFP4 ? w->tensor_scale : nullptr;
    a.y = y;
    a.idx_out = topk_idx_out;
    a.w_out = topk_w_out;
    a.ev = ev;
    return hip_status(moe::launch_prefill(a, st), "prefill launch");
}

moe_status moe_layer_forward_prefill(const moe_dims *d, const moe_layer_weights *w, const void *x, int32_t act,
                                     int32_t n_tokens, float *y, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                                     size_t ws_bytes, void *stream) {
    return prefill_impl(d, w, x, act, n_tokens, y, topk_idx_out, topk_w_out, ws, ws_bytes,
                        static_cast<hipStream_t>(stream), nullptr);
}

}  // extern "C"

namespace {

// Shared body of the stack entry points; ev (optional) holds
// n_layers * 2 * MAX_KERNEL_SLOTS events, *path receives the decode path.
moe_status stack_check(const moe_dims *d, int32_t n_layers, const moe_layer_weights *layers, const float *x0,
                       int32_t n_tokens, float *y, float *y_trace, int32_t *idx_trace, void *ws, size_t ws_bytes) {
    MOE_TRY(check_dims(d));
    if (n_layers < 1) return fail(MOE_ERR_INVALID_ARG, "n_layers must be >= 1");
    if (n_tokens < 1 || n_tokens > moe::MAX_DECODE_T)
        return fail(MOE_ERR_INVALID_ARG, "n_tokens must be in [1, 8] for stack decode");
    if (!layers) return fail(MOE_ERR_INVALID_ARG, "layers is NULL");
    for (int l = 0; l < n_layers; l++) MOE_TRY(check_layer(d, &layers[l]));
    MOE_TRY(check_ptr(x0, "x0"));
    MOE_TRY(check_ptr(y, "y"));
    MOE_TRY(check_ptr(y_trace, "y_trace", false));
    MOE_TRY(check_ptr(idx_trace, "idx_trace", false));
    return check_ws(d, n_tokens, ws, ws_bytes);
}

moe_status stack_impl(const moe_dims *d, int32_t n_layers, const moe_layer_weights *layers, const float *x0,
                      int32_t n_tokens, float *y, float *y_trace, int32_t *idx_trace, void *ws, size_t ws_bytes,
                      hipStream_t st, hipEvent_t *ev, int *path) {
    MOE_TRY(stack_check(d, n_layers, layers, x0, n_tokens, y, y_trace, idx_trace, ws, ws_bytes));
    const DecodeWs L = decode_ws(*d, n_tokens);
    if (use_persistent(*d, n_tokens)) {
        if (path) *path = 4;
        return persistent_impl(*d, n_layers, layers, x0, y, y_trace, idx_trace, nullptr, ws, L, st, ev);
    }
    if (use_xcd(*d, n_tokens)) {
        if (path) *path = 5;
        return xcd_impl(*d, n_layers, layers, x0, y, y_trace, idx_trace, nullptr, ws, L, st, ev);
    }
    const size_t TD = (size_t)n_tokens * d->d_model;
    const float *prev = nullptr;
    for (int l = 0; l < n_layers; l++) {
        moe::DecodeParams p = base_params(*d, n_tokens, ws, L);
        p.x = l == 0 ? x0 : nullptr;
        p.x_prev = l == 0 ? nullptr : prev;
        p.router = static_cast<const uint16_t *>(layers[l].router);
        p.bias = layers[l].router_bias;
        p.experts = static_cast<const uint8_t *>(layers[l].experts);
        p.tscale = d->wfmt == MOE_W_NVFP4 ? layers[l].tensor_scale : nullptr;
        p.idx_out = idx_trace ? idx_trace + (size_t)l * n_tokens * d->top_k : nullptr;
        p.want_router = 1;
        p.want_shared = 1;
        p.ev = ev ? ev + (size_t)l * 2 * moe::MAX_KERNEL_SLOTS : nullptr;
        float *out;
        if (l == n_layers - 1)
            out = y;
        else if (y_trace)
            out = y_trace + (size_t)l * TD;
        else
            out = at<float>(ws, (l & 1) ? L.ybuf1 : L.ybuf0);
        p.y = out;
        MOE_TRY(hip_status(launch_any(p, st, path), "stack layer launch"));
        prev = out;
    }
    if (y_trace)
        MOE_TRY(hip_status(hipMemcpyAsync(y_trace + (size_t)(n_layers - 1) * TD, y, TD * 4, hipMemcpyDeviceToDevice, st),
                           "trace copy"));
    return ok();
}

}  // namespace

extern "C" {

moe_status moe_stack_decode(const moe_dims *d, int32_t n_layers, const moe_layer_weights *layers, const float *x0,
                            int32_t n_tokens, float *y, float *y_trace, int32_t *idx_trace, void *ws,
                            size_t ws_bytes, void *stream) {
    return stack_impl(d, n_layers, layers, x0, n_tokens, y, y_trace, idx_trace, ws, ws_bytes,
                      static_cast<hipStream_t>(stream), nullptr, nullptr);
}

moe_status moe_stack_decode_timed(const moe_dims *d, int32_t n_layers, const moe_layer_weights *layers,
                                  const float *x0, int32_t n_tokens, float *y, int32_t *idx_trace, void *ws,
                                  size_t ws_bytes, float *kernel_us, int32_t *n_kernels, char *names,
                                  size_t names_cap, void *stream) {
    if (!kernel_us || !n_kernels) return fail(MOE_ERR_INVALID_ARG, "kernel_us / n_kernels is NULL");
    if (n_layers < 1 || n_layers > 4096) return fail(MOE_ERR_INVALID_ARG, "n_layers must be in [1, 4096]");
    MOE_TRY(stack_check(d, n_layers, layers, x0, n_tokens, y, nullptr, idx_trace, ws, ws_bytes));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t n_ev = (size_t)n_layers * 2 * moe::MAX_KERNEL_SLOTS;
    std::vector<hipEvent_t> ev(n_ev, nullptr);
    auto destroy = [&]() {
        for (hipEvent_t e : ev)
            if (e) (void)hipEventDestroy(e);
    };
    for (size_t i = 0; i < n_ev; i++) {
        if (hipEventCreate(&ev[i]) != hipSuccess) {
            destroy();
            return fail(MOE_ERR_HIP, "hipEventCreate failed");
        }
    }
    int path = 0;
    StreamGate gate(st);
    moe_status s = stack_impl(d, n_layers, layers, x0, n_tokens, y, nullptr, idx_trace, ws, ws_bytes, st,
                              ev.data(), &path);
    gate.release();
    if (s == MOE_OK && hipStreamSynchronize(st) != hipSuccess) s = fail(MOE_ERR_HIP, "stream synchronize failed");
    if (s != MOE_OK) {
        (void)hipStreamSynchronize(st);  // launches enqueued before the failure may still use the events
        destroy();
        return s;
    }
    if (path == 4) {
        // persistent kernel: its launches' time per layer, then the clear per call
        double tot = 0.0;
        const int chunks = (n_layers + moe::PS_MAX_LAYERS - 1) / moe::PS_MAX_LAYERS;
        bool okt = true;
        for (int c = 0; c < chunks; c++) {
            float ms = 0.f;
            okt &= hipEventElapsedTime(&ms, ev[2 * (1 + c)], ev[2 * (1 + c) + 1]) == hipSuccess;
            tot += ms;
        }
        float ms_clear = 0.f;
        okt &= hipEventElapsedTime(&ms_clear, ev[0], ev[1]) == hipSuccess;
        destroy();
        if (!okt) return fail(MOE_ERR_HIP, "event timing failed");
        kernel_us[0] = (float)(tot / n_layers * 1e3);
        kernel_us[1] = ms_clear * 1e3f;
        *n_kernels = 2;
        if (names && names_cap) snprintf(names, names_cap, "%s", kPsNames);
        return ok();
    }
    const int slots = path == 2 ? 4 : 3;  // the one-kernel-per-layer path (5): layer, final sum, clear
    for (int k = 0; k < slots; k++) {
        double tot = 0.0;
        int cnt = 0;
        for (int l = 0; l < n_layers; l++) {
            float ms = 0.f;
            const size_t b = (size_t)l * 2 * moe::MAX_KERNEL_SLOTS + 2 * k;
            if (hipEventElapsedTime(&ms, ev[b], ev[b + 1]) == hipSuccess) {
                tot += ms;
                cnt++;
            }
        }
        kernel_us[k] = cnt ? (float)(tot / cnt * 1e3) : -1.f;
    }
    (void)hipGetLastError();  // elapsed-time queries of slots a layer did not launch
    destroy();
    *n_kernels = slots;
    if (names && names_cap) {
        const char *src = path == 1 ? kB1Names : path == 3 ? kBnNames : path == 5 ? kXlNames : kGenericNames;
        snprintf(names, names_cap, "%s", src);
    }
    return ok();
}

moe_status moe_layer_forward_prefill_timed(const moe_dims *d, const moe_layer_weights *w, const void *x, int32_t act,
                                           int32_t n_tokens, float *y, void *ws, size_t ws_bytes, float *kernel_us,
                                           int32_t *n_kernels, char *names, size_t names_cap, void *stream) {
    if (!kernel_us || !n_kernels) return fail(MOE_ERR_INVALID_ARG, "kernel_us / n_kernels is NULL");
    MOE_TRY(prefill_check(d, w, x, act, n_tokens, y, nullptr, nullptr, ws, ws_bytes));
    hipEvent_t ev[2 * moe::PREFILL_SLOTS] = {};
    for (auto &e : ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            for (auto &f : ev)
                if (f) (void)hipEventDestroy(f);
            return fail(MOE_ERR_HIP, "hipEventCreate failed");
        }
    }
    StreamGate gate(static_cast<hipStream_t>(stream));
    moe_status s = prefill_impl(d, w, x, act, n_tokens, y, nullptr, nullptr, ws, ws_bytes,
                                static_cast<hipStream_t>(stream), ev);
    gate.release();
    if (s == MOE_OK && hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
        s = fail(MOE_ERR_HIP, "stream synchronize failed");
    if (s != MOE_OK) (void)hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (s == MOE_OK) {
        for (int k = 0; k < moe::PREFILL_SLOTS; k++) {
            float ms = 0.f;
            kernel_us[k] = hipEventElapsedTime(&ms, ev[2 * k], ev[2 * k + 1]) == hipSuccess ? ms * 1e3f : -1.f;
        }
        (void)hipGetLastError();
        *n_kernels = moe::PREFILL_SLOTS;
        if (names && names_cap) snprintf(names, names_cap, "%s", moe::prefill_names(act, moe::prefill_fused(d->wfmt, d->d_model, d->d_ff)));
    }
    for (auto &e : ev) (void)hipEventDestroy(e);
    return s == MOE_OK ? ok() : s;
}

// ---- output layer (lm_head) ----

static bool lm_head_fmt_ok(int32_t f) { return f == MOE_W_BF16 || f == MOE_W_Q4_1 || f == MOE_W_NVFP4; }

size_t moe_lm_head_bytes(int32_t vocab, int32_t d_model, int32_t wfmt) {
    if (vocab < 1 || vocab > MOE_LM_HEAD_MAX_VOCAB || d_model < 32 || d_model > MOE_LM_HEAD_MAX_D || d_model % 32 ||
        !lm_head_fmt_ok(wfmt))
        return 0;
    return mat_bytes(wfmt, (size_t)vocab, (size_t)d_model);
}

static moe_status lm_head_check_shape(int32_t vocab, int32_t d_model, int32_t wfmt) {
    if (!lm_head_fmt_ok(wfmt)) return fail(MOE_ERR_UNSUPPORTED, "unknown weight format " + std::to_string(wfmt));
    if (vocab < 1 || vocab > MOE_LM_HEAD_MAX_VOCAB)
        return fail(MOE_ERR_INVALID_ARG, "vocab must be in [1, " + std::to_string(MOE_LM_HEAD_MAX_VOCAB) + "]");
    if (d_model < 32 || d_model > MOE_LM_HEAD_MAX_D || d_model % 32)
        return fail(MOE_ERR_INVALID_ARG,
                    "d_model must be a multiple of 32 in [32, " + std::to_string(MOE_LM_HEAD_MAX_D) + "]");
    return MOE_OK;
}

moe_status moe_lm_head_repack(int32_t vocab, int32_t d_model, int32_t wfmt, const void *canonical, void *packed,
                              void *stream) {
    MOE_TRY(lm_head_check_shape(vocab, d_model, wfmt));
    MOE_TRY(check_ptr(canonical, "canonical"));
    MOE_TRY(check_ptr(packed, "packed"));
    const size_t nb = moe_lm_head_bytes(vocab, d_model, wfmt);
    const char *c0 = static_cast<const char *>(canonical), *p0 = static_cast<const char *>(packed);
    if (c0 < p0 + nb && p0 < c0 + nb) return fail(MOE_ERR_INVALID_ARG, "canonical and packed overlap");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (wfmt != MOE_W_Q4_1)
        return hip_status(hipMemcpyAsync(packed, canonical, nb, hipMemcpyDeviceToDevice, st), "lm_head copy");
    return hip_status(moe::launch_repack_q4_1_matrix(static_cast<const uint8_t *>(canonical),
                                                     static_cast<uint8_t *>(packed), vocab, d_model, st),
                      "lm_head repack launch");
}

static moe_status lm_head_args(int32_t vocab, int32_t d_model, int32_t wfmt, const void *weights,
                               const float *tensor_scale, const void *x, int32_t act, int32_t n_tokens,
                               float *logits, moe::LmHeadArgs *a) {
    MOE_TRY(lm_head_check_shape(vocab, d_model, wfmt));
    if (act != MOE_ACT_F32 && act != MOE_ACT_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "unknown activation type " + std::to_string(act));
    if (n_tokens < 1 || n_tokens > MOE_LM_HEAD_MAX_TOKENS)
        return fail(MOE_ERR_INVALID_ARG, "n_tokens must be in [1, " + std::to_string(MOE_LM_HEAD_MAX_TOKENS) + "]");
    MOE_TRY(check_ptr(weights, "weights"));
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(logits, "logits"));
    if (wfmt == MOE_W_NVFP4) {
        if (!tensor_scale) return fail(MOE_ERR_INVALID_ARG, "tensor_scale is NULL (NVFP4)");
        if (reinterpret_cast<uintptr_t>(tensor_scale) & 3u)
            return fail(MOE_ERR_ALIGNMENT, "tensor_scale is not 4-byte aligned");
    }
    const size_t out_bytes = (size_t)n_tokens * vocab * 4, x_bytes = (size_t)n_tokens * d_model * (act ? 2 : 4);
    const size_t w_bytes = moe_lm_head_bytes(vocab, d_model, wfmt);
    auto overlaps = [&](const void *p, size_t n) {
        const char *a0 = reinterpret_cast<const char *>(logits), *b0 = static_cast<const char *>(p);
        return a0 < b0 + n && b0 < a0 + out_bytes;
    };
    if (overlaps(x, x_bytes) || overlaps(weights, w_bytes) || (tensor_scale && overlaps(tensor_scale, 4)))
        return fail(MOE_ERR_INVALID_ARG, "logits overlaps an input");
    a->w = static_cast<const uint8_t *>(weights);
    a->tscale = tensor_scale;
    a->x = x;
    a->logits = logits;
    a->V = vocab;
    a->D = d_model;
    a->T = n_tokens;
    a->act = act;
    a->fmt = wfmt;
    return MOE_OK;
}

moe_status moe_lm_head(int32_t vocab, int32_t d_model, int32_t wfmt, const void *weights, const float *tensor_scale,
                       const void *x, int32_t act, int32_t n_tokens, float *logits, void *stream) {
    moe::LmHeadArgs a{};
    MOE_TRY(lm_head_args(vocab, d_model, wfmt, weights, tensor_scale, x, act, n_tokens, logits, &a));
    return hip_status(moe::launch_lm_head(a, static_cast<hipStream_t>(stream)), "lm_head launch");
}

moe_status moe_lm_head_timed(int32_t vocab, int32_t d_model, int32_t wfmt, const void *weights,
                             const float *tensor_scale, const void *x, int32_t act, int32_t n_tokens, float *logits,
                             float *kernel_us, void *stream) {
    if (!kernel_us) return fail(MOE_ERR_INVALID_ARG, "kernel_us is NULL");
    moe::LmHeadArgs a{};
    MOE_TRY(lm_head_args(vocab, d_model, wfmt, weights, tensor_scale, x, act, n_tokens, logits, &a));
    if (hipEventCreate(&a.ev0) != hipSuccess) return fail(MOE_ERR_HIP, "hipEventCreate failed");
    if (hipEventCreate(&a.ev1) != hipSuccess) {
        (void)hipEventDestroy(a.ev0);
        return fail(MOE_ERR_HIP, "hipEventCreate failed");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    moe_status s = hip_status(moe::launch_lm_head(a, st), "lm_head launch");
    if (s == MOE_OK && hipStreamSynchronize(st) != hipSuccess) s = fail(MOE_ERR_HIP, "stream synchronize failed");
    if (s == MOE_OK) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, a.ev0, a.ev1) != hipSuccess) s = fail(MOE_ERR_HIP, "hipEventElapsedTime failed");
        *kernel_us = ms * 1e3f;
    }
    (void)hipEventDestroy(a.ev0);
    (void)hipEventDestroy(a.ev1);
    return s == MOE_OK ? ok() : s;
}

// ---- decode attention ----

struct AttnWs {
    size_t part_m, part_l, part_o, total;
};

static AttnWs attn_ws(const moe_attn_dims &d, int B, int max_len) {
    AttnWs L{};
    const size_t nc = (size_t)moe::attn_chunk_slots(d.window, max_len,
                                                    moe::attn_chunk_size(d.window, max_len, B, d.n_q_heads, d.n_kv_heads));
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o += align_up(bytes);
        return at;
    };
    L.part_m = take((size_t)B * d.n_q_heads * nc * 4);
    L.part_l = take((size_t)B * d.n_q_heads * nc * 4);
    L.part_o = take((size_t)B * d.n_q_heads * nc * 128 * 4);
    L.total = o;
    return L;
}

static moe_status attn_check(const moe_attn_dims *d, int32_t B, int32_t max_len) {
    if (!d) return fail(MOE_ERR_INVALID_ARG, "dims is NULL");
    if (d->head_dim != 128) return fail(MOE_ERR_UNSUPPORTED, "head_dim must be 128");
    if (d->n_kv_heads < 1 || d->n_q_heads < d->n_kv_heads || d->n_q_heads % d->n_kv_heads || d->n_q_heads > 1024)
        return fail(MOE_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads (at most 1024)");
    const int grp = d->n_q_heads / d->n_kv_heads;
    if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
        return fail(MOE_ERR_UNSUPPORTED, "query heads per key/value head must be 1, 2, 4 or 8");
    if (d->window < 0) return fail(MOE_ERR_INVALID_ARG, "window must be >= 0");
    if (d->window > 0 && !(d->rope_base > 0.f)) return fail(MOE_ERR_INVALID_ARG, "rope_base must be > 0");
    if (!(d->norm_eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "norm_eps must be >= 0");
    if (B < 1 || B > 4096) return fail(MOE_ERR_INVALID_ARG, "n_seqs must be in [1, 4096]");
    if (max_len < 1 || max_len > 16777216) return fail(MOE_ERR_INVALID_ARG, "max_len must be in [1, 16777216]");
    return MOE_OK;
}

moe_status moe_attn_workspace_size(const moe_attn_dims *d, int32_t n_seqs, int32_t max_len, size_t *bytes) {
    MOE_TRY(attn_check(d, n_seqs, max_len));
    if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = attn_ws(*d, n_seqs, max_len).total;
    return ok();
}

moe_status moe_attn_chunk_plan(const moe_attn_dims *d, int32_t n_seqs, int32_t max_len, int32_t *chunk,
                               int32_t *slots) {
    MOE_TRY(attn_check(d, n_seqs, max_len));
    if (!chunk || !slots) return fail(MOE_ERR_INVALID_ARG, "chunk or slots is NULL");
    *chunk = moe::attn_chunk_size(d->window, max_len, n_seqs, d->n_q_heads, d->n_kv_heads);
    *slots = moe::attn_chunk_slots(d->window, max_len, *chunk);
    return ok();
}

// Host checks and the kernel arguments; nothing touches the device.
static moe_status attn_prepare(const moe_attn_dims *d, int32_t B, int32_t max_len, const float *q, const float *k_new,
                               const float *v_new, const float *q_norm_w, const float *k_norm_w, const float *sinks,
                               const int32_t *pos, uint16_t *k_cache, uint16_t *v_cache, float *out, void *ws,
                               size_t ws_bytes, moe::AttnArgs *args) {
    MOE_TRY(attn_check(d, B, max_len));
    const void *ins[] = {q, k_new, v_new, q_norm_w, k_norm_w, sinks, pos, k_cache, v_cache, out};
    const char *names[] = {"q", "k_new", "v_new", "q_norm_w", "k_norm_w", "sinks", "pos", "k_cache", "v_cache", "out"};
    for (int i = 0; i < 10; i++) MOE_TRY(check_ptr(ins[i], names[i]));
    const AttnWs L = attn_ws(*d, B, max_len);
    if (!ws || ws_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE, "workspace needs " + std::to_string(L.total) + " bytes, got " +
                                           std::to_string(ws ? ws_bytes : 0));
    MOE_TRY(check_ptr(ws, "ws"));
    // the written buffers must not overlap anything else
    const size_t cache_bytes = (size_t)B * d->n_kv_heads * max_len * 128 * 2;
    const size_t out_bytes = (size_t)B * d->n_q_heads * 128 * 4;
    struct R {
        const void *p;
        size_t n;
    } rs[] = {{q, (size_t)B * d->n_q_heads * 512}, {k_new, (size_t)B * d->n_kv_heads * 512},
              {v_new, (size_t)B * d->n_kv_heads * 512}, {q_norm_w, 512}, {k_norm_w, 512},
              {sinks, (size_t)d->n_q_heads * 4}, {pos, (size_t)B * 4}, {k_cache, cache_bytes},
              {v_cache, cache_bytes}, {out, out_bytes}, {ws, L.total}};
    const int nr = sizeof(rs) / sizeof(rs[0]);
    for (int i = 7; i < nr; i++)  // caches, out and ws against every other buffer
        for (int j = 0; j < nr; j++) {
            if (i == j || (j > 6 && j < i)) continue;
            const char *a0 = static_cast<const char *>(rs[i].p), *b0 = static_cast<const char *>(rs[j].p);
            if (a0 < b0 + rs[j].n && b0 < a0 + rs[i].n)
                return fail(MOE_ERR_INVALID_ARG, std::string(names[i < 10 ? i : 0]) + " overlaps another buffer");
        }
    moe::AttnArgs a{};
    a.B = B;
    a.Hq = d->n_q_heads;
    a.Hkv = d->n_kv_heads;
    a.window = d->window;
    a.max_len = max_len;
    a.chunk = moe::attn_chunk_size(d->window, max_len, B, d->n_q_heads, d->n_kv_heads);
    a.n_chunks = moe::attn_chunk_slots(d->window, max_len, a.chunk);
    a.rope_base = d->rope_base;
    a.eps = d->norm_eps;
    for (int i = 0; i < 64; i++) a.rope_freq[i] = std::pow((double)d->rope_base, -2.0 * i / 128.0);
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.q_norm_w = q_norm_w;
    a.k_norm_w = k_norm_w;
    a.sinks = sinks;
    a.pos = pos;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.out = out;
    a.part_m = at<float>(ws, L.part_m);
    a.part_l = at<float>(ws, L.part_l);
    a.part_o = at<float>(ws, L.part_o);
    *args = a;
    return MOE_OK;
}

moe_status moe_attn_decode(const moe_attn_dims *d, int32_t n_seqs, int32_t max_len, const float *q, const float *k_new,
                           const float *v_new, const float *q_norm_w, const float *k_norm_w, const float *sinks,
                           const int32_t *pos, uint16_t *k_cache, uint16_t *v_cache, float *out, void *ws,
                           size_t ws_bytes, void *stream) {
    moe::AttnArgs a{};
    MOE_TRY(attn_prepare(d, n_seqs, max_len, q, k_new, v_new, q_norm_w, k_norm_w, sinks, pos, k_cache, v_cache, out,
                         ws, ws_bytes, &a));
    return hip_status(moe::launch_attn(a, static_cast<hipStream_t>(stream)), "attention launch");
}

moe_status moe_attn_decode_timed(const moe_attn_dims *d, int32_t n_seqs, int32_t max_len, const float *q,
                                 const float *k_new, const float *v_new, const float *q_norm_w, const float *k_norm_w,
                                 const float *sinks, const int32_t *pos, uint16_t *k_cache, uint16_t *v_cache,
                                 float *out, void *ws, size_t ws_bytes, float *kernel_us, void *stream) {
    if (!kernel_us) return fail(MOE_ERR_INVALID_ARG, "kernel_us is NULL");
    moe::AttnArgs a{};
    MOE_TRY(attn_prepare(d, n_seqs, max_len, q, k_new, v_new, q_norm_w, k_norm_w, sinks, pos, k_cache, v_cache, out,
                         ws, ws_bytes, &a));
    hipEvent_t ev[4] = {};
    for (auto &e : ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            for (auto &f : ev)
                if (f) (void)hipEventDestroy(f);
            return fail(MOE_ERR_HIP, "hipEventCreate failed");
        }
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    a.ev = ev;
    StreamGate gate(st);
    moe_status s = hip_status(moe::launch_attn(a, st), "attention launch");
    gate.release();
    if (s == MOE_OK && hipStreamSynchronize(st) != hipSuccess) s = fail(MOE_ERR_HIP, "stream synchronize failed");
    if (s != MOE_OK) (void)hipStreamSynchronize(st);
    if (s == MOE_OK) {
        for (int k = 0; k < 2; k++) {
            float ms = 0.f;
            kernel_us[k] = hipEventElapsedTime(&ms, ev[2 * k], ev[2 * k + 1]) == hipSuccess ? ms * 1e3f : -1.f;
        }
        (void)hipGetLastError();
    }
    for (auto &e : ev) (void)hipEventDestroy(e);
    return s == MOE_OK ? ok() : s;
}

moe_status moe_set_decode_path(int32_t path) {
    if (path != MOE_PATH_KERNELS && path != MOE_PATH_PERSISTENT && path != MOE_PATH_XCD)
        return fail(MOE_ERR_INVALID_ARG, "path must be MOE_PATH_KERNELS, MOE_PATH_PERSISTENT or MOE_PATH_XCD");
    g_decode_path = path;
    return ok();
}

moe_status moe_decode_check(const moe_dims *d, int32_t n_tokens, const void *ws, size_t ws_bytes, void *stream) {
    MOE_TRY(check_ws(d, n_tokens, ws, ws_bytes));
    if (!decode_tokens(*d, n_tokens)) return ok();
    const DecodeWs L = decode_ws(*d, n_tokens);
    const size_t nslot = (size_t)moe::PS_BLOCKS * moe::PS_SLOT_WORDS;
    const char *ctrl = static_cast<const char *>(ws) + L.ps + 3 * nslot * 8;
    uint32_t flag = 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    MOE_TRY(hip_status(hipMemcpyAsync(&flag, ctrl, 4, hipMemcpyDeviceToHost, st), "error word copy"));
    MOE_TRY(hip_status(hipStreamSynchronize(st), "stream synchronize"));
    if (flag)
        return fail(MOE_ERR_HIP, "a wait of the batch-1 decode kernels (persistent, or one kernel per layer) gave up "
                                 "or crossed an XCD (outputs set to NaN)");
    return ok();
}

const char *moe_status_string(moe_status s) {
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer";
    case MOE_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *moe_last_error(void) { return g_err.c_str(); }

}  // extern "C"
