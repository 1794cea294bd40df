// Decode path of libmoe: router + shared-expert gate/up, top-k selection and
// expert union, routed gate/up, down projection with the weighted combine.
//
// The layer follows the Flint 40B-A2.5B pages ("Recursive Flint 40B-A2.5B",
// orcarouter.ai blog, section "The architecture is a memory-bandwidth
// argument": 256 routed experts, 6 chosen per token, one shared expert;
// decode is bound by moving weights).  Every kernel streams 4-bit (or bf16)
// weight units with 16-byte loads per lane, decodes them in registers and
// accumulates in fp32.  No floating-point atomics: every sum has a fixed
// order, so results do not depend on scheduling.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// x for token t scaled by xs (1, or the inverse RMS of the previous output).
template <int FMT>
__device__ __forceinline__ void load_x_scaled(XUnit<FMT> &xv, const float *src, int u, float xs, bool scaled) {
    load_x<FMT>(xv, src, u);
    if (scaled) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < Unit<FMT>::E; i++) {
            xv.v[i] *= xs;
            s += xv.v[i];
        }
        if (FMT == FMT_Q4_1) xv.sum = s;
    }
}

// h[slot, t, f] = silu(Wg x_t)[f] * (Wu x_t)[f] for the features of one wave.
template <int FMT, int LPR, int RG, int MAXT>
__device__ void gateup_unit(const DecodeParams &p, int slot, int expert, uint32_t mask, int f0, const float *xin,
                            const float *xs, bool scaled) {
    const int lane = threadIdx.x & (MOE_WAVE - 1);
    const int grp = lane / LPR, sub = lane % LPR;
    const int D = p.D, F = p.F;
    const uint8_t *eb = p.experts + (size_t)expert * p.expert_bytes;
    Mat mg{eb, F, D, tensor_scale<FMT>(p.tscale, 3 * expert + 0)};
    Mat mu{eb + mat_bytes<FMT>(F, D), F, D, tensor_scale<FMT>(p.tscale, 3 * expert + 1)};
    const int units = D / Unit<FMT>::E;
    const int fbase = f0 + grp * RG;
    float ag[RG][MAXT], au[RG][MAXT];
#pragma unroll
    for (int r = 0; r < RG; r++)
#pragma unroll
        for (int t = 0; t < MAXT; t++) ag[r][t] = au[r][t] = 0.f;
    for (int u = sub; u < units; u += LPR) {
        WUnit wg[RG], wu[RG];
#pragma unroll
        for (int r = 0; r < RG; r++) {
            int f = min(fbase + r, F - 1);
            wg[r] = load_unit<FMT>(mg, f, u);
            wu[r] = load_unit<FMT>(mu, f, u);
        }
#pragma unroll
        for (int t = 0; t < MAXT; t++) {
            if (t >= p.T || !((mask >> t) & 1u)) continue;
            XUnit<FMT> xv;
            load_x_scaled<FMT>(xv, xin + (size_t)t * D, u, xs[t], scaled);
#pragma unroll
            for (int r = 0; r < RG; r++) {
                ag[r][t] += unit_dot<FMT>(wg[r], xv, mg.ts);
                au[r][t] += unit_dot<FMT>(wu[r], xv, mu.ts);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RG; r++) {
#pragma unroll
        for (int t = 0; t < MAXT; t++) {
            if (t >= p.T || !((mask >> t) & 1u)) continue;
            float g = group_sum<LPR>(ag[r][t]);
            float u = group_sum<LPR>(au[r][t]);
            int f = fbase + r;
            if (sub == 0 && f < F) p.h[((size_t)slot * p.T + t) * F + f] = silu_mul(g, u);
        }
    }
}

// logits[t, e] = Wr[e, :] . x_t (+ bias[e]) for all tokens, one wave.
template <int MAXT>
__device__ void router_row(const DecodeParams &p, int e, const float *xin, const float *xs, bool scaled) {
    const int lane = threadIdx.x & (MOE_WAVE - 1);
    const int D = p.D;
    Mat mr{(const uint8_t *)p.router, p.E, D, 1.f};
    float acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; t++) acc[t] = 0.f;
    for (int u = lane; u < D / 8; u += MOE_WAVE) {
        WUnit w = load_unit<FMT_BF16>(mr, e, u);
#pragma unroll
        for (int t = 0; t < MAXT; t++) {
            if (t >= p.T) continue;
            XUnit<FMT_BF16> xv;
            load_x_scaled<FMT_BF16>(xv, xin + (size_t)t * D, u, xs[t], scaled);
            acc[t] += unit_dot<FMT_BF16>(w, xv, 1.f);
        }
    }
#pragma unroll
    for (int t = 0; t < MAXT; t++) {
        if (t >= p.T) continue;
        float s = group_sum<MOE_WAVE>(acc[t]);
        if (p.bias) s += p.bias[e];
        if (lane == 0) p.logits[(size_t)t * p.E + e] = s;
    }
}

// Phase A: router rows (if wanted) then the shared experts' gate/up feature
// groups, one wave per block.  For stacked layers every block derives the
// inverse RMS of the previous output itself and the grid writes the
// normalised input to xbuf for the routed gate/up kernel.
template <int FMT, int LPR_D, int RG, int MAXT>
__global__ void __launch_bounds__(MOE_WAVE) phase_a_kernel(DecodeParams p) {
    const int lane = threadIdx.x;
    float xs[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; t++) xs[t] = 1.f;
    const bool scaled = p.x_prev != nullptr;
    const float *xin = scaled ? p.x_prev : p.x;
    if (scaled) {
#pragma unroll
        for (int t = 0; t < MAXT; t++) {
            if (t >= p.T) continue;
            const float *y = p.x_prev + (size_t)t * p.D;
            float ss = 0.f;
            for (int i = lane; i < p.D; i += MOE_WAVE) ss += y[i] * y[i];
            ss = group_sum<MOE_WAVE>(ss);
            xs[t] = 1.0f / sqrtf(ss / (float)p.D + 1e-6f);
            for (int i = blockIdx.x * MOE_WAVE + lane; i < p.D; i += gridDim.x * MOE_WAVE)
                p.xbuf[(size_t)t * p.D + i] = y[i] * xs[t];
        }
    }
    const int n_router = p.want_router ? p.E : 0;
    const int unit = blockIdx.x;
    if (unit < n_router) {
        router_row<MAXT>(p, unit, xin, xs, scaled);
    } else if (p.want_shared) {
        constexpr int G = MOE_WAVE / LPR_D;
        const int per_expert = (p.F + G * RG - 1) / (G * RG);
        const int v = unit - n_router;
        const int s = v / per_expert, f0 = (v % per_expert) * G * RG;
        if (s < p.S) gateup_unit<FMT, LPR_D, RG, MAXT>(p, s, p.E + s, 0xFFFFFFFFu, f0, xin, xs, scaled);
    }
}

// Decode selection (T <= 8, one block): top-k per token (or the caller's
// routing), then the union of chosen experts: shared experts first, then
// routed experts in ascending index with a bitmask of the tokens using them.
__global__ void __launch_bounds__(512) select_kernel(DecodeParams p) {
    __shared__ int sel[MAX_DECODE_T][8];
    __shared__ float selw[MAX_DECODE_T][8];
    const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
    if (wave < p.T) {
        int e;
        float wi;
        if (p.route_given) {
            e = lane < p.K ? p.idx[wave * p.K + lane] : 0;
            wi = lane < p.K ? p.w[wave * p.K + lane] : 0.f;
        } else {
            wave_topk(p.logits + (size_t)wave * p.E, p.E, p.K, &e, &wi);
        }
        if (lane < p.K) {
            sel[wave][lane] = e;
            selw[wave][lane] = wi;
            if (!p.route_given) {
                p.idx[wave * p.K + lane] = e;
                p.w[wave * p.K + lane] = wi;
            }
            if (p.idx_out) p.idx_out[wave * p.K + lane] = e;
            if (p.w_out) p.w_out[wave * p.K + lane] = wi;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const uint32_t all = (1u << p.T) - 1u;
        if (lane < p.S) {
            p.act_expert[lane] = p.E + lane;
            p.act_mask[lane] = all;
            for (int t = 0; t < p.T; t++) p.act_w[lane * p.T + t] = 1.f;
        }
        int base = p.S;
        for (int c = 0; c < (p.E + 63) / 64; c++) {
            const int e = c * 64 + lane;
            uint32_t mask = 0;
            float wt[MAX_DECODE_T];
#pragma unroll
            for (int t = 0; t < MAX_DECODE_T; t++) wt[t] = 0.f;
            if (e < p.E) {
                // a repeated given index adds its slots' weights (slot order)
                for (int t = 0; t < p.T; t++)
                    for (int i = 0; i < p.K; i++)
                        if (sel[t][i] == e) {
                            mask |= 1u << t;
                            wt[t] += selw[t][i];
                        }
            }
            const uint64_t bal = __ballot(mask != 0);
            const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
            if (mask && pos < p.amax) {
                p.act_expert[pos] = e;
                p.act_mask[pos] = mask;
                for (int t = 0; t < p.T; t++) p.act_w[pos * p.T + t] = wt[t];
            }
            base += __popcll(bal);
        }
        if (lane == 0) p.meta[0] = min(base, p.amax);
    }
}

// Routed gate/up: one wave per (active slot, feature group).
template <int FMT, int LPR_D, int RG, int MAXT>
__global__ void __launch_bounds__(MOE_WAVE) gateup_kernel(DecodeParams p) {
    constexpr int G = MOE_WAVE / LPR_D;
    const int per_expert = (p.F + G * RG - 1) / (G * RG);
    const int slot = p.S + blockIdx.x / per_expert;
    const int f0 = (blockIdx.x % per_expert) * G * RG;
    if (slot >= p.meta[0]) return;
    const float *xin = p.x_prev ? p.xbuf : p.x;
    float xs[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; t++) xs[t] = 1.f;
    gateup_unit<FMT, LPR_D, RG, MAXT>(p, slot, p.act_expert[slot], p.act_mask[slot], f0, xin, xs, false);
}

// Down + combine: one wave per group of output rows, looping over every
// active slot (shared first, then routed in ascending expert order).
template <int FMT, int LPR_F, int RR, int MAXT>
__global__ void __launch_bounds__(MOE_WAVE) down_kernel(DecodeParams p) {
    constexpr int G = MOE_WAVE / LPR_F;
    const int lane = threadIdx.x & (MOE_WAVE - 1);
    const int grp = lane / LPR_F, sub = lane % LPR_F;
    const int D = p.D, F = p.F;
    const int r0 = blockIdx.x * G * RR + grp * RR;
    const int n_active = p.meta[0];
    const int units = F / Unit<FMT>::E;
    float acc[RR][MAXT];
#pragma unroll
    for (int r = 0; r < RR; r++)
#pragma unroll
        for (int t = 0; t < MAXT; t++) acc[r][t] = 0.f;
    for (int a = 0; a < n_active; a++) {
        const int e = p.act_expert[a];
        const uint32_t mask = p.act_mask[a];
        const uint8_t *eb = p.experts + (size_t)e * p.expert_bytes;
        Mat md{eb + 2 * mat_bytes<FMT>(F, D), D, F, tensor_scale<FMT>(p.tscale, 3 * e + 2)};
        for (int u = sub; u < units; u += LPR_F) {
            WUnit wd[RR];
#pragma unroll
            for (int r = 0; r < RR; r++) wd[r] = load_unit<FMT>(md, min(r0 + r, D - 1), u);
#pragma unroll
            for (int t = 0; t < MAXT; t++) {
                if (t >= p.T || !((mask >> t) & 1u)) continue;
                XUnit<FMT> hv;
                load_x<FMT>(hv, p.h + ((size_t)a * p.T + t) * F, u);
                const float c = p.act_w[a * p.T + t];
#pragma unroll
                for (int r = 0; r < RR; r++)
                    acc[r][t] = __builtin_fmaf(c, unit_dot<FMT>(wd[r], hv, md.ts), acc[r][t]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RR; r++) {
#pragma unroll
        for (int t = 0; t < MAXT; t++) {
            if (t >= p.T) continue;
            float s = group_sum<LPR_F>(acc[r][t]);
            if (sub == 0 && r0 + r < D) p.y[(size_t)t * D + r0 + r] = s;
        }
    }
}

__global__ void bf16_to_f32_kernel(const uint16_t *in, float *out, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = __uint_as_float((uint32_t)in[i] << 16);
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
constexpr int RG_GATEUP = 4;  // features per lane group in gate/up
constexpr int RR_DOWN = 1;    // output rows per lane group in down

template <int FMT, int LPR_D, int LPR_F, int MAXT>
static hipError_t launch_decode_t(const DecodeParams &p, hipStream_t st, bool route_only) {
    constexpr int GD = MOE_WAVE / LPR_D, GF = MOE_WAVE / LPR_F;
    const int per_expert = (p.F + GD * RG_GATEUP - 1) / (GD * RG_GATEUP);
    const int grid_a = (p.want_router ? p.E : 0) + (p.want_shared ? p.S * per_expert : 0);
    if (grid_a > 0)
        MOE_LAUNCH(0, (phase_a_kernel<FMT, LPR_D, RG_GATEUP, MAXT>), dim3(grid_a), dim3(MOE_WAVE), st, p);
    MOE_LAUNCH(1, select_kernel, dim3(1), dim3(512), st, p);
    if (route_only) return hipGetLastError();
    const int routed_slots = p.amax - p.S;
    if (routed_slots > 0)
        MOE_LAUNCH(2, (gateup_kernel<FMT, LPR_D, RG_GATEUP, MAXT>), dim3(routed_slots * per_expert),
                   dim3(MOE_WAVE), st, p);
    const int grid_d = (p.D + GF * RR_DOWN - 1) / (GF * RR_DOWN);
    MOE_LAUNCH(3, (down_kernel<FMT, LPR_F, RR_DOWN, MAXT>), dim3(grid_d), dim3(MOE_WAVE), st, p);
    return hipGetLastError();
}

static int lanes_for(int units) {
    int l = 4;
    while (l < units && l < 64) l <<= 1;
    return l;
}

template <int FMT, int MAXT>
static hipError_t launch_decode_f(const DecodeParams &p, hipStream_t st, bool route_only) {
    const int ld = lanes_for(p.D / Unit<FMT>::E), lf = lanes_for(p.F / Unit<FMT>::E);
#define MOE_CASE(A, B) \
    if (ld == A && lf == B) return launch_decode_t<FMT, A, B, MAXT>(p, st, route_only);
#define MOE_ROW(A) MOE_CASE(A, 4) MOE_CASE(A, 8) MOE_CASE(A, 16) MOE_CASE(A, 32) MOE_CASE(A, 64)
    MOE_ROW(4) MOE_ROW(8) MOE_ROW(16) MOE_ROW(32) MOE_ROW(64)
#undef MOE_ROW
#undef MOE_CASE
    return hipErrorInvalidValue;
}

static hipError_t dispatch(const DecodeParams &p, hipStream_t st, bool route_only) {
    const int maxt = p.T <= 1 ? 1 : (p.T <= 2 ? 2 : (p.T <= 4 ? 4 : 8));
#define MOE_T(FMTV)                                                        \
    if (maxt == 1) return launch_decode_f<FMTV, 1>(p, st, route_only);     \
    if (maxt == 2) return launch_decode_f<FMTV, 2>(p, st, route_only);     \
    if (maxt == 4) return launch_decode_f<FMTV, 4>(p, st, route_only);     \
    return launch_decode_f<FMTV, 8>(p, st, route_only);
    if (route_only || p.fmt == FMT_BF16) {
        MOE_T(FMT_BF16)
    }
    if (p.fmt == FMT_Q4_1) {
        MOE_T(FMT_Q4_1)
    }
    MOE_T(FMT_NVFP4)
#undef MOE_T
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t st) {
    if (p.T > MAX_DECODE_T) return hipErrorNotSupported;  // this path holds at most 8 tokens
    return dispatch(p, st, false);
}
hipError_t launch_route_only(const DecodeParams &p, hipStream_t st) { return dispatch(p, st, true); }

hipError_t launch_bf16_to_f32(const uint16_t *in, float *out, int n, hipStream_t st) {
    hipLaunchKernelGGL(bf16_to_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, in, out, n);
    return hipGetLastError();
}


}  // namespace moe
