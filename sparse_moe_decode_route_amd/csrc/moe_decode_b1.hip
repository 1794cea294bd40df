// Batch-1 decode path: three kernels per layer (the persistent kernel of
// moe_stack_persist.hip replaces it for the shapes that kernel is built for).
//
//   A  router logits (one wave per routed expert row); in a stack each wave
//      also applies the RMSNorm of the previous layer's output, and block 0
//      writes the normalised x.
//   B  h = silu(Wg x) * (Wu x), two features per wave, for every active
//      expert: the shared experts' waves issue their loads at once (they do
//      not depend on the routing, so they stream while the routed waves wait
//      for the logits); every routed wave finds its own expert, the j-th
//      largest logit (DPP argmax rounds, no barrier and no separate selection
//      kernel); wave 0 of the first blocks also runs the full selection with
//      weights for the routing outputs.
//   C  down projection with the weighted combine: a block owns 8 output
//      rows, each of its eight waves takes one active expert, h is staged in
//      LDS, the waves' partial sums are added in a fixed order.
//
// Decode is bound by moving weights (the Flint 40B-A2.5B pages, "Recursive
// Flint 40B-A2.5B", orcarouter.ai blog, section "The architecture is a
// memory-bandwidth argument"); at batch 1 one layer's 13.8 MB is under 2 us
// of HBM time, so what this path minimises is the chain of dependent memory
// round trips and the ALU latency of each wave: every wave issues all of its
// loads before the first use (loads are unconditional, with clamped
// indices, so that the compiler counts outstanding loads exactly), and
// reductions use DPP lane exchanges.
#include <hip/hip_fp16.h>
#include <algorithm>
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int B1_RG = 2;          // features (gate+up row pairs) per wave in A and B
constexpr int B1_WAVES_B = 4;     // waves per block in B
constexpr int B1_WAVES_C = 8;     // waves per block in C (one active slot each)
constexpr int B1_RR = 2;          // output rows per lane group in C
constexpr int B1_MAX_ACTIVE = 8;  // shared + routed slots
constexpr int B1_SLOTS_PER_WAVE = B1_MAX_ACTIVE / B1_WAVES_C;

// Gate/up rows f0..f0+RG-1 of one expert: loads issued first, used later.
template <int FMT, int UPLD, int RG>
struct GateUp {
    WUnit wg[RG][UPLD], wu[RG][UPLD];
    float tsg, tsu;
};

template <int FMT, int UPLD, int RG>
__device__ __forceinline__ void gateup_issue(GateUp<FMT, UPLD, RG> &g, const DecodeParams &p, int expert, int f0) {
    const int lane = threadIdx.x & (MOE_WAVE - 1);
    const uint8_t *eb = p.experts + (size_t)expert * p.expert_bytes;
    Mat mg{eb, p.F, p.D, tensor_scale<FMT>(p.tscale, 3 * expert + 0)};
    Mat mu{eb + mat_bytes<FMT>(p.F, p.D), p.F, p.D, tensor_scale<FMT>(p.tscale, 3 * expert + 1)};
    g.tsg = mg.ts;
    g.tsu = mu.ts;
#pragma unroll
    for (int r = 0; r < RG; r++)
#pragma unroll
        for (int i = 0; i < UPLD; i++) {
            g.wg[r][i] = load_unit<FMT>(mg, f0 + r, lane + MOE_WAVE * i);
            g.wu[r][i] = load_unit<FMT>(mu, f0 + r, lane + MOE_WAVE * i);
        }
}

// h[slot, f0 + r] = silu(g) * u from issued loads and x in registers.
template <int FMT, int UPLD, int RG>
__device__ __forceinline__ void gateup_finish(const GateUp<FMT, UPLD, RG> &g, const DecodeParams &p, int slot, int f0,
                                              const XUnit<FMT> (&xv)[UPLD]) {
    const int lane = threadIdx.x & (MOE_WAVE - 1);
    float ag[RG], au[RG];
#pragma unroll
    for (int r = 0; r < RG; r++) {
        ag[r] = 0.f;
        au[r] = 0.f;
#pragma unroll
        for (int i = 0; i < UPLD; i++) {
            ag[r] += unit_dot<FMT>(g.wg[r][i], xv[i], g.tsg);
            au[r] += unit_dot<FMT>(g.wu[r][i], xv[i], g.tsu);
        }
    }
    // the RG gate and RG up sums in one halving reduction: value k (gate r at
    // k = r, up r at k = RG + r) ends in lanes l % (2 RG) == k, so lane r holds
    // gate r and its up sum sits RG lanes on
    static_assert(RG == 1 || RG == 2 || RG == 4, "one exchange pairs the gate and up sums");
    float v[2 * RG];
#pragma unroll
    for (int r = 0; r < RG; r++) {
        v[r] = ag[r];
        v[RG + r] = au[r];
    }
    const float red = wave_reduce_rows<2 * RG>(v, lane);
    const float up = xor_lane(red, RG == 4 ? 2 : RG == 2 ? 1 : 0);  // lane ^ RG
    if (lane < RG) p.h[(size_t)slot * p.F + f0 + lane] = silu_mul(red, up);
}

// ---------------------------------------------------------------------------
// A: router rows (one wave per block)
// ---------------------------------------------------------------------------
template <int UPLR, bool SCALED>
__global__ void __launch_bounds__(MOE_WAVE) b1_route(DecodeParams p) {
    const int lane = threadIdx.x;
    constexpr bool scaled = SCALED;  // compile-time: no branch around loads
    const float *xin = scaled ? p.x_prev : p.x;
    float4 yr[2 * UPLR];
    // the rms partition is exactly this wave's router units: x = yr * xs
    const int e = blockIdx.x;
    load_rms_part<UPLR>(yr, xin);
    Mat mr{(const uint8_t *)p.router, p.E, p.D, 1.f};
    WUnit w[UPLR];
#pragma unroll
    for (int i = 0; i < UPLR; i++) w[i] = load_unit<FMT_BF16>(mr, e, lane + MOE_WAVE * i);
    __builtin_amdgcn_sched_barrier(0);
    const float xs = scaled ? inv_rms_from<UPLR>(yr) : 1.f;
    if (scaled && e == 0) {
#pragma unroll
        for (int i = 0; i < UPLR; i++) {
            const float4 a = yr[2 * i], b = yr[2 * i + 1];
            ((float4 *)p.xbuf)[2 * lane + 128 * i] = make_float4(a.x * xs, a.y * xs, a.z * xs, a.w * xs);
            ((float4 *)p.xbuf)[2 * lane + 1 + 128 * i] = make_float4(b.x * xs, b.y * xs, b.z * xs, b.w * xs);
        }
    }
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < UPLR; i++) {
        XUnit<FMT_BF16> xv;
        const float4 a = yr[2 * i], b = yr[2 * i + 1];
        xv.v[0] = a.x * xs;
        xv.v[1] = a.y * xs;
        xv.v[2] = a.z * xs;
        xv.v[3] = a.w * xs;
        xv.v[4] = b.x * xs;
        xv.v[5] = b.y * xs;
        xv.v[6] = b.z * xs;
        xv.v[7] = b.w * xs;
        xv.sum = 0.f;
        acc += unit_dot<FMT_BF16>(w[i], xv, 1.f);
    }
    const float s = wave_sum(acc);
    if (lane == 0) p.logits[e] = p.bias ? s + p.bias[e] : s;
}

// ---------------------------------------------------------------------------
// B: every active expert's gate/up; top-k in every routed wave
// ---------------------------------------------------------------------------
template <int FMT, int UPLD>
__global__ void __launch_bounds__(MOE_WAVE *B1_WAVES_B) b1_topk_gateup(DecodeParams p) {
    const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
    const int per_expert = p.F / B1_RG;
    const int gw = blockIdx.x * B1_WAVES_B + wave;
    // waves of routed slot j < K, then of shared expert j - K
    const int j = gw / per_expert, f0 = (gw % per_expert) * B1_RG;
    const float *xin = p.x_prev ? p.xbuf : p.x;
    if (j >= p.K) {
        // a shared expert: no routing dependency, its loads go out at once
        if (j >= p.K + p.S) return;
        const int s = j - p.K;
        GateUp<FMT, UPLD, B1_RG> g;
        gateup_issue<FMT, UPLD, B1_RG>(g, p, p.E + s, f0);
        XUnit<FMT> xv[UPLD];
#pragma unroll
        for (int i = 0; i < UPLD; i++) load_x<FMT>(xv[i], xin, lane + MOE_WAVE * i);
        __builtin_amdgcn_sched_barrier(0);
        gateup_finish<FMT, UPLD, B1_RG>(g, p, s, f0, xv);
        return;
    }
    float lv[4];
    wave_topk_load(p.logits, p.E, lv);
    int e = -1;
    if (wave == 0 && ((int)blockIdx.x < p.b1_ncopy || blockIdx.x == 0)) {
        // the full selection with weights, for the routing outputs and the
        // down kernel
        int es;
        float wi;
        wave_topk_regs(lv, p.E, p.K, &es, &wi);
        if (j < p.K) e = __shfl(es, j, MOE_WAVE);
        if ((int)blockIdx.x < p.b1_ncopy) {
            // one copy of the active list per XCD (block b runs on XCD b % 8),
            // read by the down kernel's blocks of the same XCD
            int32_t *cp = p.b1_list + 16 * blockIdx.x;
            if (lane < p.S) {
                cp[lane] = p.E + lane;
                cp[8 + lane] = __float_as_int(1.f);
            }
            if (lane < p.K) {
                cp[p.S + lane] = es;
                cp[8 + p.S + lane] = __float_as_int(wi);
            }
        }
        if (blockIdx.x == 0) {
            if (lane < p.K) {
                p.idx[lane] = es;
                p.w[lane] = wi;
                p.act_expert[p.S + lane] = es;
                p.act_w[p.S + lane] = wi;
                if (p.idx_out) p.idx_out[lane] = es;
                if (p.w_out) p.w_out[lane] = wi;
            }
            if (lane < p.S) {
                p.act_expert[lane] = p.E + lane;
                p.act_w[lane] = 1.f;
            }
            if (lane == 0) p.meta[0] = p.S + p.K;
        }
    }
    // every other wave finds its own expert (the j-th largest logit): no
    // barrier between the selection and the weight loads
    if (e < 0) e = wave_topk_nth(lv, p.E, j);
    GateUp<FMT, UPLD, B1_RG> g;
    gateup_issue<FMT, UPLD, B1_RG>(g, p, e, f0);
    // x in the same round trip as the weights (loaded before the top-k, a
    // wait for the logits would also wait for these)
    XUnit<FMT> xv[UPLD];
#pragma unroll
    for (int i = 0; i < UPLD; i++) load_x<FMT>(xv[i], xin, lane + MOE_WAVE * i);
    __builtin_amdgcn_sched_barrier(0);
    gateup_finish<FMT, UPLD, B1_RG>(g, p, p.S + j, f0, xv);
}

// ---------------------------------------------------------------------------
// C: down projection + combine; block = 8 waves over the same 8 rows, wave w
// takes slot w (two waves per SIMD keep a wave's LDS and FMA latencies
// hidden behind the other's).
// ---------------------------------------------------------------------------
template <int FMT, int LPR_F>
__global__ void __launch_bounds__(MOE_WAVE *B1_WAVES_C) b1_down(DecodeParams p) {
    constexpr int UE = Unit<FMT>::E;
    constexpr int F = LPR_F * UE;          // d_ff: one unit per lane of a row group
    constexpr int UP = UE + 4;             // padded LDS unit (floats)
    constexpr int PU = UP / 4;             // float4 positions per padded unit
    constexpr int G = MOE_WAVE / LPR_F;    // row groups per wave
    constexpr int ROWS = G * B1_RR;        // rows per block
    constexpr int NT = MOE_WAVE * B1_WAVES_C;
    constexpr int POS = B1_MAX_ACTIVE * LPR_F * PU;  // padded float4 positions (max)
    constexpr int NH = (POS + NT - 1) / NT;           // direct-to-LDS loads per thread
    __shared__ float4 hs4[NH * NT];
    __shared__ float part[B1_WAVES_C][ROWS];
    const float *hs = (const float *)hs4;
    const int tid = threadIdx.x, lane = tid % MOE_WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);  // uniform (SGPR)
    const int grp = lane / LPR_F, sub = lane % LPR_F;
    const int D = p.D;
    const int n_active = p.S + p.K;
    const int rb = blockIdx.x * ROWS;
    const int r0 = rb + grp * B1_RR;
    // 1) the active list (one load per lane) from this XCD's copy, read back
    //    per slot below
    const int la = min(lane, n_active - 1);
    const int32_t *lst = p.b1_list + 16 * (blockIdx.x % p.b1_ncopy);
    const int my_e = lst[la];
    const float my_c = __int_as_float(lst[8 + la]);
    // 2) this wave's slots' down rows (issued as soon as the list arrives)
    WUnit wd[B1_SLOTS_PER_WAVE][B1_RR];
    float ts[B1_SLOTS_PER_WAVE], coef[B1_SLOTS_PER_WAVE];
#pragma unroll
    for (int q = 0; q < B1_SLOTS_PER_WAVE; q++) {
        const int a = wave + B1_WAVES_C * q;
        const int e = __builtin_amdgcn_readlane(my_e, min(a, n_active - 1));
        coef[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_c), min(a, n_active - 1)));
        const uint8_t *eb = p.experts + (size_t)e * p.expert_bytes;
        Mat md{eb + 2 * mat_bytes<FMT>(F, D), D, F, tensor_scale<FMT>(p.tscale, 3 * e + 2)};
        ts[q] = md.ts;
#pragma unroll
        for (int r = 0; r < B1_RR; r++) wd[q][r] = load_unit<FMT>(md, min(r0 + r, D - 1), sub);
    }
    // 3) every slot's h straight into LDS (global_load_lds: lane L of a wave
    //    instruction writes 16 bytes at the instruction's LDS base + 16 L, so
    //    each lane gathers the source for its padded position; pad positions
    //    and slots past the active ones read h[0], a valid address); issued
    //    after the weight loads so that waiting for the list never waits for them
    const int wv = wave;
#pragma unroll
    for (int k = 0; k < NH; k++) {
        const int pos = (k * B1_WAVES_C + wv) * MOE_WAVE + lane;
        const int a = pos / (LPR_F * PU), r = pos % (LPR_F * PU);
        const int u = r / PU, q = r % PU;
        const bool real = (a < n_active) & (q < UE / 4);
        const uint32_t off = real ? (uint32_t)(a * F + u * UE + q * 4) : 0u;  // 32-bit select, no branch
        const float *src = p.h + off;
        __builtin_amdgcn_global_load_lds((const void *)src,
                                         (__attribute__((address_space(3))) void *)(hs4 + (k * B1_WAVES_C + wv) * MOE_WAVE),
                                         16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // h in LDS (and the weights) have arrived
    __syncthreads();
    // 4) dots of this wave's slots
    float acc[B1_RR];
#pragma unroll
    for (int r = 0; r < B1_RR; r++) acc[r] = 0.f;
#pragma unroll
    for (int q = 0; q < B1_SLOTS_PER_WAVE; q++) {
        // branch-free: every LDS slot holds finite data (inactive slots got
        // copies of h[0]), an inactive slot's term is dropped by the select
        const int a = wave + B1_WAVES_C * q;
        XUnit<FMT> hv;
        const float *src = hs + a * LPR_F * UP + sub * UP;
#pragma unroll
        for (int i = 0; i < UE / 4; i++) {
            const float4 f = ((const float4 *)src)[i];
            hv.v[4 * i + 0] = f.x;
            hv.v[4 * i + 1] = f.y;
            hv.v[4 * i + 2] = f.z;
            hv.v[4 * i + 3] = f.w;
        }
        float sum = 0.f;
        if (FMT == FMT_Q4_1) {
#pragma unroll
            for (int i = 0; i < UE; i++) sum += hv.v[i];
        }
        hv.sum = sum;
#pragma unroll
        for (int r = 0; r < B1_RR; r++) {
            const float t = __builtin_fmaf(coef[q], unit_dot<FMT>(wd[q][r], hv, ts[q]), acc[r]);
            acc[r] = a < n_active ? t : acc[r];
        }
    }
#pragma unroll
    for (int r = 0; r < B1_RR; r++) {
        const float s = group_sum<LPR_F>(acc[r]);
        if (sub == 0) part[wave][grp * B1_RR + r] = s;
    }
    __syncthreads();
    // 5) fixed-order sum of the waves' partials
    if (tid < ROWS && rb + tid < D) {
        float y = part[0][tid];
#pragma unroll
        for (int w = 1; w < B1_WAVES_C; w++) y += part[w][tid];
        p.y[rb + tid] = y;
    }
}

template <int FMT, int UPLD>
hipError_t launch_fmt(const DecodeParams &pin, hipStream_t st, int uplr, int lpr_f) {
    DecodeParams p = pin;
    p.b1_ncopy = std::min(8, (p.K * (p.F / B1_RG) + B1_WAVES_B - 1) / B1_WAVES_B);
    const int per_expert = p.F / B1_RG;
    const int grid_a = p.E;
#define MOE_A(U)                                                                          \
    if (p.x_prev)                                                                         \
        MOE_LAUNCH(0, (b1_route<U, true>), dim3(grid_a), dim3(MOE_WAVE), st, p);          \
    else                                                                                  \
        MOE_LAUNCH(0, (b1_route<U, false>), dim3(grid_a), dim3(MOE_WAVE), st, p);
    switch (uplr) {
    case 1: MOE_A(1) break;
    case 2: MOE_A(2) break;
    case 4: MOE_A(4) break;
    default: MOE_A(8) break;
    }
#undef MOE_A
    const int waves_b = (p.K + p.S) * per_expert;
    const int grid_b = (waves_b + B1_WAVES_B - 1) / B1_WAVES_B;
    MOE_LAUNCH(1, (b1_topk_gateup<FMT, UPLD>), dim3(grid_b), dim3(MOE_WAVE * B1_WAVES_B), st, p);
    const int rows_per_block = (MOE_WAVE / lpr_f) * B1_RR;
    const int grid_c = (p.D + rows_per_block - 1) / rows_per_block;
    switch (lpr_f) {
    case 8: MOE_LAUNCH(2, (b1_down<FMT, 8>), dim3(grid_c), dim3(MOE_WAVE * B1_WAVES_C), st, p); break;
    case 16: MOE_LAUNCH(2, (b1_down<FMT, 16>), dim3(grid_c), dim3(MOE_WAVE * B1_WAVES_C), st, p); break;
    default: MOE_LAUNCH(2, (b1_down<FMT, 32>), dim3(grid_c), dim3(MOE_WAVE * B1_WAVES_C), st, p); break;
    }
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_b1_fmt(const DecodeParams &p, hipStream_t st) {
    constexpr int UE = Unit<FMT>::E;
    if (p.D % (MOE_WAVE * UE) || p.D % 512) return hipErrorNotSupported;
    const int upld = p.D / (MOE_WAVE * UE), uplr = p.D / 512;
    const int lpr_f = p.F / UE;
    if (upld > 2 || (uplr != 1 && uplr != 2 && uplr != 4 && uplr != 8)) return hipErrorNotSupported;
    if (lpr_f != 8 && lpr_f != 16 && lpr_f != 32) return hipErrorNotSupported;
    if (p.F % B1_RG) return hipErrorNotSupported;
    return upld == 1 ? launch_fmt<FMT, 1>(p, st, uplr, lpr_f) : launch_fmt<FMT, 2>(p, st, uplr, lpr_f);
}

}  // namespace

hipError_t launch_decode_b1(const DecodeParams &p, hipStream_t st) {
    if (p.T != 1 || p.route_given || !p.want_router || !p.want_shared) return hipErrorNotSupported;
    if (p.S + p.K > B1_MAX_ACTIVE || p.S < 0) return hipErrorNotSupported;
    if (p.fmt == FMT_Q4_1) return launch_b1_fmt<FMT_Q4_1>(p, st);
    if (p.fmt == FMT_NVFP4) return launch_b1_fmt<FMT_NVFP4>(p, st);
    return launch_b1_fmt<FMT_BF16>(p, st);
}

}  // namespace moe
