// Batch-1 decode of a whole stack of MoE layers in one persistent kernel.
//
// The Flint 40B-A2.5B pages put decode time in moving weights ("Recursive
// Flint 40B-A2.5B", orcarouter.ai blog, section "The architecture is a
// memory-bandwidth argument") and describe a decode megakernel that fuses
// the whole forward pass into one dispatch (same page, section "The
// quantisation recipe is the most transferable part").  At batch 1 one
// layer moves 13.8 MB, under 2 us of HBM time, so what costs time is the
// chain of global dependencies per layer (x -> logits -> top-k -> h -> y)
// and the memory round trip after each.  Here one block per CU (256 blocks
// of 8 waves, all co-resident) runs every layer:
//
//   block g owns router row g, features FPB*g .. FPB*g+FPB-1 of every active
//   expert's gate/up, and output rows RB*g .. RB*g+RB-1 of the down projection.
//   wave 0      the shared expert's gate/up (its weights loaded one layer ahead)
//   waves 1..K  routed expert j = wave-1: gate/up and down, loaded after the top-k
//   wave 7      the router row (loaded one layer ahead), the logits exchange,
//               the shared expert's down projection (loaded one layer ahead)
//
// The three all-to-all dependencies of a layer go through per-block mailbox
// slots in the workspace: 8-byte words {fp32 value, tag}, written and read
// with agent-scope (sc1) accesses, tag = global layer index + 1, so a reader
// polls the data itself until every word carries the current tag.  A
// prologue kernel clears the slots at every call.  A layer reuses the slots
// of the one before: a block writes layer l+1 only after reading every
// block's y of layer l, which every block writes only after it has read the
// layer's logits and h, so no write can overtake a read of the slot's old
// value.  Every wait is bounded: a wave that polls too long, or sees another
// block's abort flag, stops; its block then writes NaN to its output rows
// and the error word is set.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_persist.h"

namespace moe {
namespace {

constexpr int NB = PS_BLOCKS;
constexpr int NW = 8;              // waves per block
constexpr int NT = NW * MOE_WAVE;  // 512 threads
constexpr int SLOT = PS_SLOT_WORDS;
constexpr int W_ROUTER = NW - 1;

typedef unsigned long long u64;

__device__ __forceinline__ u64 mb_load(const u64 *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void mb_store(u64 *p, float v, uint32_t tag) {
    __hip_atomic_store(p, ((u64)tag << 32) | (u64)__float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctrl_load(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(u64 v, uint32_t tag) { return (uint32_t)(v >> 32) == tag; }
__device__ __forceinline__ float val_of(u64 v) { return __uint_as_float((uint32_t)v); }

// Poll N mailbox words per lane until all carry `tag` in every lane of the
// wave.  A wave that polls `spin` times raises the abort flag (ctrl[0]) and
// returns false; so does a wave that finds the flag raised (checked every 64
// polls), and then v holds whatever was read last.  The kernel runs on after
// an abort (every block keeps its barriers) with waits that end at once, and
// its outputs are overwritten with NaN at the end.
template <int N>
__device__ __forceinline__ bool mb_poll(const u64 *const (&a)[N], u64 (&v)[N], uint32_t tag, uint32_t *ctrl,
                                        int spin) {
    for (int n = 0;; n++) {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] = mb_load(a[i]);
        bool ok = true;
#pragma unroll
        for (int i = 0; i < N; i++) ok &= tag_is(v[i], tag);
        if (__all(ok)) return true;
        if ((n & 63) == 63 && ctrl_load(ctrl) != 0u) return false;
        if (n >= spin) {
            __hip_atomic_fetch_or(ctrl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
    }
}

// LDS carve-up (floats) of the block's 96 KB pool; the pool is sized so that
// one block fills a CU's LDS share and the blocks spread one per CU.
constexpr int L_X = 0;                       // x of the layer [D <= 4096] (y of the previous layer during the gather)
constexpr int L_SSQ = L_X + 4096;            // per-block sums of squares [NB]
constexpr int L_LG = L_SSQ + NB;             // logits [256]
constexpr int L_PART = L_LG + 256;           // down partial rows [8 waves][RB <= 16]
constexpr int L_H = L_PART + NW * 16;        // h of each slot [8][F <= 1024]
constexpr int L_END = L_H + NW * 1024;
constexpr int L_POOL = 24576;                // 96 KB
static_assert(L_END <= L_POOL, "LDS pool");

template <int FMT, int UPLD, int FPB, int RB, int NDU>
struct PsShape {
    static constexpr int UE = Unit<FMT>::E;
    static constexpr int D = UPLD * MOE_WAVE * UE;     // d_model
    static constexpr int F = FPB * NB;                 // d_ff
    static constexpr int UF = F / UE;                  // down units per row
    static constexpr int UPLR = D / 512;               // router units (8 bf16) per lane
    static_assert(RB * NB == D, "down rows per block");
    static_assert(RB * UF == NDU * MOE_WAVE, "down units per lane");
    static_assert(UF % NDU == 0 && (UF / NDU) <= 64, "a lane's down units stay in one row");
};

template <int FMT, int UPLD>
__device__ __forceinline__ void x_units(XUnit<FMT> (&xv)[UPLD], const float *xs, int lane) {
    constexpr int UE = Unit<FMT>::E;
#pragma unroll
    for (int i = 0; i < UPLD; i++) {
        const float4 *p = reinterpret_cast<const float4 *>(xs + (size_t)(lane + MOE_WAVE * i) * UE);
#pragma unroll
        for (int c = 0; c < UE / 4; c++) {
            const float4 f = p[c];
            xv[i].v[4 * c + 0] = f.x;
            xv[i].v[4 * c + 1] = f.y;
            xv[i].v[4 * c + 2] = f.z;
            xv[i].v[4 * c + 3] = f.w;
        }
        float s = 0.f;
        if (FMT == FMT_Q4_1) {
#pragma unroll
            for (int k = 0; k < UE; k++) s += xv[i].v[k];
        }
        xv[i].sum = s;
    }
}

// gate/up rows of features f0 .. f0+FPB-1 of expert e (UPLD units per lane per row)
template <int FMT, int UPLD, int FPB>
struct GU {
    WUnit g[FPB][UPLD], u[FPB][UPLD];
    float tg, tu;
};
template <int FMT, int UPLD, int FPB>
__device__ __forceinline__ void gu_load(GU<FMT, UPLD, FPB> &w, const uint8_t *experts, const float *tscale,
                                        size_t expert_bytes, int D, int F, int e, int f0, int lane) {
    const uint8_t *eb = experts + (size_t)e * expert_bytes;
    Mat mg{eb, F, D, tensor_scale<FMT>(tscale, 3 * e + 0)};
    Mat mu{eb + mat_bytes<FMT>(F, D), F, D, tensor_scale<FMT>(tscale, 3 * e + 1)};
    w.tg = mg.ts;
    w.tu = mu.ts;
#pragma unroll
    for (int r = 0; r < FPB; r++)
#pragma unroll
        for (int i = 0; i < UPLD; i++) {
            w.g[r][i] = load_unit<FMT>(mg, f0 + r, lane + MOE_WAVE * i);
            w.u[r][i] = load_unit<FMT>(mu, f0 + r, lane + MOE_WAVE * i);
        }
}
// h = silu(gate . x) * (up . x) for the FPB features; lane r < FPB returns feature r
template <int FMT, int UPLD, int FPB>
__device__ __forceinline__ float gu_finish(const GU<FMT, UPLD, FPB> &w, const XUnit<FMT> (&xv)[UPLD], int lane) {
    float v[2 * FPB];
#pragma unroll
    for (int r = 0; r < FPB; r++) {
        float ag = 0.f, au = 0.f;
#pragma unroll
        for (int i = 0; i < UPLD; i++) {
            ag += unit_dot<FMT>(w.g[r][i], xv[i], w.tg);
            au += unit_dot<FMT>(w.u[r][i], xv[i], w.tu);
        }
        v[r] = ag;
        v[FPB + r] = au;
    }
    static_assert(FPB == 1 || FPB == 2 || FPB == 4, "one exchange pairs the gate and up sums");
    const float red = wave_reduce_rows<2 * FPB>(v, lane);
    const float up = xor_lane(red, FPB == 4 ? 2 : FPB == 2 ? 1 : 0);
    return silu_mul(red, up);
}

// down units of rows r0 .. r0+RB-1 of expert e: lane l holds units
// l*NDU .. l*NDU+NDU-1 of the block's RB x UF grid (one row per lane)
template <int FMT, int NDU>
struct DN {
    WUnit w[NDU];
    float ts;
};
template <int FMT, int NDU, int UF>
__device__ __forceinline__ void dn_load(DN<FMT, NDU> &d, const uint8_t *experts, const float *tscale,
                                        size_t expert_bytes, int D, int F, int e, int r0, int lane) {
    const uint8_t *eb = experts + (size_t)e * expert_bytes;
    Mat md{eb + 2 * mat_bytes<FMT>(F, D), D, F, tensor_scale<FMT>(tscale, 3 * e + 2)};
    d.ts = md.ts;
#pragma unroll
    for (int k = 0; k < NDU; k++) {
        const int q = lane * NDU + k;
        d.w[k] = load_unit<FMT>(md, r0 + q / UF, q % UF);
    }
}
// partial of row (lane*NDU)/UF from the slot's h in LDS, summed over the
// lanes of the row (all of them end with the row's sum)
template <int FMT, int NDU, int UF>
__device__ __forceinline__ float dn_dot(const DN<FMT, NDU> &d, const float *hs, int lane) {
    constexpr int UE = Unit<FMT>::E;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < NDU; k++) {
        const int u = (lane * NDU + k) % UF;
        XUnit<FMT> hv;
        const float4 *p = reinterpret_cast<const float4 *>(hs + u * UE);
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < UE / 4; c++) {
            const float4 f = p[c];
            hv.v[4 * c + 0] = f.x;
            hv.v[4 * c + 1] = f.y;
            hv.v[4 * c + 2] = f.z;
            hv.v[4 * c + 3] = f.w;
        }
        if (FMT == FMT_Q4_1) {
#pragma unroll
            for (int k2 = 0; k2 < UE; k2++) s += hv.v[k2];
        }
        hv.sum = s;
        acc += unit_dot<FMT>(d.w[k], hv, d.ts);
    }
    return group_sum<UF / NDU>(acc);
}

template <int FMT, int UPLD, int FPB, int RB, int NDU>
__global__ void __launch_bounds__(NT, 1) ps_stack(PsParams p) {
    using SH = PsShape<FMT, UPLD, FPB, RB, NDU>;
    static_assert(RB == 8, "the y gather reads 8 rows and a sum of squares per slot");
    constexpr int D = SH::D, F = SH::F, UF = SH::UF, UPLR = SH::UPLR;
    __shared__ float pool[L_POOL];
    float *xs = pool + L_X;
    float *ssq = pool + L_SSQ;
    float *lgs = pool + L_LG;
    float *part = pool + L_PART;
    const int tid = threadIdx.x, lane = tid & (MOE_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
    const int g = blockIdx.x;
    const int E = p.E, K = p.K;
    const int f0 = FPB * g, r0 = RB * g;
    u64 *const my_lg = p.mb_lg + (size_t)g * SLOT;
    u64 *const my_h = p.mb_h + (size_t)g * SLOT;
    u64 *const my_y = p.mb_y + (size_t)g * SLOT;

    // weights loaded one layer ahead (for the launch's first layer: here)
    WUnit wr[UPLR];                  // wave 7: router row g
    GU<FMT, UPLD, FPB> gs;           // wave 0: shared expert gate/up
    DN<FMT, NDU> ds;                 // wave 7: shared expert down
    {
        const PsLayer &L0 = p.layer[0];
        if (wave == W_ROUTER) {
            Mat mr{(const uint8_t *)L0.router, E, D, 1.f};
            const int row = min(g, E - 1);
#pragma unroll
            for (int i = 0; i < UPLR; i++) wr[i] = load_unit<FMT_BF16>(mr, row, lane + MOE_WAVE * i);
            dn_load<FMT, NDU, UF>(ds, L0.experts, L0.tscale, p.expert_bytes, D, F, E, r0, lane);
        } else if (wave == 0) {
            gu_load<FMT, UPLD, FPB>(gs, L0.experts, L0.tscale, p.expert_bytes, D, F, E, f0, lane);
        }
    }
    __syncthreads();

    for (int li = 0; li < p.n_layers; li++) {
        const int l = p.l0 + li;            // global layer index
        const uint32_t tag = (uint32_t)l + 1u;
        const PsLayer &LW = p.layer[li];
        // ---- x of the layer: the stack input, or the normalised y of layer l-1
        if (l == 0) {
            for (int i = tid; i < D / 4; i += NT) reinterpret_cast<float4 *>(xs)[i] = reinterpret_cast<const float4 *>(p.x0)[i];
            __syncthreads();
        } else {
            // thread t: slot t/2, words 4*(t&1) .. +3 (y rows), thread with t&1 == 0 also word 8 (sum of squares)
            const int slot = tid >> 1, half = tid & 1;
            const u64 *base = p.mb_y + (size_t)slot * SLOT;
            const u64 *a[5] = {base + 4 * half, base + 4 * half + 1, base + 4 * half + 2, base + 4 * half + 3,
                               base + (half ? 4 * half + 3 : RB)};
            u64 v[5];
            mb_poll<5>(a, v, tag - 1u, p.ctrl, p.spin);
#pragma unroll
            for (int k = 0; k < 4; k++) xs[slot * RB + 4 * half + k] = val_of(v[k]);
            if (!half) ssq[slot] = val_of(v[4]);
            __syncthreads();
            // 1 / rms from the blocks' sums of squares, summed in block order
            // (the same order in every wave of every block)
            float s4 = 0.f;
#pragma unroll
            for (int k = 0; k < NB / MOE_WAVE; k++) s4 += ssq[lane * (NB / MOE_WAVE) + k];
            const float inv = 1.0f / sqrtf(wave_sum(s4) / (float)D + 1e-6f);
            __syncthreads();
            for (int i = tid; i < D; i += NT) xs[i] *= inv;
            __syncthreads();
        }

        // ---- router logit (wave 7) and shared gate/up (wave 0)
        if (wave == W_ROUTER) {
            if (g < E) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < UPLR; i++) {
                    XUnit<FMT_BF16> xv;
                    const float4 *xp = reinterpret_cast<const float4 *>(xs + 8 * (lane + MOE_WAVE * i));
                    const float4 a0 = xp[0], a1 = xp[1];
                    xv.v[0] = a0.x; xv.v[1] = a0.y; xv.v[2] = a0.z; xv.v[3] = a0.w;
                    xv.v[4] = a1.x; xv.v[5] = a1.y; xv.v[6] = a1.z; xv.v[7] = a1.w;
                    xv.sum = 0.f;
                    acc += unit_dot<FMT_BF16>(wr[i], xv, 1.f);
                }
                float lg = wave_sum(acc);
                if (LW.bias) lg += LW.bias[g];
                if (lane == 0) mb_store(my_lg, lg, tag);
            }
            // every block's logit, into LDS for the top-k
            const u64 *a[4];
#pragma unroll
            for (int k = 0; k < 4; k++) a[k] = p.mb_lg + (size_t)min(lane + MOE_WAVE * k, E - 1) * SLOT;
            u64 v[4];
            mb_poll<4>(a, v, tag, p.ctrl, p.spin);
#pragma unroll
            for (int k = 0; k < 4; k++) lgs[lane + MOE_WAVE * k] = val_of(v[k]);
        } else if (wave == 0) {
            XUnit<FMT> xv[UPLD];
            x_units<FMT, UPLD>(xv, xs, lane);
            const float h = gu_finish<FMT, UPLD, FPB>(gs, xv, lane);
            if (lane < FPB) mb_store(my_h + lane, h, tag);
        }
        __syncthreads();
        const bool has_next = li + 1 < p.n_layers;
        const PsLayer &LN = p.layer[has_next ? li + 1 : li];

        if (wave >= 1 && wave <= K) {
            // ---- routed expert j: top-k (every such wave computes it), then its rows
            const int j = wave - 1;
            float lv[4];
#pragma unroll
            for (int k = 0; k < 4; k++) lv[k] = lgs[min(lane + MOE_WAVE * k, E - 1)];
            int es;
            float wi;
            wave_topk_regs(lv, E, K, &es, &wi);
            const int e = __builtin_amdgcn_readlane(es, j);
            const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wi), j));
            if (g == 0 && j == 0 && lane < K) {
                if (p.idx_trace) p.idx_trace[(size_t)l * K + lane] = es;
                if (p.w_trace) p.w_trace[(size_t)l * K + lane] = wi;
            }
            GU<FMT, UPLD, FPB> gw;
            DN<FMT, NDU> dw;
            gu_load<FMT, UPLD, FPB>(gw, LW.experts, LW.tscale, p.expert_bytes, D, F, e, f0, lane);
            dn_load<FMT, NDU, UF>(dw, LW.experts, LW.tscale, p.expert_bytes, D, F, e, r0, lane);
            XUnit<FMT> xv[UPLD];
            x_units<FMT, UPLD>(xv, xs, lane);
            const float h = gu_finish<FMT, UPLD, FPB>(gw, xv, lane);
            if (lane < FPB) mb_store(my_h + FPB * wave + lane, h, tag);
            // the slot's h from every block
            float *hs = pool + L_H + wave * 1024;
            {
                const u64 *a[4 * FPB];
#pragma unroll
                for (int k = 0; k < 4; k++)
#pragma unroll
                    for (int q = 0; q < FPB; q++)
                        a[FPB * k + q] = p.mb_h + (size_t)(lane + MOE_WAVE * k) * SLOT + FPB * wave + q;
                u64 v[4 * FPB];
                mb_poll<4 * FPB>(a, v, tag, p.ctrl, p.spin);
#pragma unroll
                for (int k = 0; k < 4; k++)
#pragma unroll
                    for (int q = 0; q < FPB; q++) hs[FPB * (lane + MOE_WAVE * k) + q] = val_of(v[FPB * k + q]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const float rs = dn_dot<FMT, NDU, UF>(dw, hs, lane);
            if ((lane * NDU) % UF == 0) part[wave * 16 + (lane * NDU) / UF] = c * rs;
        } else if (wave == W_ROUTER) {
            // ---- shared expert down (slot 0), then next layer's router row and shared down
            float *hs = pool + L_H;
            {
                const u64 *a[4 * FPB];
#pragma unroll
                for (int k = 0; k < 4; k++)
#pragma unroll
                    for (int q = 0; q < FPB; q++) a[FPB * k + q] = p.mb_h + (size_t)(lane + MOE_WAVE * k) * SLOT + q;
                u64 v[4 * FPB];
                mb_poll<4 * FPB>(a, v, tag, p.ctrl, p.spin);
#pragma unroll
                for (int k = 0; k < 4; k++)
#pragma unroll
                    for (int q = 0; q < FPB; q++) hs[FPB * (lane + MOE_WAVE * k) + q] = val_of(v[FPB * k + q]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const float rs = dn_dot<FMT, NDU, UF>(ds, hs, lane);
            if ((lane * NDU) % UF == 0) part[0 * 16 + (lane * NDU) / UF] = rs;
            if (has_next) {
                Mat mr{(const uint8_t *)LN.router, E, D, 1.f};
                const int row = min(g, E - 1);
#pragma unroll
                for (int i = 0; i < UPLR; i++) wr[i] = load_unit<FMT_BF16>(mr, row, lane + MOE_WAVE * i);
                dn_load<FMT, NDU, UF>(ds, LN.experts, LN.tscale, p.expert_bytes, D, F, E, r0, lane);
            }
        } else if (wave == 0) {
            if (has_next) gu_load<FMT, UPLD, FPB>(gs, LN.experts, LN.tscale, p.expert_bytes, D, F, E, f0, lane);
        }
        __syncthreads();

        // ---- output rows r0 .. r0+RB-1: slots summed in order (shared, then selection order)
        if (tid < RB) {
            float y = part[tid];
            for (int a2 = 1; a2 <= K; a2++) y += part[a2 * 16 + tid];
            xs[tid] = y;  // x of this layer is no longer read (all waves passed the barrier)
            if (p.y_trace) p.y_trace[(size_t)l * D + r0 + tid] = y;
            if (l == p.last_layer && p.y) p.y[r0 + tid] = y;
            mb_store(my_y + tid, y, tag);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (tid == 0) {
            float s = 0.f;
            for (int r = 0; r < RB; r++) s = __builtin_fmaf(xs[r], xs[r], s);
            mb_store(my_y + RB, s, tag);
        }
        __syncthreads();
    }
    // after an abort the results are meaningless: NaN in this block's rows of
    // the output (every block gets here, the flag is raised for good)
    if (tid < RB && ctrl_load(p.ctrl) != 0u) {
        if (p.y) p.y[r0 + tid] = __builtin_nanf("");
        if (p.y_trace) p.y_trace[(size_t)(p.l0 + p.n_layers - 1) * D + r0 + tid] = __builtin_nanf("");
    }
}

// clears the mailboxes and the control words before a call
__global__ void __launch_bounds__(256) ps_clear(PsParams p) {
    const int n = 3 * NB * SLOT;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p.mb_lg[i] = 0ull;
    if (blockIdx.x == 0 && threadIdx.x < 64) p.ctrl[threadIdx.x] = 0u;
}

template <int FMT, int UPLD, int FPB, int RB, int NDU>
hipError_t ps_launch_fmt(const PsParams &p, hipStream_t st, hipEvent_t *ev) {
    auto kern = ps_stack<FMT, UPLD, FPB, RB, NDU>;
    if (ev)
        hipExtLaunchKernelGGL(kern, dim3(NB), dim3(NT), 0, st, ev[0], ev[1], 0, p);
    else
        hipLaunchKernelGGL(kern, dim3(NB), dim3(NT), 0, st, p);
    return hipGetLastError();
}

template <int FMT, int UPLD, int FPB, int RB, int NDU>
bool ps_occupancy_ok() {
    static int ok = -1;
    if (ok < 0) {
        int dev = 0, cus = 0, nb = 0;
        ok = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void *>(&ps_stack<FMT, UPLD, FPB, RB, NDU>),
                                                         NT, 0) == hipSuccess)
            ok = (nb >= 1 && cus >= NB) ? 1 : 0;
        (void)hipGetLastError();
    }
    return ok == 1;
}

}  // namespace

bool ps_supported(int fmt, int D, int F, int E, int S, int K) {
    if (S != 1 || K < 1 || K > NW - 2 || E < K || E > NB) return false;
    if (fmt == FMT_Q4_1 && D == 2048 && F == 512) return ps_occupancy_ok<FMT_Q4_1, 1, 2, 8, 2>();
    if (fmt == FMT_NVFP4 && D == 2048 && F == 512) return ps_occupancy_ok<FMT_NVFP4, 1, 2, 8, 2>();
    return false;
}

hipError_t ps_clear_launch(const PsParams &p, hipStream_t st, hipEvent_t *ev) {
    if (ev)
        hipExtLaunchKernelGGL(ps_clear, dim3(48), dim3(256), 0, st, ev[0], ev[1], 0, p);
    else
        hipLaunchKernelGGL(ps_clear, dim3(48), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t ps_launch(const PsParams &p, int fmt, hipStream_t st, hipEvent_t *ev) {
    if (p.n_layers < 1 || p.n_layers > PS_MAX_LAYERS) return hipErrorInvalidValue;
    if (fmt == FMT_Q4_1 && p.D == 2048 && p.F == 512) return ps_launch_fmt<FMT_Q4_1, 1, 2, 8, 2>(p, st, ev);
    if (fmt == FMT_NVFP4 && p.D == 2048 && p.F == 512) return ps_launch_fmt<FMT_NVFP4, 1, 2, 8, 2>(p, st, ev);
    return hipErrorNotSupported;
}

}  // namespace moe
