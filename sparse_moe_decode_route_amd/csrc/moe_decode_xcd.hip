// Batch-1 decode, one kernel per layer, each XCD running one active expert.
//
// Decode is bound by moving weights ("Recursive Flint 40B-A2.5B",
// orcarouter.ai blog, section "The architecture is a memory-bandwidth
// argument": 6 of 256 routed experts plus one shared expert per token), and at
// batch 1 a layer's 13.8 MB take under 2 us of HBM time, so the layer's cost is
// its chain of dependencies: all of x before any logit, all logits before the
// top-k, all of h before any output row.  The three-kernel path crosses each of
// them with a kernel boundary, because blocks on different XCDs (each with its
// own L2) see each other's stores only after a cache writeback.  Here each
// dependency but the last stays inside one XCD:
//
//   * the 8 XCDs take one expert each: XCD j < K the routed expert of rank j,
//     XCDs K.. one part of the shared expert's features each;
//   * every routed XCD computes all 256 logits itself (32 blocks x 8 router
//     rows) and passes them to its own blocks through its L2;
//   * each XCD computes h of its expert and, after an XCD-local barrier, its
//     expert's whole down projection: a partial output y_x per XCD;
//   * the next layer's kernel adds the 8 partials (in XCD order) and applies
//     the RMSNorm: the only cross-XCD step, at the kernel boundary.
//
// XCD-local barriers go through L2 atomics without cache maintenance.  Each
// arrival carries the block's XCC id; a barrier whose arrivals came from
// another XCC than the waiting block's (blocks not placed round-robin on the
// XCDs), or that waits longer than its limit (20 ms), sets the error word and makes the
// block write NaN, so a broken exchange never passes stale values or hangs.
#include <hip/hip_fp16.h>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_xcd.h"

namespace moe {

XlWs xl_ws(int D, int F, int E) {
    XlWs L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += (bytes + 255) & ~(size_t)255;
        return at;
    };
    L.ypart0 = take((size_t)XL_XCDS * D * 4);
    L.ypart1 = take((size_t)XL_XCDS * D * 4);
    L.lg = take((size_t)XL_XCDS * E * 4);
    L.hb = take((size_t)XL_XCDS * F * 4);
    L.bar = take((size_t)XL_MAX_LAYERS * 2 * XL_XCDS * XL_LINE * 4);
    L.total = o;
    return L;
}

namespace {

constexpr int XL_D = 2048, XL_F = 512, XL_E = 256, XL_K = 6;
constexpr int XL_THREADS = MOE_WAVE * XL_WAVES;
constexpr int XL_ID_SHIFT = 8;               // barrier word: arrivals below, sum of XCC ids above

__device__ __forceinline__ int xl_xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15; }  // HW_REG_XCC_ID

// Barrier of the n blocks of one XCD on counter ctr.  Every wave's stores have
// reached L2 before the block arrives; thread 0 then polls the counter with
// L1-bypassing loads for at most spin ticks of the 100 MHz real-time counter.
// Returns nonzero (in every thread) if the wait gave up or an arrival came from
// another XCC.
__device__ __forceinline__ int xl_barrier(int32_t *ctr, int n, uint32_t spin) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int bad = 0;
    if (threadIdx.x == 0) {
        const int id = xl_xcc_id();
        __hip_atomic_fetch_add(ctr, 1 + (id << XL_ID_SHIFT), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        int v;
        while (((v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) & ((1 << XL_ID_SHIFT) - 1)) <
               n) {
            if (__builtin_amdgcn_s_memrealtime() - t0 > spin) {
                bad = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if ((v >> XL_ID_SHIFT) != n * id) bad = 1;
    }
    return __syncthreads_or(bad);
}

// x of the 4-bit dot from the LDS copy: lane l holds elements 32l .. 32l + 31.
template <int FMT>
__device__ __forceinline__ void xl_x4(XUnit<FMT> &xv, const float4 *xs4, int lane) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float4 f = xs4[8 * lane + i];
        xv.v[4 * i + 0] = f.x;
        xv.v[4 * i + 1] = f.y;
        xv.v[4 * i + 2] = f.z;
        xv.v[4 * i + 3] = f.w;
    }
    float s = 0.f;
    if (FMT == FMT_Q4_1) {
#pragma unroll
        for (int i = 0; i < 32; i++) s += xv.v[i];
    }
    xv.sum = s;
}

// h[f0 + r] (r < RG) of expert e from issued gate/up loads: one halving
// reduction of the RG gate and RG up sums, silu(g) * u in lanes r < RG.
template <int FMT, int RG>
__device__ __forceinline__ void xl_gateup(const WUnit (&wg)[RG], const WUnit (&wu)[RG], float tsg, float tsu,
                                          const XUnit<FMT> &xv, float *hdst, int lane) {
    float v[2 * RG];
#pragma unroll
    for (int r = 0; r < RG; r++) {
        v[r] = unit_dot<FMT>(wg[r], xv, tsg);
        v[RG + r] = unit_dot<FMT>(wu[r], xv, tsu);
    }
    const float red = wave_reduce_rows<2 * RG>(v, lane);
    const float up = xor_lane(red, RG == 2 ? 1 : 0);  // lane ^ RG
    if (lane < RG) hdst[lane] = silu_mul(red, up);
}

// Partial down rows of one expert: LPR lanes per row (one 32-feature unit
// each), RR rows per lane group; h of the expert's feature slice from hsrc.
template <int FMT, int LPR, int RR>
__device__ __forceinline__ void xl_down(const WUnit (&wd)[RR], float ts, const float *hsrc, float coef, float *ydst,
                                        int lane) {
    const int sub = lane % LPR;
    XUnit<FMT> hv;
    const float4 *h4 = reinterpret_cast<const float4 *>(hsrc) + 8 * sub;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float4 f = h4[i];
        hv.v[4 * i + 0] = f.x;
        hv.v[4 * i + 1] = f.y;
        hv.v[4 * i + 2] = f.z;
        hv.v[4 * i + 3] = f.w;
    }
    float s = 0.f;
    if (FMT == FMT_Q4_1) {
#pragma unroll
        for (int i = 0; i < 32; i++) s += hv.v[i];
    }
    hv.sum = s;
#pragma unroll
    for (int r = 0; r < RR; r++) {
        const float t = group_sum<LPR>(unit_dot<FMT>(wd[r], hv, ts));
        if (sub == 0) ydst[r] = coef * t;
    }
}

template <int FMT>
__global__ void __launch_bounds__(XL_THREADS) xl_layer(XlParams p) {
    __shared__ float4 xs4[XL_D / 4];
    __shared__ float red[XL_WAVES];
    const int tid = threadIdx.x, lane = tid & (MOE_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int xcd = blockIdx.x % XL_XCDS, q = blockIdx.x / XL_XCDS;
    constexpr int NSH = XL_XCDS - XL_K;      // XCDs sharing the shared expert
    constexpr int FSH = XL_F / NSH;          // its features per XCD
    const bool shared = xcd >= XL_K;
    const uint8_t *exp_sh = p.experts + (size_t)XL_E * p.expert_bytes;
    const size_t MB = mat_bytes<FMT>(XL_F, XL_D);  // bytes of one matrix
    int bad = 0;

    // ---- the shared expert's XCDs: every weight load goes out first ----
    // features f_lo + 8q + wave (one per wave), down rows 64q + 8 wave + grp
    // (8 lanes per row over the FSH features)
    WUnit sg[1], su[1], sd[1];
    float sts_g = 1.f, sts_u = 1.f, sts_d = 1.f;
    // ---- routed XCDs: the router rows first (8q + wave) ----
    WUnit wr[XL_D / 512];
    if (shared) {
        const int f_lo = (xcd - XL_K) * FSH;
        const int f = f_lo + 8 * q + wave;
        Mat mg{exp_sh, XL_F, XL_D, tensor_scale<FMT>(p.tscale, 3 * XL_E + 0)};
        Mat mu{exp_sh + MB, XL_F, XL_D, tensor_scale<FMT>(p.tscale, 3 * XL_E + 1)};
        Mat md{exp_sh + 2 * MB, XL_D, XL_F, tensor_scale<FMT>(p.tscale, 3 * XL_E + 2)};
        sts_g = mg.ts;
        sts_u = mu.ts;
        sts_d = md.ts;
        sg[0] = load_unit<FMT>(mg, f, lane);
        su[0] = load_unit<FMT>(mu, f, lane);
        sd[0] = load_unit<FMT>(md, 64 * q + 8 * wave + lane / 8, f_lo / 32 + lane % 8);
    } else {
        Mat mr{(const uint8_t *)p.router, XL_E, XL_D, 1.f};
#pragma unroll
        for (int i = 0; i < XL_D / 512; i++) wr[i] = load_unit<FMT_BF16>(mr, 8 * q + wave, lane + MOE_WAVE * i);
    }
    // ---- x: the previous layer's partial outputs summed in XCD order, then
    //      RMSNorm (or the stack's input) into LDS; thread t owns float4 t ----
    {
        float4 y4;
        if (p.first) {
            y4 = reinterpret_cast<const float4 *>(p.x0)[tid];
        } else {
            float4 a[XL_XCDS];
#pragma unroll
            for (int s = 0; s < XL_XCDS; s++) a[s] = reinterpret_cast<const float4 *>(p.yin + (size_t)s * XL_D)[tid];
            y4 = a[0];
#pragma unroll
            for (int s = 1; s < XL_XCDS; s++) {
                y4.x += a[s].x;
                y4.y += a[s].y;
                y4.z += a[s].z;
                y4.w += a[s].w;
            }
            if (p.y_prev && blockIdx.x == 0) reinterpret_cast<float4 *>(p.y_prev)[tid] = y4;
        }
        __builtin_amdgcn_sched_barrier(0);
        float inv = 1.f;
        if (!p.first) {
            float ss = y4.x * y4.x;
            ss = __builtin_fmaf(y4.y, y4.y, ss);
            ss = __builtin_fmaf(y4.z, y4.z, ss);
            ss = __builtin_fmaf(y4.w, y4.w, ss);
            ss = wave_sum(ss);
            if (lane == 0) red[wave] = ss;
            __syncthreads();
            float tot = red[0];
#pragma unroll
            for (int w = 1; w < XL_WAVES; w++) tot += red[w];
            inv = 1.0f / sqrtf(tot / (float)XL_D + 1e-6f);
        }
        xs4[tid] = make_float4(y4.x * inv, y4.y * inv, y4.z * inv, y4.w * inv);
        __syncthreads();
    }

    float *ydst;
    if (shared) {
        // ---- shared expert: h of its features, then its partial down rows ----
        XUnit<FMT> xv;
        xl_x4<FMT>(xv, xs4, lane);
        float *hx = p.hb + (size_t)xcd * XL_F;
        xl_gateup<FMT, 1>(sg, su, sts_g, sts_u, xv, hx + 8 * q + wave, lane);
        bad |= xl_barrier(p.bar + (XL_XCDS + xcd) * XL_LINE, XL_BPX, p.spin);
        ydst = p.yout + (size_t)xcd * XL_D + 64 * q + 8 * wave + lane / 8;
        xl_down<FMT, 8, 1>(sd, sts_d, hx, bad ? __builtin_nanf("") : 1.f, ydst, lane);
    } else {
        // ---- routed XCD: 8 logits per block, all 256 through this XCD's L2 ----
        {
            XUnit<FMT_BF16> xb;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < XL_D / 512; i++) {
                const float4 a = xs4[2 * (lane + MOE_WAVE * i)], b = xs4[2 * (lane + MOE_WAVE * i) + 1];
                xb.v[0] = a.x;
                xb.v[1] = a.y;
                xb.v[2] = a.z;
                xb.v[3] = a.w;
                xb.v[4] = b.x;
                xb.v[5] = b.y;
                xb.v[6] = b.z;
                xb.v[7] = b.w;
                xb.sum = 0.f;
                acc += unit_dot<FMT_BF16>(wr[i], xb, 1.f);
            }
            const float s = wave_sum(acc);
            const int e = 8 * q + wave;
            if (lane == 0) p.lg[(size_t)xcd * XL_E + e] = p.bias ? s + p.bias[e] : s;
        }
        bad |= xl_barrier(p.bar + xcd * XL_LINE, XL_BPX, p.spin);
        // ---- top-k in every wave; this XCD's expert is rank xcd ----
        float lv[4];
        wave_topk_load(p.lg + (size_t)xcd * XL_E, XL_E, lv);
        int es;
        float wi;
        wave_topk_regs(lv, XL_E, p.K, &es, &wi);
        const int e = __builtin_amdgcn_readlane(es, xcd);
        const float coef = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wi), xcd));
        if (xcd == 0 && q == 0 && wave == 0 && lane < p.K) {
            if (p.idx_out) p.idx_out[lane] = es;
            if (p.w_out) p.w_out[lane] = wi;
        }
        // ---- its weights: features 16q + 2 wave + r, down rows 64q + 8 wave +
        //      2 (lane / 16) + r (16 lanes per row) ----
        const uint8_t *eb = p.experts + (size_t)e * p.expert_bytes;
        Mat mg{eb, XL_F, XL_D, tensor_scale<FMT>(p.tscale, 3 * e + 0)};
        Mat mu{eb + MB, XL_F, XL_D, tensor_scale<FMT>(p.tscale, 3 * e + 1)};
        Mat md{eb + 2 * MB, XL_D, XL_F, tensor_scale<FMT>(p.tscale, 3 * e + 2)};
        const int f0 = 16 * q + 2 * wave;
        const int r0 = 64 * q + 8 * wave + 2 * (lane / 16);
        WUnit wg[2], wu[2], wd[2];
#pragma unroll
        for (int r = 0; r < 2; r++) {
            wg[r] = load_unit<FMT>(mg, f0 + r, lane);
            wu[r] = load_unit<FMT>(mu, f0 + r, lane);
        }
#pragma unroll
        for (int r = 0; r < 2; r++) wd[r] = load_unit<FMT>(md, r0 + r, lane % 16);
        XUnit<FMT> xv;
        xl_x4<FMT>(xv, xs4, lane);
        __builtin_amdgcn_sched_barrier(0);
        float *hx = p.hb + (size_t)xcd * XL_F;
        xl_gateup<FMT, 2>(wg, wu, mg.ts, mu.ts, xv, hx + f0, lane);
        bad |= xl_barrier(p.bar + (XL_XCDS + xcd) * XL_LINE, XL_BPX, p.spin);
        ydst = p.yout + (size_t)xcd * XL_D + r0;
        xl_down<FMT, 16, 2>(wd, md.ts, hx, bad ? __builtin_nanf("") : coef, ydst, lane);
    }
    if (bad && tid == 0) *p.err = 1;
}

__global__ void __launch_bounds__(1024) xl_clear(int32_t *bar, int n, int32_t *err, int clear_err) {
    for (int i = blockIdx.x * 1024 + threadIdx.x; i < n; i += gridDim.x * 1024) bar[i] = 0;
    if (clear_err && blockIdx.x == 0 && threadIdx.x == 0) *err = 0;
}

__global__ void __launch_bounds__(256) xl_reduce(const float *ypart, float *y, int D4) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= D4) return;
    float4 s = reinterpret_cast<const float4 *>(ypart)[i];
#pragma unroll
    for (int x = 1; x < XL_XCDS; x++) {
        const float4 a = reinterpret_cast<const float4 *>(ypart)[(size_t)x * D4 + i];
        s.x += a.x;
        s.y += a.y;
        s.z += a.z;
        s.w += a.w;
    }
    reinterpret_cast<float4 *>(y)[i] = s;
}

template <typename K, typename... A>
hipError_t xl_launch(K kern, dim3 grid, dim3 block, hipStream_t st, hipEvent_t *ev, A... args) {
    if (ev)
        hipExtLaunchKernelGGL(kern, grid, block, 0, st, ev[0], ev[1], 0, args...);
    else
        hipLaunchKernelGGL(kern, grid, block, 0, st, args...);
    return hipGetLastError();
}

}  // namespace

bool xl_supported(int fmt, int D, int F, int E, int S, int K) {
    if ((fmt != FMT_Q4_1 && fmt != FMT_NVFP4) || D != XL_D || F != XL_F || E != XL_E || S != 1 || K != XL_K)
        return false;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    // the device query once per (device, format): 0 unknown, 1 yes, 2 no
    static std::atomic<int> known[64][2];
    const int slot = fmt == FMT_Q4_1 ? 0 : 1;
    if (dev >= 0 && dev < 64) {
        const int k = known[dev][slot].load(std::memory_order_relaxed);
        if (k) return k == 1;
    }
    int cus = 0, nb = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    const hipError_t e = fmt == FMT_Q4_1
                             ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, xl_layer<FMT_Q4_1>, XL_THREADS, 0)
                             : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, xl_layer<FMT_NVFP4>, XL_THREADS, 0);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    // every block of the grid resident at once, 32 per XCD
    const bool ok = cus == XL_BLOCKS && nb >= 1;
    if (dev >= 0 && dev < 64) known[dev][slot].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok;
}

hipError_t xl_clear_launch(int32_t *bar, int32_t *err, bool clear_err, hipStream_t st, hipEvent_t *ev) {
    const int n = XL_MAX_LAYERS * 2 * XL_XCDS * XL_LINE;
    return xl_launch(xl_clear, dim3(8), dim3(1024), st, ev, bar, n, err, clear_err ? 1 : 0);
}

hipError_t xl_layer_launch(const XlParams &p, int fmt, hipStream_t st, hipEvent_t *ev) {
    if (fmt == FMT_Q4_1) return xl_launch(xl_layer<FMT_Q4_1>, dim3(XL_BLOCKS), dim3(XL_THREADS), st, ev, p);
    return xl_launch(xl_layer<FMT_NVFP4>, dim3(XL_BLOCKS), dim3(XL_THREADS), st, ev, p);
}

hipError_t xl_reduce_launch(const float *ypart, float *y, int D, hipStream_t st, hipEvent_t *ev) {
    const int D4 = D / 4;
    return xl_launch(xl_reduce, dim3((D4 + 255) / 256), dim3(256), st, ev, ypart, y, D4);
}

}  // namespace moe
