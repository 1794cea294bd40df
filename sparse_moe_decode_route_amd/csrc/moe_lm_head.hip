// Output layer (lm_head) at decode: logits[t, v] = x_t . W[v, :] over a
// 4-bit (q4_1, NVFP4) or bf16 matrix W [V, D] in the device layout.
//
// What it computes: "Recursive Flint 40B-A2.5B" (orcarouter.ai blog),
// section "The quantisation recipe is the most transferable part": the
// output layer ships in 4 bits, because with 2.5 B active parameters it is
// a large share of the weights that every decoded token reads.
//
// The matrix is read once per call, in full, so the kernel is a stream:
//   - one wave owns a tile of 16 or 32 consecutive rows and keeps the
//     tokens' activations for its lanes' columns in registers for the tile;
//   - a row is read by the whole wave at once (lane l takes units l, l+64,
//     ...: for q4_1 / NVFP4 at D = 2048 one 1 KB coalesced load of codes and
//     one 256 B / 128 B load of scales), the next group of rows is in flight
//     while the current one is reduced;
//   - the partial sums of a group of rows are added across the wave in a
//     fixed order (DPP and swizzles, each level halving the values a lane
//     carries), and lane j of the wave keeps row j's logit, so a tile's
//     logits leave in one coalesced store per token.
// Tokens beyond TG per wave are split into groups that re-read the same
// tile; the groups of one tile are placed on the same XCD (blocks b and b+8
// share one), so the second read is served from that XCD's L2.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {


// fp32 activations of unit u of one token (widened from bf16 if act == 1),
// with their in-order sum for q4_1 (same order as the unit dot below).
template <int FMT>
__device__ __forceinline__ void lm_load_x(XUnit<FMT> &x, const void *src, int act, int u) {
    constexpr int E = Unit<FMT>::E;
    if (act == 0) {
        load_x<FMT>(x, static_cast<const float *>(src), u);
        return;
    }
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + (size_t)u * E);
#pragma unroll
    for (int i = 0; i < E / 8; i++) {
        const uint4 v = p[i];
        const uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            x.v[8 * i + 2 * j] = bf16lo(a[j]);
            x.v[8 * i + 2 * j + 1] = bf16hi(a[j]);
        }
    }
    float s = 0.f;
    if (FMT == FMT_Q4_1) {
#pragma unroll
        for (int i = 0; i < E; i++) s += x.v[i];
    }
    x.sum = s;
}

// Raw buffer resource over [base, base + bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t lm_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int LM_NT = 2;  // non-temporal: the matrix is streamed once

// dot of one weight unit with NT tokens' activations: each weight is decoded
// once and multiplied into every token's sum.  q_inv undoes the scale of the
// 8-bit float conversion that turns q4_1 codes into floats (below).
template <int FMT, int NT>
__device__ __forceinline__ void unit_dot_multi(const WUnit &w, const XUnit<FMT> (&x)[NT], float ts, float q_inv,
                                               float (&r)[NT]) {
    const uint32_t a[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
    if constexpr (FMT == FMT_BF16) {
        float s[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) s[t] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float lo = bf16lo(a[i]), hi = bf16hi(a[i]);
#pragma unroll
            for (int t = 0; t < NT; t++) {
                s[t] = __builtin_fmaf(lo, x[t].v[2 * i], s[t]);
                s[t] = __builtin_fmaf(hi, x[t].v[2 * i + 1], s[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; t++) r[t] = s[t];
    } else if constexpr (FMT == FMT_Q4_1) {
        // sum_i (d q_i + m) x_i = d * sum_i q_i x_i + m * sum_i x_i.  A byte
        // holding a code q < 16 is, read as an E4M3 float, the subnormal or
        // first-binade value q * 2^-9 (exact), so one packed conversion turns
        // two codes into floats; the power of two is folded into d.
        float s0[NT], s1[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) s0[t] = s1[t] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t lo = a[i] & 0x0F0F0F0Fu, hi = (a[i] >> 4) & 0x0F0F0F0Fu;
            const auto l01 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
            const auto l23 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
            const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
            const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
            const float ql[4] = {l01[0], l01[1], l23[0], l23[1]}, qh[4] = {h01[0], h01[1], h23[0], h23[1]};
#pragma unroll
            for (int b = 0; b < 4; b++)
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    s0[t] = __builtin_fmaf(ql[b], x[t].v[4 * i + b], s0[t]);
                    s1[t] = __builtin_fmaf(qh[b], x[t].v[16 + 4 * i + b], s1[t]);
                }
        }
        const float d = half_bits_to_float(w.s) * q_inv, m = half_bits_to_float(w.s >> 16);
#pragma unroll
        for (int t = 0; t < NT; t++) r[t] = __builtin_fmaf(d, s0[t] + s1[t], m * x[t].sum);
    } else {
        // two blocks of 16 e2m1 codes, each with its E4M3 scale
        float s[NT][2];
#pragma unroll
        for (int t = 0; t < NT; t++) s[t][0] = s[t][1] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 0);
            const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 1);
            const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 2);
            const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 3);
            const float v[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
            for (int j = 0; j < 8; j++)
#pragma unroll
                for (int t = 0; t < NT; t++) s[t][i >> 1] = __builtin_fmaf(v[j], x[t].v[8 * i + j], s[t][i >> 1]);
        }
        const float b0 = e4m3_to_float(w.s & 0xFFu), b1 = e4m3_to_float((w.s >> 8) & 0xFFu);
#pragma unroll
        for (int t = 0; t < NT; t++) r[t] = ts * __builtin_fmaf(b0, s[t][0], b1 * s[t][1]);
    }
}

template <int FMT> constexpr int lm_scale_bytes() { return FMT == FMT_Q4_1 ? 4 : FMT == FMT_NVFP4 ? 2 : 0; }

// XR = activations per token per lane (32 or 64: D <= 2048 or <= 4096), TG =
// tokens per wave, FULL: D fills every lane's units (no unit guard), RT rows
// per tile (one wave, RT <= 64).  UPL units per lane; P rows per load group
// (UPL * P = 8 unit loads per group, 4 for three tokens per wave and for
// NVFP4 at four); two groups in registers, the next one loading while the
// current one is reduced.
template <int FMT, int XR, int TG, bool FULL, int RT>
__global__ __launch_bounds__(64) void lm_head_kernel(LmHeadArgs p) {
    constexpr int E = Unit<FMT>::E;
    constexpr int UPL = XR / E;
    // halved groups where the tokens' registers leave too little room (measured)
    constexpr int PDIV = (TG == 3 || (FMT == FMT_NVFP4 && TG == 4)) ? 2 : 1;
    constexpr int P = UPL >= 8 ? 1 : 8 / UPL / PDIV > 0 ? 8 / UPL / PDIV : 1;
    constexpr int NGR = RT / P;
    static_assert(RT <= 64 && NGR % 2 == 0, "tile of at most 64 rows, an even number of groups");
    constexpr int SB = lm_scale_bytes<FMT>();
    const int lane = threadIdx.x;
    const int G = p.n_groups;
    const int b = blockIdx.x;
    const int tg = (b >> 3) % G;
    const int tile = (b & 7) + 8 * ((b >> 3) / G);
    if (tile >= p.n_tiles) return;
    const int t0 = tg * TG;
    const int nt = min(TG, p.T - t0);
    const int U = p.D / E;
    const float ts = FMT == FMT_NVFP4 ? *p.tscale : 1.f;
    const float q_inv = FMT == FMT_Q4_1 ? 1.0f / __builtin_amdgcn_cvt_pk_f32_fp8(1u, false)[0] : 1.f;
    const size_t xrow_bytes = (size_t)p.D * (p.act ? 2 : 4);

    XUnit<FMT> xu[UPL][TG];
#pragma unroll
    for (int i = 0; i < UPL; i++) {
        const int u = lane + 64 * i;
#pragma unroll
        for (int t = 0; t < TG; t++) {
            if ((FULL || u < U) && t < nt) {
                lm_load_x<FMT>(xu[i][t], static_cast<const char *>(p.x) + (size_t)(t0 + t) * xrow_bytes, p.act, u);
            } else {
#pragma unroll
                for (int e = 0; e < E; e++) xu[i][t].v[e] = 0.f;
                xu[i][t].sum = 0.f;
            }
        }
    }

    // this tile's rows of the code plane [V, U * 16 B] and of the scale plane
    // [V, U * SB B]; rows past the last are read as the last row
    const int r0 = tile * RT;
    const int last = min(RT, p.V - r0) - 1;
    const uint32_t cstride = (uint32_t)U * 16u, sstride = (uint32_t)U * SB;
    const __amdgpu_buffer_rsrc_t rc = lm_rsrc(p.w + (size_t)r0 * cstride, (uint32_t)(last + 1) * cstride);
    const __amdgpu_buffer_rsrc_t rs =
        lm_rsrc(p.w + (size_t)p.V * cstride + (size_t)r0 * sstride, (uint32_t)(last + 1) * sstride);
    auto issue = [&](WUnit (&dst)[P][UPL], int g) {
#pragma unroll
        for (int j = 0; j < P; j++) {
            const int row = min(g * P + j, last);
#pragma unroll
            for (int i = 0; i < UPL; i++) {
                const int u = lane + 64 * i;
                if (FULL || u < U) {
                    const auto c = __builtin_amdgcn_raw_buffer_load_b128(rc, u * 16, row * (int)cstride, LM_NT);
                    dst[j][i].c = make_uint4(c[0], c[1], c[2], c[3]);
                    if constexpr (SB == 4)
                        dst[j][i].s = __builtin_amdgcn_raw_buffer_load_b32(rs, u * 4, row * (int)sstride, LM_NT);
                    else if constexpr (SB == 2)
                        dst[j][i].s = __builtin_amdgcn_raw_buffer_load_b16(rs, u * 2, row * (int)sstride, LM_NT);
                    else
                        dst[j][i].s = 0;
                }
            }
        }
    };

    float out[TG];
#pragma unroll
    for (int t = 0; t < TG; t++) out[t] = 0.f;
    auto reduce = [&](const WUnit (&src)[P][UPL], int g) {
        float part[TG][P];
#pragma unroll
        for (int j = 0; j < P; j++) {
#pragma unroll
            for (int t = 0; t < TG; t++) part[t][j] = 0.f;
#pragma unroll
            for (int i = 0; i < UPL; i++) {
                if (FULL || lane + 64 * i < U) {
                    float r[TG];
                    unit_dot_multi<FMT, TG>(src[j][i], xu[i], ts, q_inv, r);
#pragma unroll
                    for (int t = 0; t < TG; t++) part[t][j] += r[t];
                }
            }
        }
        const bool mine = lane / P == g;  // lane l keeps row l of the tile
#pragma unroll
        for (int t = 0; t < TG; t++) {
            const float s = wave_reduce_rows<P>(part[t], lane);
            out[t] = mine ? s : out[t];
        }
    };

    WUnit b0[P][UPL], b1[P][UPL];
    issue(b0, 0);
    for (int g = 0; g < NGR; g += 2) {
        issue(b1, g + 1);
        reduce(b0, g);
        if (g + 2 < NGR) issue(b0, g + 2);
        reduce(b1, g + 1);
    }
    if (lane <= last) {
#pragma unroll
        for (int t = 0; t < TG; t++)
            if (t < nt) p.logits[(size_t)(t0 + t) * p.V + r0 + lane] = out[t];
    }
}

// Tiles of 16 rows for one or two tokens per wave (many short waves keep
// more rows in flight per CU), of 32 rows for more tokens (their register
// footprint limits occupancy; the longer waves amortise the activations).
template <int FMT, int XR, int TG>
hipError_t launch_one(const LmHeadArgs &a, hipStream_t st) {
    constexpr int RT = TG <= 2 ? 16 : 32;
    LmHeadArgs p = a;
    p.n_tiles = (a.V + RT - 1) / RT;
    p.n_groups = (a.T + TG - 1) / TG;
    const unsigned grid = 8u * (unsigned)p.n_groups * (unsigned)((p.n_tiles + 7) / 8);
    const bool full = a.D == XR * 64;
    auto kern = full ? lm_head_kernel<FMT, XR, TG, true, RT> : lm_head_kernel<FMT, XR, TG, false, RT>;
    if (a.ev0)
        hipExtLaunchKernelGGL(kern, dim3(grid), dim3(64), 0, st, a.ev0, a.ev1, 0, p);
    else
        hipLaunchKernelGGL(kern, dim3(grid), dim3(64), 0, st, p);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const LmHeadArgs &a, hipStream_t st) {
    if (a.D <= 2048) {
        if (a.T == 1) return launch_one<FMT, 32, 1>(a, st);
        if (a.T == 2) return launch_one<FMT, 32, 2>(a, st);
        if (a.T == 3 || a.T == 5 || a.T == 6) return launch_one<FMT, 32, 3>(a, st);
        return launch_one<FMT, 32, 4>(a, st);
    }
    if (a.T == 1) return launch_one<FMT, 64, 1>(a, st);
    return launch_one<FMT, 64, 2>(a, st);
}

}  // namespace

hipError_t launch_lm_head(const LmHeadArgs &a, hipStream_t st) {
    if (a.fmt == FMT_Q4_1) return launch_fmt<FMT_Q4_1>(a, st);
    if (a.fmt == FMT_NVFP4) return launch_fmt<FMT_NVFP4>(a, st);
    return launch_fmt<FMT_BF16>(a, st);
}

}  // namespace moe
