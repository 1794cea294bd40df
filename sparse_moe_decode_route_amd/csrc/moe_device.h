// Device helpers for libmoe (gfx950, wave64): weight-unit decoding and
// wave reductions.  Formats as defined by the device layout in moe.h.
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

namespace moe {

enum { FMT_BF16 = 0, FMT_Q4_1 = 1, FMT_NVFP4 = 2 };

// Hide a value's provenance from the optimiser so that byte extraction after
// a nibble mask maps onto v_cvt_f32_ubyteN (one VALU op per weight) instead of
// a bit-field extract followed by a conversion.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return __half2float(__ushort_as_half((unsigned short)(h & 0xFFFFu)));
}

// OCP E4M3 (FN) byte (the low 8 bits of c) -> fp32, exact, by the hardware
// converter (the NaN code is not produced by encoders).
__device__ __forceinline__ float e4m3_to_float(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// ---- elements per weight unit (one lane's share of a row per step) ----
template <int FMT> struct Unit;
template <> struct Unit<FMT_BF16> { static constexpr int E = 8; };
template <> struct Unit<FMT_Q4_1> { static constexpr int E = 32; };
template <> struct Unit<FMT_NVFP4> { static constexpr int E = 32; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream16(const void *p) {
    u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw bytes of one unit of one row, as loaded from HBM.
struct WUnit {
    uint4 c;     // 16 bytes of codes (bf16: 8 values)
    uint32_t s;  // q4_1: {fp16 d, fp16 m}; NVFP4: two E4M3 scale bytes; bf16: unused
};

// Matrix view in the device layout: [rows, K].
struct Mat {
    const uint8_t *base;
    int rows, k;
    float ts;  // NVFP4 tensor scale (1 otherwise)
};

// Tensor scale i of an NVFP4 layer, 1 for the other formats.  The choice is
// made at compile time (an NVFP4 call always carries its scales, which the
// host checks): a load under a run-time condition gets a wait of its own, and
// that wait would sit in front of the weight loads issued after it.
template <int FMT>
__device__ __forceinline__ float tensor_scale(const float *ts, int i) {
    return FMT == FMT_NVFP4 ? ts[i] : 1.f;
}

template <int FMT>
__device__ __forceinline__ size_t mat_bytes(int rows, int k) {
    if (FMT == FMT_BF16) return (size_t)rows * k * 2;
    if (FMT == FMT_Q4_1) return (size_t)rows * (k / 2) + (size_t)rows * (k / 32) * 4;
    return (size_t)rows * (k / 2) + (size_t)rows * (k / 16);
}

template <int FMT>
__device__ __forceinline__ WUnit load_unit(const Mat &m, int row, int u) {
    WUnit w;
    if (FMT == FMT_BF16) {
        w.c = ld_stream16((const uint4 *)(m.base + (size_t)row * m.k * 2) + u);
        w.s = 0;
    } else if (FMT == FMT_Q4_1) {
        w.c = ld_stream16((const uint4 *)(m.base + (size_t)row * (m.k / 2)) + u);
        const uint32_t *sp = (const uint32_t *)(m.base + (size_t)m.rows * (m.k / 2) + (size_t)row * (m.k / 32) * 4);
        w.s = __builtin_nontemporal_load(sp + u);
    } else {
        w.c = ld_stream16((const uint4 *)(m.base + (size_t)row * (m.k / 2)) + u);
        const uint16_t *sp = (const uint16_t *)(m.base + (size_t)m.rows * (m.k / 2) + (size_t)row * (m.k / 16));
        w.s = __builtin_nontemporal_load(sp + u);
    }
    return w;
}

// Activation unit in registers: the unit's elements and (4-bit formats) their sum.
template <int FMT> struct XUnit {
    float v[Unit<FMT>::E];
    float sum;
};

template <int FMT>
__device__ __forceinline__ void load_x(XUnit<FMT> &x, const float *src, int u) {
    const float4 *p = (const float4 *)(src + (size_t)u * Unit<FMT>::E);
#pragma unroll
    for (int i = 0; i < Unit<FMT>::E / 4; i++) {
        float4 f = p[i];
        x.v[4 * i + 0] = f.x;
        x.v[4 * i + 1] = f.y;
        x.v[4 * i + 2] = f.z;
        x.v[4 * i + 3] = f.w;
    }
    if (FMT == FMT_Q4_1) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < Unit<FMT>::E; i++) s += x.v[i];
        x.sum = s;
    } else {
        x.sum = 0.f;
    }
}

// Activations staged in LDS as 16-byte chunks, unit u's chunk c at slot
// u * (E / 4) + (c ^ ((u >> 1) & (E / 4 - 1))): 16 lanes reading one chunk of
// 16 consecutive units then hit distinct banks.
template <int FMT>
__device__ __forceinline__ int xs_slot(int q) {
    constexpr int CPU = Unit<FMT>::E / 4;
    const int u = q / CPU, c = q % CPU;
    return u * CPU + (c ^ ((u >> 1) & (CPU - 1)));
}

// load_x from the LDS staging (same values, same sum order)
template <int FMT>
__device__ __forceinline__ void load_x_lds(XUnit<FMT> &x, const uint4 *xs, int u) {
    constexpr int CPU = Unit<FMT>::E / 4;
#pragma unroll
    for (int i = 0; i < CPU; i++) {
        const uint4 f = xs[u * CPU + (i ^ ((u >> 1) & (CPU - 1)))];
        x.v[4 * i + 0] = __uint_as_float(f.x);
        x.v[4 * i + 1] = __uint_as_float(f.y);
        x.v[4 * i + 2] = __uint_as_float(f.z);
        x.v[4 * i + 3] = __uint_as_float(f.w);
    }
    if (FMT == FMT_Q4_1) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < Unit<FMT>::E; i++) s += x.v[i];
        x.sum = s;
    } else {
        x.sum = 0.f;
    }
}

// dot(unit weights, unit activations) in fp32.
template <int FMT>
__device__ __forceinline__ float unit_dot(const WUnit &w, const XUnit<FMT> &x, float ts) {
    if (FMT == FMT_BF16) {
        uint32_t a[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            acc = __builtin_fmaf(bf16lo(a[i]), x.v[2 * i], acc);
            acc = __builtin_fmaf(bf16hi(a[i]), x.v[2 * i + 1], acc);
        }
        return acc;
    } else if (FMT == FMT_Q4_1) {
        // sum_i (d q_i + m) x_i = d * sum_i q_i x_i + m * sum_i x_i.  A byte
        // holding a code q < 16, read as an E4M3 float, is exactly q * 2^-9, so
        // one packed conversion turns two codes into floats; every partial sum
        // is then exactly 2^-9 of the integer-code one and d * 2^9 restores it
        // (same roundings, same result).
        uint32_t a[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t lo = a[i] & 0x0F0F0F0Fu, hi = (a[i] >> 4) & 0x0F0F0F0Fu;
            const auto l01 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false), l23 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
            const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false), h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
            const float ql[4] = {l01[0], l01[1], l23[0], l23[1]}, qh[4] = {h01[0], h01[1], h23[0], h23[1]};
#pragma unroll
            for (int b = 0; b < 4; b++) {
                acc0 = __builtin_fmaf(ql[b], x.v[4 * i + b], acc0);
                acc1 = __builtin_fmaf(qh[b], x.v[16 + 4 * i + b], acc1);
            }
        }
        float d = half_bits_to_float(w.s) * 512.0f, m = half_bits_to_float(w.s >> 16);
        return __builtin_fmaf(d, acc0 + acc1, m * x.sum);
    } else {
        // two blocks of 16: e2m1 codes decoded by the hardware converter
        // (scale 1.0: exact), each block scaled by its E4M3 scale.
        uint32_t a[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
        float acc[2] = {0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 0);
            auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 1);
            auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 2);
            auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 3);
            float s = acc[i >> 1];
            s = __builtin_fmaf(p0[0], x.v[8 * i + 0], s);
            s = __builtin_fmaf(p0[1], x.v[8 * i + 1], s);
            s = __builtin_fmaf(p1[0], x.v[8 * i + 2], s);
            s = __builtin_fmaf(p1[1], x.v[8 * i + 3], s);
            s = __builtin_fmaf(p2[0], x.v[8 * i + 4], s);
            s = __builtin_fmaf(p2[1], x.v[8 * i + 5], s);
            s = __builtin_fmaf(p3[0], x.v[8 * i + 6], s);
            s = __builtin_fmaf(p3[1], x.v[8 * i + 7], s);
            acc[i >> 1] = s;
        }
        float s0 = e4m3_to_float(w.s & 0xFFu), s1 = e4m3_to_float((w.s >> 8) & 0xFFu);
        return ts * __builtin_fmaf(s0, acc[0], s1 * acc[1]);
    }
}

// dot(unit weights, x) for two tokens at once: each weight is decoded once.
template <int FMT>
__device__ __forceinline__ void unit_dot2(const WUnit &w, const XUnit<FMT> &xa, const XUnit<FMT> &xb, float ts,
                                          float &ra, float &rb) {
    if (FMT == FMT_BF16) {
        uint32_t a[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float lo = bf16lo(a[i]), hi = bf16hi(a[i]);
            sa = __builtin_fmaf(lo, xa.v[2 * i], sa);
            sb = __builtin_fmaf(lo, xb.v[2 * i], sb);
            sa = __builtin_fmaf(hi, xa.v[2 * i + 1], sa);
            sb = __builtin_fmaf(hi, xb.v[2 * i + 1], sb);
        }
        ra = sa;
        rb = sb;
    } else if (FMT == FMT_Q4_1) {
        uint32_t a[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
        float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t lo = opaque(a[i] & 0x0F0F0F0Fu);
            uint32_t hi = opaque((a[i] >> 4) & 0x0F0F0F0Fu);
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const float ql = (float)((lo >> (8 * b)) & 0xFFu), qh = (float)((hi >> (8 * b)) & 0xFFu);
                a0 = __builtin_fmaf(ql, xa.v[4 * i + b], a0);
                b0 = __builtin_fmaf(ql, xb.v[4 * i + b], b0);
                a1 = __builtin_fmaf(qh, xa.v[16 + 4 * i + b], a1);
                b1 = __builtin_fmaf(qh, xb.v[16 + 4 * i + b], b1);
            }
        }
        const float d = half_bits_to_float(w.s), m = half_bits_to_float(w.s >> 16);
        ra = __builtin_fmaf(d, a0 + a1, m * xa.sum);
        rb = __builtin_fmaf(d, b0 + b1, m * xb.sum);
    } else {
        uint32_t a[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
        float sa[2] = {0.f, 0.f}, sb[2] = {0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 0);
            const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 1);
            const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 2);
            const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(a[i], 1.0f, 3);
            const float v[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
            for (int j = 0; j < 8; j++) {
                sa[i >> 1] = __builtin_fmaf(v[j], xa.v[8 * i + j], sa[i >> 1]);
                sb[i >> 1] = __builtin_fmaf(v[j], xb.v[8 * i + j], sb[i >> 1]);
            }
        }
        const float s0 = e4m3_to_float(w.s & 0xFFu), s1 = e4m3_to_float((w.s >> 8) & 0xFFu);
        ra = ts * __builtin_fmaf(s0, sa[0], s1 * sa[1]);
        rb = ts * __builtin_fmaf(s0, sb[0], s1 * sb[1]);
    }
}

// DPP lane exchange within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
constexpr int DPP_XOR1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within each 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within each 16

// Sum over groups of LPR consecutive lanes (LPR a power of two <= 64).  Each
// step pairs every lane with one partner of the same group and adds, so all
// lanes of a group end with the same value, in a fixed order.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    if (LPR >= 2) v += dpp_f<DPP_XOR1>(v);
    if (LPR >= 4) v += dpp_f<DPP_XOR2>(v);
    if (LPR >= 8) v += dpp_f<DPP_HALF_MIRROR>(v);
    if (LPR >= 16) v += dpp_f<DPP_MIRROR>(v);
    if (LPR >= 32) v += __shfl_xor(v, 16, MOE_WAVE);
    if (LPR >= 64) v += __shfl_xor(v, 32, MOE_WAVE);
    return v;
}

// Sum over the whole wave, returned uniform (an SGPR value): rows of 16
// reduced by DPP, then row 1 += row 0 and row 3 += row 2 (row_bcast:15),
// rows 2-3 += row 1 (row_bcast:31), and lane 63 read back.  Fixed order, and
// no LDS round trip (unlike a shuffle through ds_bpermute).
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    v += dpp_f<DPP_HALF_MIRROR>(v);
    v += dpp_f<DPP_MIRROR>(v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// v from lane ^ (1 << s) (every lane active)
__device__ __forceinline__ float xor_lane(float v, int s) {
    const int i = __float_as_int(v);
    if (s == 0) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
    if (s == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
    if (s == 2) return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x101F));             // xor 4
    if (s == 3) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x128, 0xF, 0xF, true)); // row_ror 8
    if (s == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x401F));             // xor 16
    return __shfl_xor(v, 32, 64);
}

// Sums of P values (P a power of two <= 64) over the 64 lanes; value j ends in
// every lane l with l % P == j.  Level s pairs lane l with l ^ (1 << s): each
// keeps the half of its values whose index has bit s equal to its own lane
// bit and adds the partner's copy of that half, so after log2(P) levels one
// value remains, and the last levels add it over the remaining lane bits.
// Each sum has a fixed order.
template <int P>
__device__ __forceinline__ float wave_reduce_rows(float (&v)[P], int lane) {
    float a[P];
#pragma unroll
    for (int j = 0; j < P; j++) a[j] = v[j];
    int lev = 0;
#pragma unroll
    for (int n = P; n > 1; n >>= 1, lev++) {
        const bool hi = (lane >> lev) & 1;
#pragma unroll
        for (int m = 0; m < n / 2; m++) {
            const float keep = hi ? a[2 * m + 1] : a[2 * m];
            const float send = hi ? a[2 * m] : a[2 * m + 1];
            a[m] = keep + xor_lane(send, lev);
        }
    }
    float r = a[0];
#pragma unroll
    for (int s = lev; s < 6; s++) r += xor_lane(r, s);
    return r;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Order-preserving map of fp32 to uint32 (larger float -> larger key, -0 is
// folded into +0 first so that the two compare equal as floats do); key 0
// is below every float key, including -inf.
__device__ __forceinline__ uint32_t f2key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// max with a DPP-exchanged copy (lanes whose source is invalid read 0).
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true));
}
// rows enabled in ROW_MASK take the max with lane 15 (0x142) or lane 31
// (0x143) of the wave; other rows keep their value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t max_bcast(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false));
}

// Largest key of the wave, valid in every lane (read back from lane 63).
__device__ __forceinline__ uint32_t wave_max_key(uint32_t v) {
    v = max_dpp<DPP_XOR1>(v);
    v = max_dpp<DPP_XOR2>(v);
    v = max_dpp<DPP_HALF_MIRROR>(v);
    v = max_dpp<DPP_MIRROR>(v);
    v = max_bcast<0x142, 0xA>(v);
    v = max_bcast<0x143, 0xC>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of one token's logits by one wave: (value descending, index
// ascending), decided on the fp32 logits; weights w_i = exp(l_i - l_0) /
// sum_j exp(l_j - l_0), the softmax over all experts renormalised over the
// chosen ones.  Lane i < K returns slot i (its expert in *e_out, its weight
// in *w_out); other lanes return expert 0, weight 0.  Each round takes the
// wave's largest key, then the lowest expert index holding it (ballots over
// index = lane + 64k, k ascending).  No per-thread arrays: an array indexed
// by the lane would be moved to LDS and need the dispatch packet (in host
// memory) to compute thread offsets.
// The selection on logits already in registers: lv[k] = logit of expert
// lane + 64 k (any value for indices >= E).
__device__ __forceinline__ void wave_topk_regs(const float lv[4], int E, int K, int *e_out, float *w_out) {
    const int lane = threadIdx.x & (MOE_WAVE - 1);
    uint32_t key[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int ix = lane + 64 * k;
        const float v = __uint_as_float(opaque(__float_as_uint(lv[k])));
        key[k] = ix < E ? f2key(v) : 0u;
    }
    int my_e = 0;
    uint32_t my_key = 0, first_key = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t m = wave_max_key(max(max(key[0], key[1]), max(key[2], key[3])));
        int gi = 0;
#pragma unroll
        for (int k = 3; k >= 0; k--) {
            const uint64_t b = __ballot(key[k] == m);
            gi = b ? 64 * k + (int)__builtin_ctzll(b) : gi;
        }
        if (i == 0) first_key = m;
        my_e = (lane == i) ? gi : my_e;
        my_key = (lane == i) ? m : my_key;
#pragma unroll
        for (int k = 0; k < 4; k++) key[k] = (lane + 64 * k == gi) ? 0u : key[k];
        if (i + 1 >= K) break;
    }
    const float ev = lane < K ? __expf(key2f(my_key) - key2f(first_key)) : 0.f;
    const float den = wave_sum(ev);
    *e_out = lane < K ? my_e : 0;
    *w_out = ev / den;
}

// 1 / sqrt(mean(y^2) + 1e-6), summed in the same order in every wave of
// every kernel: lane l takes elements 8l + 512i + j (j < 8) for i < UPLR
// (d_model = 512 * UPLR), in order, then the DPP/shuffle butterfly.  y holds
// the 2*UPLR float4 at float4 indices 2l + 128i and 2l + 1 + 128i.
template <int UPLR>
__device__ __forceinline__ float inv_rms_from(const float4 (&y)[2 * UPLR]) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 2 * UPLR; i++) {
        ss = __builtin_fmaf(y[i].x, y[i].x, ss);
        ss = __builtin_fmaf(y[i].y, y[i].y, ss);
        ss = __builtin_fmaf(y[i].z, y[i].z, ss);
        ss = __builtin_fmaf(y[i].w, y[i].w, ss);
    }
    ss = wave_sum(ss);
    return 1.0f / sqrtf(ss / (float)(UPLR * 512) + 1e-6f);
}

template <int UPLR>
__device__ __forceinline__ void load_rms_part(float4 (&y)[2 * UPLR], const float *src) {
    const int lane = threadIdx.x & (MOE_WAVE - 1);
#pragma unroll
    for (int i = 0; i < UPLR; i++) {
        y[2 * i] = ((const float4 *)src)[2 * lane + 128 * i];
        y[2 * i + 1] = ((const float4 *)src)[2 * lane + 1 + 128 * i];
    }
}

// Index of the n-th largest logit (n = 0: the largest) by the same rounds as
// wave_topk_regs, stopping after round n: the same expert that wave_topk
// returns in lane n.
__device__ __forceinline__ int wave_topk_nth(const float lv[4], int E, int n) {
    const int lane = threadIdx.x & (MOE_WAVE - 1);
    uint32_t key[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int ix = lane + 64 * k;
        const float v = __uint_as_float(opaque(__float_as_uint(lv[k])));
        key[k] = ix < E ? f2key(v) : 0u;
    }
    int gi = 0;
    for (int i = 0; i <= n; i++) {
        const uint32_t m = wave_max_key(max(max(key[0], key[1]), max(key[2], key[3])));
        gi = 0;
#pragma unroll
        for (int k = 3; k >= 0; k--) {
            const uint64_t b = __ballot(key[k] == m);
            gi = b ? 64 * k + (int)__builtin_ctzll(b) : gi;
        }
#pragma unroll
        for (int k = 0; k < 4; k++) key[k] = (lane + 64 * k == gi) ? 0u : key[k];
    }
    return gi;
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP only: row_shr
// 1, 2, 4, 8 scan each 16-lane row (lanes shifted in from outside the row
// read 0), then lane 15 of row 0 / 2 is added to rows 1 / 3 (row_bcast:15)
// and lane 31 to rows 2 and 3 (row_bcast:31).  Rows outside a row mask keep
// the old value 0, so they add nothing.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return v;
}

// Loads of one token's logits for wave_topk_regs (clamped in-bounds indices).
__device__ __forceinline__ void wave_topk_load(const float *l, int E, float lv[4]) {
    const int lane = threadIdx.x & (MOE_WAVE - 1);
#pragma unroll
    for (int k = 0; k < 4; k++) lv[k] = l[min(lane + 64 * k, E - 1)];
}

__device__ __forceinline__ void wave_topk(const float *l, int E, int K, int *e_out, float *w_out) {
    // four loads issued back to back; the opaque copy in wave_topk_regs keeps
    // the compiler from sinking a load into the (ix < E) branch
    float lv[4];
    wave_topk_load(l, E, lv);
    wave_topk_regs(lv, E, K, e_out, w_out);
}

}  // namespace moe
