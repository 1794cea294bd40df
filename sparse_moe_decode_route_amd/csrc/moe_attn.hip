// Decode attention: one new token per sequence against its key/value cache.
//
// What it computes: "Recursive Flint 40B-A2.5B" (orcarouter.ai blog),
// section "The architecture is a memory-bandwidth argument", attention and
// positional-encoding bullets: 32 query heads share 4 key/value heads of
// size 128; sliding-window layers see the current token and the 512 before
// it and use rotary embeddings, full layers see every earlier token and use
// none; queries and keys are RMS-normalised per head and every head has a
// learned sink.  Readings taken where the page is silent: the sink is one
// logit per query head that joins the softmax denominator only; the rotary
// embedding turns the pairs (i, i + 64) by P * base^(-2i/128); the cache
// holds bfloat16 keys (normalised and rotated) and values.
//
// Three kernels:
//   attn_prep    per head: RMSNorm, rotary embedding (angle reduced in fp64,
//                since P * freq needs more than fp32 at long positions), the
//                query scaled by 1/sqrt(128) into the workspace, the new key
//                and value rounded to bfloat16 into the caches at P;
//   attn_chunk   per (sequence, key/value head, chunk of positions): the
//                group's query heads against the chunk's keys (scores to
//                LDS), the chunk's max and exp-sum per head, then the values
//                weighted by the exponentials; partial (max, sum, output)
//                per chunk to the workspace;
//   attn_combine per (sequence, query head): the chunks merged with the
//                sink in a fixed order: out = sum_c e^(m_c - M) o_c /
//                (e^(z - M) + sum_c e^(m_c - M) l_c), M = max(z, max_c m_c).
// Chunks are 64 positions in sliding-window layers (a window spreads over
// 9-10 blocks per key/value head) and up to 1024 in full layers (about 1024
// blocks per call at the cache's length); within a chunk two load groups of
// 32 positions are in flight, the next loading while one is computed.
// The cache is the stream: a full layer at long context reads 2 KiB per
// position per key/value head pair (K and V), so attn_chunk is bound by HBM.
// Lanes: 8 lanes per position (16 dimensions each, two 16-byte loads of a
// 256-byte row), 8 positions per wave instruction; each wave serves up to 4
// query heads of the group and keeps their query slices in registers.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int AT_D = 128;       // head size
constexpr int AT_CMAX = 1024;   // largest chunk (positions)
constexpr int AT_UT = 4;        // tiles of 8 positions per load group
constexpr int AT_PREP_WAVES = 8;
constexpr int AT_COMB_WAVES = 16;

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ int attn_lo(const AttnArgs &p, int P) {
    return p.window > 0 ? max(0, P - p.window + 1) : 0;
}

// First chunk a sequence reads.
__device__ __forceinline__ int attn_first_chunk(const AttnArgs &p, int P) {
    return p.window > 0 ? attn_lo(p, P) / p.chunk : 0;
}

__global__ void __launch_bounds__(64 * AT_PREP_WAVES) attn_prep(AttnArgs p) {
    const int lane = threadIdx.x & 63;
    const int hi = blockIdx.y * AT_PREP_WAVES + (threadIdx.x >> 6);
    const int b = blockIdx.x;
    if (hi >= p.Hq + p.Hkv) return;
    const int P = p.pos[b];
    if (P < 0 || P >= p.max_len) return;  // invalid position: caches untouched, output NaN (combine)
    const bool is_q = hi < p.Hq;
    const float *src = is_q ? p.q + ((size_t)b * p.Hq + hi) * AT_D : p.k_new + ((size_t)b * p.Hkv + hi - p.Hq) * AT_D;
    const float *w = is_q ? p.q_norm_w : p.k_norm_w;
    float x0 = src[lane], x1 = src[lane + 64];
    const float inv = 1.0f / sqrtf(wave_sum(x0 * x0 + x1 * x1) / (float)AT_D + p.eps);
    float y0 = x0 * inv * w[lane], y1 = x1 * inv * w[lane + 64];
    if (p.window > 0) {
        // angle P * base^(-2 lane / 128), reduced modulo 2 pi in fp64
        const double freq = exp2(-2.0 * lane / AT_D * log2((double)p.rope_base));
        const double two_pi = 6.283185307179586476925286766559;
        double ang = (double)P * freq;
        ang -= two_pi * floor(ang / two_pi);
        double sd, cd;
        sincos(ang, &sd, &cd);
        const float c = (float)cd, s = (float)sd;
        const float r0 = y0 * c - y1 * s, r1 = y0 * s + y1 * c;
        y0 = r0;
        y1 = r1;
    }
    if (is_q) {
        const float sc = 0.08838834764831845f;  // 1 / sqrt(128)
        float *dst = p.q_prep + ((size_t)b * p.Hq + hi) * AT_D;
        dst[lane] = y0 * sc;
        dst[lane + 64] = y1 * sc;
    } else {
        const int g = hi - p.Hq;
        const size_t row = (((size_t)b * p.Hkv + g) * p.max_len + P) * AT_D;
        p.k_cache[row + lane] = to_bf16_rne(y0);
        p.k_cache[row + lane + 64] = to_bf16_rne(y1);
        const float *vs = p.v_new + ((size_t)b * p.Hkv + g) * AT_D;
        p.v_cache[row + lane] = to_bf16_rne(vs[lane]);
        p.v_cache[row + lane + 64] = to_bf16_rne(vs[lane + 64]);
    }
}

// v from lane ^ (1 << s), every lane active
__device__ __forceinline__ float at_xor(float v, int s) {
    const int i = __float_as_int(v);
    if (s == 0) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true));
    if (s == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true));
    if (s == 2) return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x101F));
    if (s == 3) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x128, 0xF, 0xF, true));
    if (s == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x401F));
    return __shfl_xor(v, 32, 64);
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int s = 0; s < 6; s++) v = fmaxf(v, at_xor(v, s));
    return v;
}

// 16 bf16 (two 16-byte chunks) -> fp32
__device__ __forceinline__ void unpack16(const uint4 &a, const uint4 &b, float (&f)[16]) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        f[2 * i] = bf16lo(w[i]);
        f[2 * i + 1] = bf16hi(w[i]);
    }
}

// HW query heads per wave, WV waves per block (HW * WV = group size).
// Score partials of one tile (8 positions) for HW heads, summed over the
// position's 8 lanes: each level halves the heads a lane carries, then the
// remaining levels add; lanes with sub < HW end holding head sub.
template <int HW>
__device__ __forceinline__ float tile_scores(const float (&qv)[HW][16], const uint4 &ka, const uint4 &kb, int lane) {
    float kf[16];
    unpack16(ka, kb, kf);
    float a[HW];
#pragma unroll
    for (int h = 0; h < HW; h++) {
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < 16; d++) s = __builtin_fmaf(qv[h][d], kf[d], s);
        a[h] = s;
    }
    int lev = 0;
#pragma unroll
    for (int m = HW; m > 1; m >>= 1, lev++) {
        const bool hib = (lane >> lev) & 1;
#pragma unroll
        for (int k = 0; k < m / 2; k++) {
            const float keep = hib ? a[2 * k + 1] : a[2 * k];
            const float send = hib ? a[2 * k] : a[2 * k + 1];
            a[k] = keep + at_xor(send, lev);
        }
    }
    float s = a[0];
#pragma unroll
    for (int l2 = lev; l2 < 3; l2++) s += at_xor(s, l2);
    return s;
}

// HW query heads per wave, WV waves per block (HW * WV = group size).
template <int HW, int WV>
__global__ void __launch_bounds__(64 * WV) attn_chunk(AttnArgs p) {
    __shared__ float sc[WV][AT_CMAX][HW];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane & 7, pg = lane >> 3;
    const int b = blockIdx.z, g = blockIdx.y;
    const int P = p.pos[b];
    if (P < 0 || P >= p.max_len) return;
    const int lo = attn_lo(p, P);
    const int c = attn_first_chunk(p, P) + blockIdx.x;
    const int c0 = c * p.chunk;
    const int start = max(c0, lo), end = min(c0 + p.chunk, P + 1);  // [start, end)
    if (start >= end) return;
    const int h0 = g * (HW * WV) + w * HW;
    float qv[HW][16];
#pragma unroll
    for (int h = 0; h < HW; h++) {
        const float4 *qs = reinterpret_cast<const float4 *>(p.q_prep + ((size_t)b * p.Hq + h0 + h) * AT_D + 16 * sub);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float4 f = qs[i];
            qv[h][4 * i] = f.x;
            qv[h][4 * i + 1] = f.y;
            qv[h][4 * i + 2] = f.z;
            qv[h][4 * i + 3] = f.w;
        }
    }
    const size_t base = ((size_t)b * p.Hkv + g) * p.max_len;
    const uint4 *K = reinterpret_cast<const uint4 *>(p.k_cache + base * AT_D) + 2 * sub;
    const uint4 *V = reinterpret_cast<const uint4 *>(p.v_cache + base * AT_D) + 2 * sub;
    const int n = end - start;
    const int ngrp = (n + 8 * AT_UT - 1) / (8 * AT_UT);  // load groups of AT_UT tiles

    // rows of group gi into (x, y); rows past the chunk's end re-read its last row
    auto issue = [&](const uint4 *M, uint4 (&x)[AT_UT], uint4 (&y)[AT_UT], int gi) {
#pragma unroll
        for (int u = 0; u < AT_UT; u++) {
            const int j = start + min((gi * AT_UT + u) * 8 + pg, n - 1);
            x[u] = ld_stream16(M + (size_t)j * 16);
            y[u] = ld_stream16(M + (size_t)j * 16 + 1);
        }
    };

    // scores, two load groups in registers
    {
        uint4 xa[AT_UT], ya[AT_UT], xb[AT_UT], yb[AT_UT];
        auto scores = [&](const uint4 (&x)[AT_UT], const uint4 (&y)[AT_UT], int gi) {
#pragma unroll
            for (int u = 0; u < AT_UT; u++) {
                const float s = tile_scores<HW>(qv, x[u], y[u], lane);
                const int jj = (gi * AT_UT + u) * 8 + pg;  // position within [start, end)
                if (jj < n && sub < HW) sc[w][jj][sub] = s;
            }
        };
        issue(K, xa, ya, 0);
        for (int gi = 0; gi < ngrp; gi += 2) {
            if (gi + 1 < ngrp) issue(K, xb, yb, gi + 1);
            scores(xa, ya, gi);
            if (gi + 2 < ngrp) issue(K, xa, ya, gi + 2);
            if (gi + 1 < ngrp) scores(xb, yb, gi + 1);
        }
    }
    __syncthreads();

    // per head: the chunk's max, exponentials in place, their sum
    float mh[HW], lh[HW];
#pragma unroll
    for (int h = 0; h < HW; h++) {
        float m = -INFINITY;
        for (int j = lane; j < n; j += 64) m = fmaxf(m, sc[w][j][h]);
        mh[h] = wave_max_f(m);
    }
#pragma unroll
    for (int h = 0; h < HW; h++) {
        float l = 0.f;
        for (int j = lane; j < n; j += 64) {
            const float e = __expf(sc[w][j][h] - mh[h]);
            sc[w][j][h] = e;
            l += e;
        }
        lh[h] = wave_sum(l);
    }
    __syncthreads();

    // values weighted by the exponentials
    float o[HW][16];
#pragma unroll
    for (int h = 0; h < HW; h++)
#pragma unroll
        for (int d = 0; d < 16; d++) o[h][d] = 0.f;
    {
        uint4 xa[AT_UT], ya[AT_UT], xb[AT_UT], yb[AT_UT];
        auto accum = [&](const uint4 (&x)[AT_UT], const uint4 (&y)[AT_UT], int gi) {
#pragma unroll
            for (int u = 0; u < AT_UT; u++) {
                const int jj = (gi * AT_UT + u) * 8 + pg;
                if (jj >= n) continue;  // lanes past the chunk's end add nothing
                float vf[16];
                unpack16(x[u], y[u], vf);
#pragma unroll
                for (int h = 0; h < HW; h++) {
                    const float e = sc[w][jj][h];
#pragma unroll
                    for (int d = 0; d < 16; d++) o[h][d] = __builtin_fmaf(e, vf[d], o[h][d]);
                }
            }
        };
        issue(V, xa, ya, 0);
        for (int gi = 0; gi < ngrp; gi += 2) {
            if (gi + 1 < ngrp) issue(V, xb, yb, gi + 1);
            accum(xa, ya, gi);
            if (gi + 2 < ngrp) issue(V, xa, ya, gi + 2);
            if (gi + 1 < ngrp) accum(xb, yb, gi + 1);
        }
    }
    // sum over the 8 position lanes (lane bits 3..5)
#pragma unroll
    for (int h = 0; h < HW; h++)
#pragma unroll
        for (int d = 0; d < 16; d++) {
            float v = o[h][d];
            v += at_xor(v, 3);
            v += at_xor(v, 4);
            v += at_xor(v, 5);
            o[h][d] = v;
        }
    const int NC = p.n_chunks;
    const int cl = blockIdx.x;  // chunk slot of this sequence
    if (pg == 0) {
#pragma unroll
        for (int h = 0; h < HW; h++) {
            float4 *dst = reinterpret_cast<float4 *>(p.part_o + (((size_t)b * p.Hq + h0 + h) * NC + cl) * AT_D + 16 * sub);
#pragma unroll
            for (int i = 0; i < 4; i++) dst[i] = make_float4(o[h][4 * i], o[h][4 * i + 1], o[h][4 * i + 2], o[h][4 * i + 3]);
        }
    }
    if (lane < HW) {
        const size_t at = ((size_t)b * p.Hq + h0 + lane) * NC + cl;
        float m = mh[0], l = lh[0];
#pragma unroll
        for (int h = 1; h < HW; h++)
            if (lane == h) {
                m = mh[h];
                l = lh[h];
            }
        p.part_m[at] = m;
        p.part_l[at] = l;
    }
}

// one block per (sequence, query head); wave w merges chunks w, w + 16, ...,
// lane covers dimensions 2 lane, 2 lane + 1; the waves' sums are added in
// wave order
__global__ void __launch_bounds__(64 * AT_COMB_WAVES) attn_combine(AttnArgs p) {
    __shared__ float red[AT_COMB_WAVES][2];
    __shared__ float2 ov[AT_COMB_WAVES][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int h = blockIdx.y, b = blockIdx.x;
    const int P = p.pos[b];
    if (P < 0 || P >= p.max_len) {
        if (w == 0)
            reinterpret_cast<float2 *>(p.out + ((size_t)b * p.Hq + h) * AT_D)[lane] = make_float2(NAN, NAN);
        return;
    }
    const int lo = attn_lo(p, P);
    const int cf = attn_first_chunk(p, P);
    const int nc = P / p.chunk - cf + 1;  // chunk slots holding this sequence's positions
    const size_t at = ((size_t)b * p.Hq + h) * p.n_chunks;
    auto valid = [&](int k) {
        const int c0 = (cf + k) * p.chunk;
        return max(c0, lo) < min(c0 + p.chunk, P + 1);
    };
    const float z = p.sinks[h];
    // M = max(z, max_c m_c): every lane of every wave takes part
    float m = z;
    for (int k = threadIdx.x; k < nc; k += 64 * AT_COMB_WAVES)
        if (valid(k)) m = fmaxf(m, p.part_m[at + k]);
    m = wave_max_f(m);
    if (lane == 0) red[w][0] = m;
    __syncthreads();
    float M = red[0][0];
#pragma unroll
    for (int i = 1; i < AT_COMB_WAVES; i++) M = fmaxf(M, red[i][0]);
    // this wave's chunks: sum of e^(m_c - M) l_c and of e^(m_c - M) o_c,
    // four chunks' loads in flight at a time
    float L = 0.f;
    float2 acc = make_float2(0.f, 0.f);
    for (int k0 = w; k0 < nc; k0 += 4 * AT_COMB_WAVES) {
        float mk[4], lk[4];
        float2 vk[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int k = min(k0 + u * AT_COMB_WAVES, nc - 1);
            mk[u] = p.part_m[at + k];
            lk[u] = p.part_l[at + k];
            vk[u] = reinterpret_cast<const float2 *>(p.part_o + (at + k) * AT_D)[lane];
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int k = k0 + u * AT_COMB_WAVES;
            if (k >= nc || !valid(k)) continue;
            const float e = __expf(mk[u] - M);
            L = __builtin_fmaf(e, lk[u], L);
            acc.x = __builtin_fmaf(e, vk[u].x, acc.x);
            acc.y = __builtin_fmaf(e, vk[u].y, acc.y);
        }
    }
    if (lane == 0) red[w][1] = L;
    ov[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
        float Ls = __expf(z - M);
        float2 o = make_float2(0.f, 0.f);
#pragma unroll
        for (int i = 0; i < AT_COMB_WAVES; i++) {
            Ls += red[i][1];
            o.x += ov[i][lane].x;
            o.y += ov[i][lane].y;
        }
        const float inv = 1.0f / Ls;
        reinterpret_cast<float2 *>(p.out + ((size_t)b * p.Hq + h) * AT_D)[lane] = make_float2(o.x * inv, o.y * inv);
    }
}

template <int HW, int WV>
void launch_chunks(const AttnArgs &p, hipStream_t st) {
    const dim3 grid(p.n_chunks, p.Hkv, p.B);
    auto kern = attn_chunk<HW, WV>;
    if (p.ev)
        hipExtLaunchKernelGGL(kern, grid, dim3(64 * WV), 0, st, p.ev[2], p.ev[3], 0, p);
    else
        hipLaunchKernelGGL(kern, grid, dim3(64 * WV), 0, st, p);
}

}  // namespace

// Chunk size: 64 positions for a sliding window (its 513 positions then
// spread over 9-10 blocks per key/value head); for full attention the
// smallest power of two in [64, 1024] that keeps the blocks of a call to
// about 1024 at the cache's full length.
int attn_chunk_size(int window, int max_len, int B, int Hkv) {
    if (window > 0) return 64;
    int c = 64;
    while (c < AT_CMAX && (long long)((max_len + c - 1) / c) * B * Hkv > 1024) c *= 2;
    return c;
}

int attn_chunk_slots(int window, int max_len, int chunk) {
    // a window of W positions spans at most ceil((W - 1) / chunk) + 1 chunks
    const int all = (max_len + chunk - 1) / chunk;
    if (window <= 0) return all;
    return min(all, (window - 1 + chunk - 1) / chunk + 1);
}

hipError_t launch_attn(const AttnArgs &a, hipStream_t st) {
    AttnArgs p = a;
    const dim3 gp(p.B, (p.Hq + p.Hkv + AT_PREP_WAVES - 1) / AT_PREP_WAVES);
    if (p.ev)
        hipExtLaunchKernelGGL(attn_prep, gp, dim3(64 * AT_PREP_WAVES), 0, st, p.ev[0], p.ev[1], 0, p);
    else
        hipLaunchKernelGGL(attn_prep, gp, dim3(64 * AT_PREP_WAVES), 0, st, p);
    const int grp = p.Hq / p.Hkv;
    if (grp == 8)
        launch_chunks<4, 2>(p, st);
    else if (grp == 4)
        launch_chunks<4, 1>(p, st);
    else if (grp == 2)
        launch_chunks<2, 1>(p, st);
    else
        launch_chunks<1, 1>(p, st);
    const dim3 gc(p.B, p.Hq);
    if (p.ev)
        hipExtLaunchKernelGGL(attn_combine, gc, dim3(64 * AT_COMB_WAVES), 0, st, p.ev[4], p.ev[5], 0, p);
    else
        hipLaunchKernelGGL(attn_combine, gc, dim3(64 * AT_COMB_WAVES), 0, st, p);
    return hipGetLastError();
}

}  // namespace moe
