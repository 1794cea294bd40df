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
// Two kernels, one block per (sequence, key/value head, chunk of positions)
// in the first, each writing the chunk's partial (max, exp-sum, output) per
// query head to the workspace:
//   attn_chunk     vector path (groups of 1, 2 or 4 query heads per key/value head):
//                  the group's query heads normalised and rotated in
//                  registers (the 64 rotary angles reduced in fp64, since
//                  P * freq needs more than fp32 at long positions); scores
//                  to LDS, the chunk's max and exp-sum per head, then the
//                  values weighted by the exponentials.  8 lanes per position,
//                  lane s holding dimensions 8 s .. + 7 and 64 + 8 s .. + 7
//                  (two 16-byte loads, 128 contiguous bytes per 8 lanes; both
//                  members of every rotary pair in one lane), 8 positions per
//                  wave instruction, two load groups of 32 positions in flight;
//   attn_chunk_mf  matrix-core path (groups of 8, full and sliding-window
//                  layers): scores and the value sums on
//                  v_mfma_f32_16x16x32_bf16 in one pass with a running
//                  softmax (details at the kernel);
//   attn_combine   per (sequence, query head): the chunks merged with the
//                  sink in a fixed order: out = sum_c e^(m_c - M) o_c /
//                  (e^(z - M) + sum_c e^(m_c - M) l_c), M = max(z, max_c m_c).
// The block whose chunk holds P computes the new key (normalised, rotated)
// and value in bf16, uses them for row P and writes them to the caches; no
// other block reads row P.  Chunks are 64 positions in sliding-window layers
// on the matrix-core path (32 on the vector path) and up to 1024 in full
// layers (about 512 blocks per call at the cache's length on the
// matrix-core path, 1024 on the vector path).  The cache
// is the stream: a full layer at long context reads 512 bytes per position
// per key/value head (K and V), so the chunk kernels are bound by HBM.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 at_bf16x8 __attribute__((ext_vector_type(8)));
typedef float at_f32x16 __attribute__((ext_vector_type(16)));

constexpr int AT_D = 128;       // head size
constexpr int AT_CMAX = 1024;   // largest chunk (positions)
constexpr int AT_UT = 4;        // tiles of 8 positions per load group
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

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)to_bf16_rne(lo) | ((uint32_t)to_bf16_rne(hi) << 16);
}

// This lane's 16 values of one head: RMSNorm over the head's 128 values (the
// 8 lanes of a position hold them), gain (this lane's 16 gain values in gv),
// and the rotary turn of the pairs (i, i + 64) with cos / sin from cs.  The
// turn needs the split layout (x[d] = dimension 8 sub + d, x[8 + d] =
// dimension 64 + 8 sub + d), which keeps both members of a pair in the lane.
__device__ __forceinline__ void head_prep(float (&x)[16], const float (&gv)[16], const float (*cs)[64], bool rope,
                                          float eps, int lane) {
    const int sub = lane & 7;
    float ss = 0.f;
#pragma unroll
    for (int d = 0; d < 16; d++) ss = __builtin_fmaf(x[d], x[d], ss);
    ss += at_xor(ss, 0);
    ss += at_xor(ss, 1);
    ss += at_xor(ss, 2);
    const float inv = 1.0f / sqrtf(ss / (float)AT_D + eps);
#pragma unroll
    for (int d = 0; d < 16; d++) x[d] = x[d] * inv * gv[d];
    if (rope) {
        const float4 *c4 = reinterpret_cast<const float4 *>(&cs[0][8 * sub]);
        const float4 *s4 = reinterpret_cast<const float4 *>(&cs[1][8 * sub]);
        const float4 ca = c4[0], cb = c4[1], sa = s4[0], sb = s4[1];
        const float c[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
        const float sn[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
        for (int d = 0; d < 8; d++) {
            const float lo = x[d], hi = x[8 + d];
            x[d] = lo * c[d] - hi * sn[d];
            x[8 + d] = hi * c[d] + lo * sn[d];
        }
    }
}

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

// This lane's 16 values of a 128-value fp32 row: dimensions 16 sub ..
// 16 sub + 15, or with split dimensions 8 sub .. + 7 then 64 + 8 sub .. + 7.
__device__ __forceinline__ void load16(const float *row, int sub, float (&x)[16], bool split = false) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int o = split ? (i < 2 ? 8 * sub + 4 * i : 64 + 8 * sub + 4 * (i - 2)) : 16 * sub + 4 * i;
        const float4 f = *reinterpret_cast<const float4 *>(row + o);
        x[4 * i] = f.x;
        x[4 * i + 1] = f.y;
        x[4 * i + 2] = f.z;
        x[4 * i + 3] = f.w;
    }
}

__device__ __forceinline__ uint4 pack8(const float (&x)[16], int o) {
    return make_uint4(pack_bf16x2(x[o], x[o + 1]), pack_bf16x2(x[o + 2], x[o + 3]), pack_bf16x2(x[o + 4], x[o + 5]),
                      pack_bf16x2(x[o + 6], x[o + 7]));
}

// raw new key, value and key-norm gains of key/value head g, this lane's 16
// dimensions
struct NewRaw {
    float k[16], v[16], gk[16];
};
__device__ __forceinline__ void new_token_load(const AttnArgs &p, int b, int g, int lane, NewRaw &r, bool split) {
    const int sub = lane & 7;
    load16(p.k_new + ((size_t)b * p.Hkv + g) * AT_D, sub, r.k, split);
    load16(p.v_new + ((size_t)b * p.Hkv + g) * AT_D, sub, r.v, split);
    load16(p.k_norm_w, sub, r.gk, split);
}
__device__ __forceinline__ void new_token(const AttnArgs &p, int b, int g, int P, const float (*cs)[64], bool rope,
                                          int lane, bool write, NewRaw &r, bool split, uint4 &k0, uint4 &k1,
                                          uint4 &v0, uint4 &v1) {
    const int sub = lane & 7;
    float(&kx)[16] = r.k;
    const float(&vx)[16] = r.v;
    head_prep(kx, r.gk, cs, rope, p.eps, lane);
    k0 = pack8(kx, 0);
    k1 = pack8(kx, 8);
    v0 = pack8(vx, 0);
    v1 = pack8(vx, 8);
    if (write) {
        const size_t row = (((size_t)b * p.Hkv + g) * p.max_len + P) * AT_D;
        uint4 *kd = reinterpret_cast<uint4 *>(p.k_cache + row);
        uint4 *vd = reinterpret_cast<uint4 *>(p.v_cache + row);
        const int c0 = split ? sub : 2 * sub, c1 = split ? 8 + sub : 2 * sub + 1;  // 16-byte chunks
        kd[c0] = k0;
        kd[c1] = k1;
        vd[c0] = v0;
        vd[c1] = v1;
    }
}

// Vector path (groups of 1, 2 and 4 query heads per key/value head): HW
// query heads per wave, WV waves per block (HW * WV = group size).
template <int HW, int WV>
__global__ void __launch_bounds__(64 * WV) attn_chunk(AttnArgs p) {
    __shared__ float scb[WV * AT_CMAX * HW];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane & 7, pg = lane >> 3;
    // score / exponential of position j for this wave's head h
    auto sc = [&](int j, int h) -> float & { return scb[(w * AT_CMAX + j) * HW + h]; };
    const int b = blockIdx.z, g = blockIdx.y;
    const int P = p.pos[b];
    if (P < 0 || P >= p.max_len) return;
    const int lo = attn_lo(p, P);
    const int c = attn_first_chunk(p, P) + blockIdx.x;
    const int c0 = c * p.chunk;
    const int start = max(c0, lo), end = min(c0 + p.chunk, P + 1);  // [start, end)
    if (start >= end) return;
    const int h0 = g * (HW * WV) + w * HW;
    const size_t base = ((size_t)b * p.Hkv + g) * p.max_len;
    // split layout: a lane reads 16-byte chunks sub and 8 + sub of a row
    const uint4 *K = reinterpret_cast<const uint4 *>(p.k_cache + base * AT_D) + sub;
    const uint4 *V = reinterpret_cast<const uint4 *>(p.v_cache + base * AT_D) + sub;
    const int n = end - start;
    const int ngrp = (n + 8 * AT_UT - 1) / (8 * AT_UT);  // load groups of AT_UT tiles
    // rows of group gi into (x, y); rows past the chunk's end re-read its last row
    auto issue = [&](const uint4 *M, uint4 (&x)[AT_UT], uint4 (&y)[AT_UT], int gi) {
#pragma unroll
        for (int u = 0; u < AT_UT; u++) {
            const int j = start + min((gi * AT_UT + u) * 8 + pg, n - 1);
            x[u] = ld_stream16(M + (size_t)j * 16);
            y[u] = ld_stream16(M + (size_t)j * 16 + 8);
        }
    };
    // the first groups of keys and values are requested before anything else
    uint4 xa[AT_UT], ya[AT_UT], va[AT_UT], vb[AT_UT];
    issue(K, xa, ya, 0);
    issue(V, va, vb, 0);

    // then this wave's raw query heads, their gains, the new key and value
    // (the chunk holding P) and the rotary frequencies: all requested before
    // the rotary table is built
    const bool rope = p.window > 0;
    const double fr = rope && threadIdx.x < 64 ? p.rope_freq[threadIdx.x] : 0.0;
    float qv[HW][16], gq[16];
#pragma unroll
    for (int h = 0; h < HW; h++) load16(p.q + ((size_t)b * p.Hq + h0 + h) * AT_D, sub, qv[h], true);
    load16(p.q_norm_w, sub, gq, true);
    const bool hasP = end == P + 1;
    NewRaw nr;
    if (hasP) new_token_load(p, b, g, lane, nr, true);
    // cos / sin of the 64 rotary angles P * freq_i: the product and its
    // reduction modulo 2 pi in fp64 (P * freq needs more than fp32 at long
    // positions), the reduced angle's sine and cosine in fp32
    __shared__ __align__(16) float cs[2][64];  // read as float4
    if (rope) {
        if (threadIdx.x < 64) {
            const double two_pi = 6.283185307179586476925286766559, inv_two_pi = 0.15915494309189533576888376337251;
            double ang = (double)P * fr;
            ang -= two_pi * floor(ang * inv_two_pi);  // within rounding of [0, 2 pi)
            float sf, cf;
            sincosf((float)ang, &sf, &cf);
            cs[0][threadIdx.x] = cf;
            cs[1][threadIdx.x] = sf;
        }
        __syncthreads();
    }
    // this wave's query heads: normalised, rotated, scaled by 1/sqrt(128)
#pragma unroll
    for (int h = 0; h < HW; h++) {
        head_prep(qv[h], gq, cs, rope, p.eps, lane);
#pragma unroll
        for (int d = 0; d < 16; d++) qv[h][d] *= 0.08838834764831845f;  // 1 / sqrt(128)
    }
    // the chunk holding P: the new key and value used in place of the cache
    // row P, which this block also writes
    uint4 kn0 = make_uint4(0, 0, 0, 0), kn1 = kn0, vn0 = kn0, vn1 = kn0;
    if (hasP) new_token(p, b, g, P, cs, rope, lane, w == 0 && pg == 0, nr, true, kn0, kn1, vn0, vn1);
    // row P of the first groups is the new key / value
#pragma unroll
    for (int u = 0; u < AT_UT; u++) {
        if (start + min(u * 8 + pg, n - 1) == P) {
            xa[u] = kn0;
            ya[u] = kn1;
            va[u] = vn0;
            vb[u] = vn1;
        }
    }
    // later groups: rows of group gi, row P replaced by (nx, ny)
    auto issue_p = [&](const uint4 *M, uint4 (&x)[AT_UT], uint4 (&y)[AT_UT], int gi, const uint4 &nx,
                       const uint4 &ny) {
        issue(M, x, y, gi);
#pragma unroll
        for (int u = 0; u < AT_UT; u++) {
            if (start + min((gi * AT_UT + u) * 8 + pg, n - 1) == P) {
                x[u] = nx;
                y[u] = ny;
            }
        }
    };

    {
        // scores, two load groups in registers
        uint4 xb[AT_UT], yb[AT_UT];
        auto scores = [&](const uint4 (&x)[AT_UT], const uint4 (&y)[AT_UT], int gi) {
#pragma unroll
            for (int u = 0; u < AT_UT; u++) {
                const float s = tile_scores<HW>(qv, x[u], y[u], lane);
                const int jj = (gi * AT_UT + u) * 8 + pg;  // position within [start, end)
                if (jj < n && sub < HW) sc(jj, sub) = s;
            }
        };
        for (int gi = 0; gi < ngrp; gi += 2) {
            if (gi + 1 < ngrp) issue_p(K, xb, yb, gi + 1, kn0, kn1);
            scores(xa, ya, gi);
            if (gi + 2 < ngrp) issue_p(K, xa, ya, gi + 2, kn0, kn1);
            if (gi + 1 < ngrp) scores(xb, yb, gi + 1);
        }
    }
    __syncthreads();

    // per head: the chunk's max, exponentials in place, their sum
    float mh[HW], lh[HW];
#pragma unroll
    for (int h = 0; h < HW; h++) {
        float m = -INFINITY;
        for (int j = lane; j < n; j += 64) m = fmaxf(m, sc(j, h));
        mh[h] = wave_max_f(m);
    }
#pragma unroll
    for (int h = 0; h < HW; h++) {
        float l = 0.f;
        for (int j = lane; j < n; j += 64) {
            const float e = __expf(sc(j, h) - mh[h]);
            sc(j, h) = e;
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
        uint4 xb[AT_UT], yb[AT_UT];
        auto accum = [&](const uint4 (&x)[AT_UT], const uint4 (&y)[AT_UT], int gi) {
#pragma unroll
            for (int u = 0; u < AT_UT; u++) {
                const int jj = (gi * AT_UT + u) * 8 + pg;
                if (jj >= n) continue;  // lanes past the chunk's end add nothing
                float vf[16];
                unpack16(x[u], y[u], vf);
#pragma unroll
                for (int h = 0; h < HW; h++) {
                    const float e = sc(jj, h);
#pragma unroll
                    for (int d = 0; d < 16; d++) o[h][d] = __builtin_fmaf(e, vf[d], o[h][d]);
                }
            }
        };
        for (int gi = 0; gi < ngrp; gi += 2) {
            if (gi + 1 < ngrp) issue_p(V, xb, yb, gi + 1, vn0, vn1);
            accum(va, vb, gi);
            if (gi + 2 < ngrp) issue_p(V, va, vb, gi + 2, vn0, vn1);
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
            float *dst = p.part_o + (((size_t)b * p.Hq + h0 + h) * NC + cl) * AT_D;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int o0 = i < 2 ? 8 * sub + 4 * i : 64 + 8 * sub + 4 * (i - 2);
                *reinterpret_cast<float4 *>(dst + o0) =
                    make_float4(o[h][4 * i], o[h][4 * i + 1], o[h][4 * i + 2], o[h][4 * i + 3]);
            }
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

constexpr int AT_NT = 2;  // non-temporal: the cache is streamed once per call

__device__ __forceinline__ __amdgpu_buffer_rsrc_t at_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

typedef short at_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) at_s16x4 lds_s16x4;
typedef float at_f32x4 __attribute__((ext_vector_type(4)));

// Matrix-core path: 8 query heads per key/value head, full and sliding-window
// layers (queries and the new key rotated on the split lane layout); the same
// partials as attn_chunk, in one pass over the chunk with a running (online)
// softmax.  Two waves; wave w takes the
// 32-position tiles w, w + 2, ... for all 8 heads and keeps its own running
// max, sum and output; the two are merged at the end in wave order.
// v_mfma_f32_16x16x32_bf16 throughout (lane l holds A[l % 16][8 (l / 16) + e],
// B[8 (l / 16) + e][l % 16], e = 0..7, and D[4 (l / 16) + i][l % 16]):
//   scores  S^T = K Q^T per 16-position half: A = 16 keys straight from the
//           cache (lane: position l % 16, dimensions 32 s + 8 (l / 16) ..
//           + 7 for step s), B = the 8 prepared queries split into bf16
//           high and low halves (columns 0-7 and 8-15: the split leaves
//           about 2^-18 of the query), 4 steps over the 128 dimensions;
//           head h's score is column h + column h + 8, one exchange between
//           lanes l and l ^ 8.  Lane l then holds head l % 8 at the 8
//           positions 4 (l / 16) + i and 16 + 4 (l / 16) + i of the tile;
//   values  O += P V: A = the exponentials of those 8 positions split high /
//           low the same way (row l % 16), exactly where the scores left
//           them; B = the same 8 positions of one dimension per lane.  The
//           tile's 32 value rows arrive 1 KB per load instruction (four whole
//           rows), go to a wave-private LDS tile, and come back transposed
//           by ds_read_b64_tr_b16: within a 16-lane group, lane i receives
//           element i % 4 of the 8-byte reads of lanes 4 j + i / 4, j = 0..3,
//           so four lanes reading 4 dimensions each of 4 rows hand every lane
//           one dimension at 4 positions.  Two reads per B operand; 8 MFMAs
//           per tile (16-dimension blocks).  The 16-byte chunk c of tile row
//           r sits at c ^ 2 (r % 4), so the 4 rows a 16-lane group reads
//           fall in distinct banks.
// Output rows: head h's high row h (lanes l / 16 = h / 4) plus its low row
// h + 8 (lanes l / 16 = 2 + h / 4), one exchange between lanes l and l ^ 32.
// Registers: keys two tiles ahead, values one, the output in 32 accumulators:
// one wave per SIMD without spills (a cap at two spills to scratch and runs
// slower), so the chunk plan keeps a call near 512 blocks, two per CU.
__global__ void __launch_bounds__(128) attn_chunk_mf(AttnArgs p) {
    __shared__ uint4 vst[2][32 * 16];  // per wave: one tile of 32 value rows
    __shared__ float qsh[8][AT_D];
    __shared__ uint4 knsh[16], vnsh[16];  // the new key and value, bf16
    __shared__ float mls[2][2][8];        // per wave: running max and sum per head
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: tile offsets go to SGPRs
    const int sub = lane & 7, col = lane & 15, G = lane >> 4;
    const int b = blockIdx.z, g = blockIdx.y;
    const int P = p.pos[b];
    if (P < 0 || P >= p.max_len) return;
    const int lo = attn_lo(p, P);
    const int c0 = (attn_first_chunk(p, P) + blockIdx.x) * p.chunk;
    const int start = max(c0, lo), end = min(c0 + p.chunk, P + 1);  // [start, end)
    if (start >= end) return;
    const int n = end - start, nt = (n + 31) / 32;
    const size_t base = ((size_t)b * p.Hkv + g) * p.max_len;
    // the chunk's valid rows as buffer resources: reads past its end return zero
    const __amdgpu_buffer_rsrc_t krs = at_rsrc(p.k_cache + (base + start) * AT_D, (uint32_t)n * 256u);
    const __amdgpu_buffer_rsrc_t vrs = at_rsrc(p.v_cache + (base + start) * AT_D, (uint32_t)n * 256u);
    const int vo_k = col * 256 + G * 16, vo_v = G * 256 + col * 16;
    // keys of tile t: k[4 ph + s] = half ph, step s (lane: position
    // 32 t + 16 ph + l % 16, dimensions 32 s + 8 (l / 16) ..); values: v[i] =
    // rows 4 i .. 4 i + 3 (lane: row 4 i + l / 16, chunk l % 16)
    auto issue_k = [&](uint4 (&k)[8], int t) {
#pragma unroll
        for (int ph = 0; ph < 2; ph++)
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const auto c = __builtin_amdgcn_raw_buffer_load_b128(krs, vo_k + 64 * s, 8192 * t + 4096 * ph, AT_NT);
                k[4 * ph + s] = make_uint4(c[0], c[1], c[2], c[3]);
            }
    };
    auto issue_v = [&](uint4 (&v)[8], int t) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const auto c = __builtin_amdgcn_raw_buffer_load_b128(vrs, vo_v + 1024 * (i & 3), 8192 * t + 4096 * (i >> 2), AT_NT);
            v[i] = make_uint4(c[0], c[1], c[2], c[3]);
        }
    };
    // the first tile's keys and values are requested before anything else
    uint4 k0[8], v0[8], k1[8], v1[8];
    if (w < nt) {
        issue_k(k0, w);
        issue_v(v0, w);
    }
    // this wave's raw query heads (4 w .. 4 w + 3), their gains, the new key
    // and value (the chunk holding P) and the rotary frequencies, all requested
    // before the rotary table is built (split layout: lane s holds dimensions
    // 8 s .. + 7 and 64 + 8 s .. + 7)
    const bool rope = p.window > 0;
    const double fr = rope && threadIdx.x < 64 ? p.rope_freq[threadIdx.x] : 0.0;
    float qx[4][16], gq[16];
#pragma unroll
    for (int h = 0; h < 4; h++) load16(p.q + ((size_t)b * p.Hq + g * 8 + 4 * w + h) * AT_D, sub, qx[h], true);
    load16(p.q_norm_w, sub, gq, true);
    const bool hasP = end == P + 1;
    NewRaw nr;
    if (hasP) new_token_load(p, b, g, lane, nr, true);
    __shared__ __align__(16) float cs[2][64];  // read as float4
    if (rope) {
        if (threadIdx.x < 64) {
            const double two_pi = 6.283185307179586476925286766559, inv_two_pi = 0.15915494309189533576888376337251;
            double ang = (double)P * fr;
            ang -= two_pi * floor(ang * inv_two_pi);  // within rounding of [0, 2 pi)
            float sf, cf;
            sincosf((float)ang, &sf, &cf);
            cs[0][threadIdx.x] = cf;
            cs[1][threadIdx.x] = sf;
        }
        __syncthreads();
    }
    // the 8 prepared queries and the new key and value through LDS
#pragma unroll
    for (int h = 0; h < 4; h++) {
        head_prep(qx[h], gq, cs, rope, p.eps, lane);
        if (lane < 8) {
#pragma unroll
            for (int d = 0; d < 16; d++)
                qsh[4 * w + h][d < 8 ? 8 * sub + d : 56 + 8 * sub + d] = qx[h][d] * 0.08838834764831845f;  // 1/sqrt(128)
        }
    }
    if (hasP) {
        uint4 nk0, nk1, nv0, nv1;
        new_token(p, b, g, P, cs, rope, lane, w == 0 && lane < 8, nr, true, nk0, nk1, nv0, nv1);
        if (w == 0 && lane < 8) {
            knsh[sub] = nk0;
            knsh[8 + sub] = nk1;
            vnsh[sub] = nv0;
            vnsh[8 + sub] = nv1;
        }
    }
    __syncthreads();
    // B operands of the scores: column col = head col % 8, high / low half
    at_bf16x8 bq[4];
#pragma unroll
    for (int s = 0; s < 4; s++) {
        const float *qr = &qsh[col & 7][32 * s + 8 * G];
        uint32_t wd[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            float x0 = qr[2 * e], x1 = qr[2 * e + 1];
            if (col >= 8) {  // low half: what the high half leaves
                x0 -= __uint_as_float((uint32_t)to_bf16_rne(x0) << 16);
                x1 -= __uint_as_float((uint32_t)to_bf16_rne(x1) << 16);
            }
            wd[e] = pack_bf16x2(x0, x1);
        }
        bq[s] = __builtin_bit_cast(at_bf16x8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
    }

    uint4 *tile = vst[w];
    at_f32x4 oacc[8];
#pragma unroll
    for (int c = 0; c < 8; c++) oacc[c] = at_f32x4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;  // head l % 8
    // B operand of values block c: dimension 16 c + l % 16 at the lane's 8
    // positions (read 0: rows 4 (l / 16) + j, read 1: rows 16 + 4 (l / 16) + j)
    const int rq = (lane >> 2) & 3, q = lane & 3;
    auto b_val = [&](int c) -> at_bf16x8 {
        const int r0 = 4 * G + rq;  // rows r0 and r0 + 16, both with r % 4 == rq
        const int ch = (2 * c + (q >> 1)) ^ (2 * rq);
        const char *t8 = reinterpret_cast<const char *>(tile) + 8 * (q & 1);
        const at_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t8 + (r0 * 16 + ch) * 16));
        const at_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t8 + ((r0 + 16) * 16 + ch) * 16));
        return __builtin_bit_cast(at_bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // tile t; next_v requests the values of the wave's next tile once this
    // tile's have left their registers
    auto process = [&](uint4 (&k)[8], const uint4 (&v)[8], int t, auto next_v) {
        // value rows to LDS (rows past the chunk's end arrive as zero); in the
        // chunk's last tile row P is the new value
        const bool last = t == nt - 1;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int r = 4 * i + G;
            uint4 x = v[i];
            if (last && start + 32 * t + r == P) x = vnsh[col];
            tile[r * 16 + (col ^ (2 * (r & 3)))] = x;
        }
        next_v();
        // scores of the two halves
        float sc[8];
#pragma unroll
        for (int ph = 0; ph < 2; ph++) {
            if (last && start + 32 * t + 16 * ph + col == P) {
#pragma unroll
                for (int s = 0; s < 4; s++) k[4 * ph + s] = knsh[4 * s + G];
            }
            at_f32x4 acc = at_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; s++)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(at_bf16x8, k[4 * ph + s]), bq[s], acc, 0,
                                                             0, 0);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float s2 = acc[i] + at_xor(acc[i], 3);  // high + low column
                const int jj = 32 * t + 16 * ph + 4 * G + i;
                sc[4 * ph + i] = jj < n ? s2 : -INFINITY;
            }
        }
        // running max, rescale, exponentials
        float tm = sc[0];
#pragma unroll
        for (int e = 1; e < 8; e++) tm = fmaxf(tm, sc[e]);
        tm = fmaxf(tm, at_xor(tm, 4));
        tm = fmaxf(tm, at_xor(tm, 5));
        const float mnew = fmaxf(mrun, tm);
        const float alpha = __expf(mrun - mnew);  // 0 on the first tile
        mrun = mnew;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
            // output row 4 (l / 16) + i belongs to head 4 ((l / 16) & 1) + i
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float a = __shfl(alpha, (lane & 0x30) | (4 * (G & 1) + i), 64);
#pragma unroll
                for (int c = 0; c < 8; c++) oacc[c][i] *= a;
            }
        }
        float pe[8], ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            pe[e] = __expf(sc[e] - mnew);
            ps += pe[e];
        }
        lrun = lrun * alpha + ps;
        uint32_t wd[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            float x0 = pe[2 * e], x1 = pe[2 * e + 1];
            if (col >= 8) {
                x0 -= __uint_as_float((uint32_t)to_bf16_rne(x0) << 16);
                x1 -= __uint_as_float((uint32_t)to_bf16_rne(x1) << 16);
            }
            wd[e] = pack_bf16x2(x0, x1);
        }
        const at_bf16x8 a = __builtin_bit_cast(at_bf16x8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
#pragma unroll
        for (int c = 0; c < 8; c++) oacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b_val(c), oacc[c], 0, 0, 0);
    };
    // keys two tiles ahead, values one
    for (int t = w; t < nt; t += 4) {
        if (t + 2 < nt) issue_k(k1, t + 2);
        process(k0, v0, t, [&] {
            if (t + 2 < nt) issue_v(v1, t + 2);
        });
        if (t + 4 < nt) issue_k(k0, t + 4);
        if (t + 2 < nt)
            process(k1, v1, t + 2, [&] {
                if (t + 4 < nt) issue_v(v0, t + 4);
            });
    }
    // this wave's sum over its lanes' positions; high + low output rows
    lrun += at_xor(lrun, 4);
    lrun += at_xor(lrun, 5);
    float o[8][4];
#pragma unroll
    for (int c = 0; c < 8; c++)
#pragma unroll
        for (int i = 0; i < 4; i++) o[c][i] = oacc[c][i] + at_xor(oacc[c][i], 5);
    if (lane < 8) {
        mls[w][0][lane] = mrun;
        mls[w][1][lane] = lrun;
    }
    // wave 1's output (lanes 0-31: heads 4 (l / 16) + i, dimension 16 c + l % 16)
    // reaches wave 0 through its own, finished tile
    float *xs = reinterpret_cast<float *>(vst[1]);
    if (w == 1 && lane < 32) {
#pragma unroll
        for (int c = 0; c < 8; c++)
#pragma unroll
            for (int i = 0; i < 4; i++) xs[(4 * c + i) * 32 + lane] = o[c][i];
    }
    __syncthreads();
    if (w != 0) return;
    const int NC = p.n_chunks;
    const int cl = blockIdx.x;
    if (lane < 32) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int h = 4 * G + i;
            const float m0 = mls[0][0][h], m1 = mls[1][0][h];
            const float M = fmaxf(m0, m1);
            const float s0 = __expf(m0 - M), s1 = __expf(m1 - M);
            float *dst = p.part_o + (((size_t)b * p.Hq + g * 8 + h) * NC + cl) * AT_D + col;
#pragma unroll
            for (int c = 0; c < 8; c++) dst[16 * c] = s0 * o[c][i] + s1 * xs[(4 * c + i) * 32 + lane];
        }
    }
    if (lane < 8) {
        const float m0 = mls[0][0][lane], m1 = mls[1][0][lane];
        const float M = fmaxf(m0, m1);
        const size_t at = ((size_t)b * p.Hq + g * 8 + lane) * NC + cl;
        p.part_m[at] = M;
        p.part_l[at] = __expf(m0 - M) * mls[0][1][lane] + __expf(m1 - M) * mls[1][1][lane];
    }
}

// one block per (sequence, query head); wave w merges chunks w, w + 16, ...
// with a running max (one round of loads: four chunks in flight per wave),
// lane covers dimensions 2 lane, 2 lane + 1; the waves' (max, sum, output)
// and the sink are then merged in wave order
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
    // this wave's chunks: running max m, sum L and output acc
    float m = -INFINITY, L = 0.f;
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
            const float mn = fmaxf(m, mk[u]);
            const float a = __expf(m - mn), e = __expf(mk[u] - mn);  // a = 0 for the first chunk
            L = a * L + e * lk[u];
            acc.x = a * acc.x + e * vk[u].x;
            acc.y = a * acc.y + e * vk[u].y;
            m = mn;
        }
    }
    if (lane == 0) {
        red[w][0] = m;
        red[w][1] = L;
    }
    ov[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
        // M = max(z, max_w m_w); waves without chunks carry m = -inf, weight 0
        const float z = p.sinks[h];
        float M = z;
#pragma unroll
        for (int i = 0; i < AT_COMB_WAVES; i++) M = fmaxf(M, red[i][0]);
        float Ls = __expf(z - M);
        float2 o = make_float2(0.f, 0.f);
#pragma unroll
        for (int i = 0; i < AT_COMB_WAVES; i++) {
            const float e = __expf(red[i][0] - M);
            Ls += e * red[i][1];
            o.x += e * ov[i][lane].x;
            o.y += e * ov[i][lane].y;
        }
        const float inv = 1.0f / Ls;
        reinterpret_cast<float2 *>(p.out + ((size_t)b * p.Hq + h) * AT_D)[lane] = make_float2(o.x * inv, o.y * inv);
    }
}

template <typename Kern>
void launch_grid(Kern kern, int threads, const AttnArgs &p, hipStream_t st) {
    const dim3 grid(p.n_chunks, p.Hkv, p.B);
    if (p.ev)
        hipExtLaunchKernelGGL(kern, grid, dim3(threads), 0, st, p.ev[0], p.ev[1], 0, p);
    else
        hipLaunchKernelGGL(kern, grid, dim3(threads), 0, st, p);
}

template <int HW, int WV>
void launch_chunks(const AttnArgs &p, hipStream_t st) {
    launch_grid(attn_chunk<HW, WV>, 64 * WV, p, st);
}

}  // namespace

// Chunk size: a sliding window takes 64 positions on the matrix-core path
// (one tile per wave; 513 positions spread over 9-10 blocks per key/value
// head; measured 11.7 us per layer against 11.6 for 32 and 13.5 for 128) and
// 32 on the vector path (one load group of keys and one of values in flight).  Full attention: the smallest power of
// two in [64, 1024] that keeps the blocks of a call at the cache's full
// length to about 512 on the matrix-core path (one wave per SIMD, two blocks
// per CU: every block resident at once) and about 1024 on the vector path.
int attn_chunk_size(int window, int max_len, int B, int Hq, int Hkv) {
    if (window > 0) return attn_uses_mfma(window, Hq, Hkv) ? 64 : 32;
    const long long target = attn_uses_mfma(window, Hq, Hkv) ? 512 : 1024;
    int c = 64;
    while (c < AT_CMAX && (long long)((max_len + c - 1) / c) * B * Hkv > target) c *= 2;
    return c;
}

bool attn_uses_mfma(int window, int Hq, int Hkv) { return Hq == 8 * Hkv; }

int attn_chunk_slots(int window, int max_len, int chunk) {
    // a window of W positions spans at most ceil((W - 1) / chunk) + 1 chunks
    const int all = (max_len + chunk - 1) / chunk;
    if (window <= 0) return all;
    return min(all, (window - 1 + chunk - 1) / chunk + 1);
}

hipError_t launch_attn(const AttnArgs &a, hipStream_t st) {
    AttnArgs p = a;
    const int grp = p.Hq / p.Hkv;
    // groups of 8 on the matrix cores (measured at 128k: 84.4 us on the
    // vector path, 46.9 us here; windows of 513: 12.2 against 11.7 us)
    if (attn_uses_mfma(p.window, p.Hq, p.Hkv))
        launch_grid(attn_chunk_mf, 128, p, st);
    else if (grp == 8)
        launch_chunks<4, 2>(p, st);
    else if (grp == 4)
        launch_chunks<4, 1>(p, st);
    else if (grp == 2)
        launch_chunks<2, 1>(p, st);
    else
        launch_chunks<1, 1>(p, st);
    const dim3 gc(p.B, p.Hq);
    if (p.ev)
        hipExtLaunchKernelGGL(attn_combine, gc, dim3(64 * AT_COMB_WAVES), 0, st, p.ev[2], p.ev[3], 0, p);
    else
        hipLaunchKernelGGL(attn_combine, gc, dim3(64 * AT_COMB_WAVES), 0, st, p);
    return hipGetLastError();
}

}  // namespace moe
