// Prefill path of the MoE layer: route every token, group the (token, slot)
// pairs by expert, run each expert as a grouped GEMM on the matrix cores, and
// combine each token's rows in a fixed order.
//
// What is computed is the same layer as the decode path ("Recursive Flint
// 40B-A2.5B", section "The architecture is a memory-bandwidth argument": 256
// routed experts, 6 chosen per token, one always-on shared expert), applied to
// many tokens at once.  With thousands of tokens each active expert sees a
// matrix of tokens, so the expert projections become dense contractions and
// run on MFMA (fp16 operands, fp32 accumulation).
//
// Kernels (one stream, in order):
//   pf_router_gemm  (bf16 tokens) partial logits x Wr^T of ksplit reduction
//               parts by a tiled bf16 MFMA GEMM, fp16 copy of x
//   pf_logits   (fp32 tokens) logits = x Wr^T + bias by bf16 MFMA on a
//               two-term bf16 split of x, fp16 copy of x
//   pf_topk     logits (sum of the parts + bias), per-token top-k,
//               per-expert 64-token bitmasks
//   pf_scan     per-expert counts and word prefixes of the masks, row
//               offsets, tile table
//   pf_scatter  position of every (token, slot) pair in its expert's rows
//   pf_gemm<0>  H = silu(X Wg^T) * (X Wu^T) per expert (fp16 H)
//   pf_gemm<1>  O = coef * (H Wd^T) per expert (fp16 O, like H)
//   pf_ffn_q4   (4-bit weights, in place of the two above) both GEMMs in
//               one dispatch: a tile's down blocks start once its gate/up
//               blocks have stored h
//   pf_combine  y[t] = sum of t's rows of O in slot order
// No floating-point atomics: integer/bitwise atomics only, so results do not
// depend on scheduling.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_prefill.h"

namespace moe {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int PF_BM = 128;          // rows (token slots) per tile of pf_gemm (and the bound of the tile count)
constexpr int PQ_BM = 128;          // rows per tile of the 4-bit GEMMs (pf_ffn_q4)
constexpr int PF_THREADS = 256;     // 4 waves
constexpr int PF_MAX_TOPK = 8;

struct PfTile {
    int e, row0, rows;
};

// Workspace layout (byte offsets), shared by the host sizing and the launcher.
struct PfWs {
    size_t x16, logits, part, idx, w, mask, wp, off, tiles, meta, done, perm_tok, perm_w, pos, h, o, total;
    int NW, R, tiles_max, ksplit;
};

size_t al(size_t v) { return (v + 255) & ~(size_t)255; }

constexpr int RG_BT = 64;  // tokens per block of the bf16 router GEMM

// Reduction parts of the bf16 router GEMM: the fewest (1, 2, 4 or 8: a
// divisor of the 8 XCDs) that give 256 blocks, one 32-input step each at least.
int pf_router_splits(int T, int D) {
    const int ntt = (T + RG_BT - 1) / RG_BT, nk = D / 32;
    int s = 1;
    while (s < 8 && ntt * s < 256 && 2 * s <= nk) s *= 2;
    return s;
}

PfWs pf_layout(int D, int F, int E, int S, int K, int T) {
    PfWs L{};
    L.NW = (T + 63) / 64;
    L.R = T * (K + S);
    L.tiles_max = (L.R + PF_BM - 1) / PF_BM + E + S;
    L.ksplit = pf_router_splits(T, D);
    size_t o = 0;
    L.x16 = o; o = al(o + (size_t)T * D * 2);
    L.logits = o; o = al(o + (size_t)T * E * 4);
    L.part = o; o = al(o + (size_t)L.ksplit * T * E * 4);
    L.idx = o; o = al(o + (size_t)T * K * 4);
    L.w = o; o = al(o + (size_t)T * K * 4);
    L.mask = o; o = al(o + (size_t)E * L.NW * 8);
    L.wp = o; o = al(o + (size_t)E * L.NW * 4);
    L.off = o; o = al(o + (size_t)(E + S + 1) * 4);
    L.tiles = o; o = al(o + (size_t)L.tiles_max * sizeof(PfTile));
    L.meta = o; o = al(o + 16 * 4);
    L.done = o; o = al(o + (size_t)L.tiles_max * 4);
    L.perm_tok = o; o = al(o + (size_t)L.R * 4);
    L.perm_w = o; o = al(o + (size_t)L.R * 4);
    L.pos = o; o = al(o + (size_t)T * (K + S) * 4);
    L.h = o; o = al(o + (size_t)L.R * F * 2);
    L.o = o; o = al(o + (size_t)L.R * D * 2);
    L.total = o;
    return L;
}

template <typename T>
T *wsp(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

struct PfParams {
    int D, F, E, S, K, T, act, NW, R, tiles_max, want_x16;
    int ksplit;          // pf_router_gemm: reduction parts
    int BM;              // token rows per GEMM tile (tile table)
    int g1;              // pf_ffn_q4: blocks of the gate/up role
    hipEvent_t *ev;
    size_t expert_bytes;
    const void *x;
    const uint16_t *router;
    const float *bias;
    const uint8_t *experts;
    const float *tscale;
    float *y;
    int32_t *idx_out;
    float *w_out;
    float *logits_out;
    float *logits;       // [T, E]: logits_out, or workspace
    float *part;         // [ksplit, T, E]: partial logits of the bf16 router GEMM
    _Float16 *x16;
    int32_t *idx;
    float *w;
    unsigned long long *mask;
    int32_t *wp;
    int32_t *off;
    PfTile *tiles;
    int32_t *meta;
    int32_t *tile_done;  // pf_ffn_q4: gate/up blocks done per tile (zeroed by pf_scan)
    int32_t *perm_tok;
    float *perm_w;
    int32_t *pos;
    _Float16 *h;
    _Float16 *o;         // [R, D] down-projection rows (coefficient applied), fp16
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// fp32 -> (hi, lo) bf16 pair with hi + lo = x up to 2^-16 |x| (both rounded to nearest)
__device__ __forceinline__ uint32_t f2bf_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// pf_logits: logits[t, e] = x[t] . Wr[e] (+ bias[e]) by bf16 MFMA.  One block
// = 32 experts x 32 tokens; its KS waves split the reduction into KS parts,
// summed in wave order through LDS.  Blocks of the first expert column also
// write the fp16 copy of x (operand of the expert GEMMs).  An fp32 input is
// split x = hi + lo into two bf16 parts, both accumulated.
// ---------------------------------------------------------------------------
constexpr int PF_LG_CH = 8;  // reduction steps of 16 per load batch

template <int ACT, int KS>
__global__ void __launch_bounds__(64 * KS) pf_logits(PfParams p) {
    __shared__ float red[KS][32][33];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int D = p.D, E = p.E, T = p.T;
    const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
    const int NKS = D / 16;                                     // reduction steps
    const int ks0 = wave * NKS / KS, ks1 = (wave + 1) * NKS / KS;  // this wave's part
    const uint16_t *wrow = p.router + (size_t)min(e0 + l32, E - 1) * D + 8 * g;
    const int trow = min(t0 + l32, T - 1);
    const bool write_x16 = p.want_x16 && blockIdx.y == 0 && t0 + l32 < T;
    f32x16_t acc;
#pragma unroll
    for (int j = 0; j < 16; j++) acc[j] = 0.f;
    for (int kc = ks0; kc < ks1; kc += PF_LG_CH) {
        // one batch: every load first, then the MFMAs
        uint4 av[PF_LG_CH];
        bf16x8_t bh[PF_LG_CH], bl[PF_LG_CH];
#pragma unroll
        for (int c = 0; c < PF_LG_CH; c++) {
            const int k0 = 16 * min(kc + c, ks1 - 1);
            const bool live = kc + c < ks1;
            av[c] = *reinterpret_cast<const uint4 *>(wrow + k0);
            if (ACT == 0) {
                const float *xs = static_cast<const float *>(p.x) + (size_t)trow * D + k0 + 8 * g;
                const float4 u0 = *reinterpret_cast<const float4 *>(xs);
                const float4 u1 = *reinterpret_cast<const float4 *>(xs + 4);
                const float xv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
                uint32_t hi[4], lo[4];
                half8_t hv;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t h0 = f2bf_rne(xv[2 * j]), h1 = f2bf_rne(xv[2 * j + 1]);
                    const uint32_t l0 = f2bf_rne(xv[2 * j] - __uint_as_float(h0 << 16));
                    const uint32_t l1 = f2bf_rne(xv[2 * j + 1] - __uint_as_float(h1 << 16));
                    hi[j] = h0 | (h1 << 16);
                    lo[j] = l0 | (l1 << 16);
                    hv[2 * j] = (_Float16)xv[2 * j];
                    hv[2 * j + 1] = (_Float16)xv[2 * j + 1];
                }
                bh[c] = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
                bl[c] = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
                if (write_x16 && live) *reinterpret_cast<half8_t *>(p.x16 + (size_t)trow * D + k0 + 8 * g) = hv;
            } else {
                const uint4 r = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.x) + (size_t)trow * D +
                                                                 k0 + 8 * g);
                bh[c] = as_bf16x8(r);
                if (write_x16 && live) {
                    const uint32_t ww[4] = {r.x, r.y, r.z, r.w};
                    half8_t hv;
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        hv[2 * j] = (_Float16)bf16lo(ww[j]);
                        hv[2 * j + 1] = (_Float16)bf16hi(ww[j]);
                    }
                    *reinterpret_cast<half8_t *>(p.x16 + (size_t)trow * D + k0 + 8 * g) = hv;
                }
            }
        }
#pragma unroll
        for (int c = 0; c < PF_LG_CH; c++) {
            if (kc + c >= ks1) break;
            const bf16x8_t a = as_bf16x8(av[c]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh[c], acc, 0, 0, 0);
            if (ACT == 0) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl[c], acc, 0, 0, 0);
        }
    }
    // acc[j] = partial logit of expert e0 + 8 (j/4) + 4 g + j%4, token t0 + l32
#pragma unroll
    for (int j = 0; j < 16; j++) red[wave][8 * (j >> 2) + 4 * g + (j & 3)][l32] = acc[j];
    __syncthreads();
    for (int i = tid; i < 32 * 32; i += 64 * KS) {
        const int el = i >> 5, tl = i & 31;
        const int e = e0 + el, t = t0 + tl;
        if (e >= E || t >= T) continue;
        float v = red[0][el][tl];
#pragma unroll
        for (int w = 1; w < KS; w++) v += red[w][el][tl];
        p.logits[(size_t)t * E + e] = v + (p.bias ? p.bias[e] : 0.f);
    }
}

// ---------------------------------------------------------------------------
// pf_topk: one block = 16 tokens (a quarter of a 64-token mask word), each
// wave PF_TOPK_TPW of them (tokens w, w + waves, ...).  Logits: NP = 0 reads finished ones
// (bias included); NP > 0 sums the bf16 router GEMM's NP partials in part
// order and adds the bias.  Then top-k with renormalised weights, and the
// block's 16 bits of every expert's token bitmask (the grid covers whole
// words, so tokens past T get zero bits).
// ---------------------------------------------------------------------------
constexpr int PF_TOPK_TOK = 16;
constexpr int PF_TOPK_TPW = 1;                                 // tokens per wave
constexpr int PF_TOPK_WAVES = PF_TOPK_TOK / PF_TOPK_TPW;
constexpr int PF_TOPK_THREADS = 64 * PF_TOPK_WAVES;

template <int NP>
__global__ void __launch_bounds__(PF_TOPK_THREADS) pf_topk(PfParams p) {
    __shared__ uint32_t smask[256];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t0 = blockIdx.x * PF_TOPK_TOK;
    const int T = p.T, E = p.E;
    for (int i = tid; i < 256; i += PF_TOPK_THREADS) smask[i] = 0u;
    // the wave's tokens' logits, all loads in flight together
    float lv[PF_TOPK_TPW][4];
    if (NP == 0) {
#pragma unroll
        for (int i = 0; i < PF_TOPK_TPW; i++)
            wave_topk_load(p.logits + (size_t)min(t0 + wave + PF_TOPK_WAVES * i, T - 1) * E, E, lv[i]);
    } else {
        float pv[PF_TOPK_TPW][NP][4];
#pragma unroll
        for (int i = 0; i < PF_TOPK_TPW; i++) {
            const int t = min(t0 + wave + PF_TOPK_WAVES * i, T - 1);
#pragma unroll
            for (int j = 0; j < NP; j++)
#pragma unroll
                for (int k = 0; k < 4; k++) pv[i][j][k] = p.part[((size_t)j * T + t) * E + min(lane + 64 * k, E - 1)];
        }
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float bk = p.bias ? p.bias[min(lane + 64 * k, E - 1)] : 0.f;
#pragma unroll
            for (int i = 0; i < PF_TOPK_TPW; i++) {
                float v = pv[i][0][k];
#pragma unroll
                for (int j = 1; j < NP; j++) v += pv[i][j][k];
                lv[i][k] = v + bk;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PF_TOPK_TPW; i++) {
        const int tl = wave + PF_TOPK_WAVES * i, t = t0 + tl;
        if (t >= T) break;
        if (NP > 0 && p.logits_out) {
#pragma unroll
            for (int k = 0; k < 4; k++)
                if (lane + 64 * k < E) p.logits_out[(size_t)t * E + lane + 64 * k] = lv[i][k];
        }
        int e;
        float wi;
        wave_topk_regs(lv[i], E, p.K, &e, &wi);
        if (lane < p.K) {
            p.idx[(size_t)t * p.K + lane] = e;
            p.w[(size_t)t * p.K + lane] = wi;
            if (p.idx_out) p.idx_out[(size_t)t * p.K + lane] = e;
            if (p.w_out) p.w_out[(size_t)t * p.K + lane] = wi;
            atomicOr(&smask[e], 1u << tl);
        }
    }
    __syncthreads();
    // 16-bit piece blockIdx.x % 4 of word blockIdx.x / 4 (little-endian words)
    for (int e = tid; e < E; e += PF_TOPK_THREADS)
        reinterpret_cast<uint16_t *>(p.mask)[(size_t)e * 4 * p.NW + blockIdx.x] = (uint16_t)smask[e];
}

// ---------------------------------------------------------------------------
// pf_x16: fp16 copy of x (the router kernel makes it otherwise)
// ---------------------------------------------------------------------------
template <int ACT>
__global__ void __launch_bounds__(PF_THREADS) pf_x16(PfParams p) {
    const size_t i = (size_t)blockIdx.x * PF_THREADS + threadIdx.x;
    if (i >= (size_t)p.T * p.D / 8) return;
    half8_t hv;
    if (ACT == 0) {
        const float4 a = reinterpret_cast<const float4 *>(p.x)[2 * i];
        const float4 b = reinterpret_cast<const float4 *>(p.x)[2 * i + 1];
        hv[0] = (_Float16)a.x; hv[1] = (_Float16)a.y; hv[2] = (_Float16)a.z; hv[3] = (_Float16)a.w;
        hv[4] = (_Float16)b.x; hv[5] = (_Float16)b.y; hv[6] = (_Float16)b.z; hv[7] = (_Float16)b.w;
    } else {
        const uint4 r = reinterpret_cast<const uint4 *>(p.x)[i];
        const uint32_t ww[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            hv[2 * j] = (_Float16)bf16lo(ww[j]);
            hv[2 * j + 1] = (_Float16)bf16hi(ww[j]);
        }
    }
    reinterpret_cast<half8_t *>(p.x16)[i] = hv;
}

// ---------------------------------------------------------------------------
// pf_mask_given: per-expert token bitmasks from a caller-given routing (one
// block per 64 tokens); indices outside [0, E) select nothing.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(PF_THREADS) pf_mask_given(PfParams p) {
    __shared__ unsigned long long smask[256];
    const int tid = threadIdx.x;
    smask[tid] = 0ull;
    __syncthreads();
    const int t0 = blockIdx.x * 64;
    for (int i = tid; i < 64 * p.K; i += PF_THREADS) {
        const int tl = i / p.K, j = i % p.K, t = t0 + tl;
        if (t >= p.T) continue;
        const int e = p.idx[(size_t)t * p.K + j];
        if (e >= 0 && e < p.E) atomicOr(&smask[e], 1ull << tl);
    }
    __syncthreads();
    if (tid < p.E) p.mask[(size_t)tid * p.NW + blockIdx.x] = smask[tid];
}

// ---------------------------------------------------------------------------
// pf_scan: one block of 1024.  Rows are ordered routed expert 0..E-1, then
// shared.  Per routed expert (one wave each): prefix popcounts of its mask
// words; then block-wide exclusive scans of the row counts and tile counts
// (the tile table lists every full tile of p.BM rows, then the partial ones).
// ---------------------------------------------------------------------------
constexpr int PF_SCAN_THREADS = 1024;

// exclusive scan over the block (one value per thread, 1024 threads)
__device__ __forceinline__ int block_excl_scan(int v, int *tmp16, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) tmp16[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int t = lane < 16 ? tmp16[lane] : 0;
        const int ti = wave_incl_scan(t);
        if (lane < 16) tmp16[lane] = ti - t;  // exclusive wave offsets
        if (lane == 15) *total = ti;
    }
    __syncthreads();
    const int r = tmp16[wave] + incl - v;
    __syncthreads();
    return r;
}

__global__ void __launch_bounds__(PF_SCAN_THREADS) pf_scan(PfParams p) {
    __shared__ int cnt[PF_SCAN_THREADS];
    __shared__ int tmp16[16];
    __shared__ int tot_rows, tot_tiles;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_exp = p.E + p.S;
    // the fused GEMM's per-tile counters start at zero on every call
    for (int i = tid; i < p.tiles_max; i += PF_SCAN_THREADS) p.tile_done[i] = 0;
    // per routed expert (wave w: experts w, w + 16, ...): word prefixes, 64
    // words per pass; the words of the wave's 16 experts are loaded together
    // (32-bit element offsets from the scalar base keep one register per address)
    constexpr int EPW = 16;
    for (int e0 = wave; e0 < p.E; e0 += 16 * EPW) {
        int carry[EPW];
#pragma unroll
        for (int i = 0; i < EPW; i++) carry[i] = 0;
        for (int w0 = 0; w0 < p.NW; w0 += 64) {
            const int w = w0 + lane;
            // every load issued before the first use, from clamped indices
            // (a load under a condition gets a wait of its own)
            unsigned long long mw[EPW];
#pragma unroll
            for (int i = 0; i < EPW; i++) {
                const int e = min(e0 + 16 * i, p.E - 1);
                mw[i] = p.mask[(uint32_t)(e * p.NW + min(w, p.NW - 1))];
            }
            int c[EPW];
#pragma unroll
            for (int i = 0; i < EPW; i++) c[i] = (e0 + 16 * i < p.E && w < p.NW) ? __popcll(mw[i]) : 0;
#pragma unroll
            for (int i = 0; i < EPW; i++) {
                const int e = e0 + 16 * i;
                const int incl = wave_incl_scan(c[i]);
                if (e < p.E && w < p.NW) p.wp[(uint32_t)(e * p.NW + w)] = carry[i] + incl - c[i];
                carry[i] += __shfl(incl, 63, 64);
            }
        }
#pragma unroll
        for (int i = 0; i < EPW; i++)
            if (lane == 0 && e0 + 16 * i < p.E) cnt[e0 + 16 * i] = carry[i];
    }
    __syncthreads();
    const int my_n = tid < p.E ? cnt[tid] : (tid < n_exp ? p.T : 0);
    // full tiles of every expert first, then the partial ones (expert order)
    const int BM = p.BM;
    const int my_full = my_n / BM, my_part = my_n % BM ? 1 : 0;
    const int off = block_excl_scan(my_n, tmp16, &tot_rows);
    const int foff = block_excl_scan(my_full, tmp16, &tot_tiles);
    const int n_full = tot_tiles;
    __syncthreads();
    const int poff = block_excl_scan(my_part, tmp16, &tot_tiles);
    if (tid < n_exp) p.off[tid] = off;
    if (tid == 0) {
        p.off[n_exp] = tot_rows;
        p.meta[0] = n_full + tot_tiles;
        p.meta[1] = tot_rows;
        p.meta[2] = n_full;
    }
    if (tid < n_exp) {
        for (int i = 0; i < my_full; i++) {
            PfTile t;
            t.e = tid;
            t.row0 = off + i * BM;
            t.rows = BM;
            p.tiles[foff + i] = t;
        }
        if (my_part) {
            PfTile t;
            t.e = tid;
            t.row0 = off + my_full * BM;
            t.rows = my_n - my_full * BM;
            p.tiles[n_full + poff] = t;
        }
    }
}

// ---------------------------------------------------------------------------
// pf_scatter: one thread per (token, slot) pair.  The rank of token t in
// routed expert e's rows is the number of tokens before t that chose e
// (prefix popcount); shared expert s takes row t of its block.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(PF_THREADS) pf_scatter(PfParams p) {
    const int KS = p.K + p.S;
    const int i = blockIdx.x * PF_THREADS + threadIdx.x;
    if (i >= p.T * KS) return;
    const int t = i / KS, j = i % KS;
    int r;
    float wt;
    if (j < p.K) {
        // the token's whole index and weight rows in one round trip (top_k <= 8)
        const int32_t *ti = p.idx + (size_t)t * p.K;
        const float *tw = p.w + (size_t)t * p.K;
        int32_t tk[8];
        float wk[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            tk[k] = ti[min(k, p.K - 1)];
            wk[k] = tw[min(k, p.K - 1)];
        }
        int e = tk[0];
#pragma unroll
        for (int k = 1; k < 8; k++) e = k == j ? tk[k] : e;
        // caller routing may hold invalid indices (no row) or repeat an index:
        // the token's first slot naming e owns the row and carries the weights
        // of all its slots naming e, added in slot order; later ones get none
        bool first = e >= 0 && e < p.E;
#pragma unroll
        for (int k = 0; k < 8; k++) first = first && !(k < j && tk[k] == e);
        if (!first) {
            p.pos[i] = -1;
            return;
        }
        const size_t mi = (size_t)e * p.NW + (t >> 6);
        const unsigned long long below = (t & 63) ? ((1ull << (t & 63)) - 1ull) : 0ull;
        r = p.off[e] + p.wp[mi] + __popcll(p.mask[mi] & below);
        wt = 0.f;
#pragma unroll
        for (int k = 0; k < 8; k++) wt += (k >= j && k < p.K && tk[k] == e) ? wk[k] : 0.f;
    } else {
        r = p.off[p.E + j - p.K] + t;
        wt = 1.f;
    }
    p.perm_tok[r] = t;
    p.perm_w[r] = wt;
    p.pos[i] = r;
}

// The grouped-GEMM helpers use device-only types (buffer resources) and are
// compiled for the device side of the build only; the host side sees the
// kernels' launch stubs.
#if defined(__HIP_DEVICE_COMPILE__)

// ---------------------------------------------------------------------------
// Weight fragments for v_mfma_f32_32x32x16_f16.  One call covers 32 inputs of
// one weight row (one q4_1 block): lane group g = lane / 32 holds, for MFMA
// step s (0, 1), the 8 inputs [16 s + 8 g, 16 s + 8 g + 8).  The token operand
// is staged with the same input order, so the reduction is unchanged.
// ---------------------------------------------------------------------------
template <int FMT> struct WRaw;
template <> struct WRaw<FMT_Q4_1> { uint2 c; uint32_t dm; };
template <> struct WRaw<FMT_NVFP4> { uint32_t c0, c1; uint32_t s; };
template <> struct WRaw<FMT_BF16> { uint4 v0, v1; };

// Raw buffer resource over [base, base + bytes): loads past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 4 nibbles (bytes of t, each < 16) -> two fp16 pairs holding the integers,
// one packed fp8 -> fp16 conversion per pair: a byte q < 16 read as OCP E4M3
// is q * 2^-9 (exponent field 0 or 1), and the power-of-two scale 2^9 makes
// it q exactly (one instruction per two weights, where placing each byte
// under an fp16 exponent took a byte permute and a packed subtract).
__device__ __forceinline__ void nib4_to_h(uint32_t t, half2_t &a, half2_t &b) {
    a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(t, 512.0f, false);  // bytes t0, t1
    b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(t, 512.0f, true);   // bytes t2, t3
}

// fragments for steps 0 and 1; NVFP4 values exclude the tensor scale
// (applied to the accumulator), and are exact in fp16.
template <int FMT>
__device__ __forceinline__ void dequant_frag(const WRaw<FMT> &w, half8_t &s0, half8_t &s1) {
    if constexpr (FMT == FMT_Q4_1) {
        // {d, d} and {m, m}: the packed FMA takes them as halves of one
        // register (operand selects), with no broadcast instructions
        const half2_t dm = __builtin_bit_cast(half2_t, w.dm);
        const half2_t d2 = __builtin_shufflevector(dm, dm, 0, 0);
        const half2_t m2 = __builtin_shufflevector(dm, dm, 1, 1);
        const uint32_t wl[2] = {w.c.x, w.c.y};
#pragma unroll
        for (int i = 0; i < 2; i++) {
            half2_t a, b;
            nib4_to_h(wl[i] & 0x0F0F0F0Fu, a, b);
            a = a * d2 + m2;
            b = b * d2 + m2;
            s0[4 * i + 0] = a[0]; s0[4 * i + 1] = a[1]; s0[4 * i + 2] = b[0]; s0[4 * i + 3] = b[1];
            nib4_to_h((wl[i] >> 4) & 0x0F0F0F0Fu, a, b);
            a = a * d2 + m2;
            b = b * d2 + m2;
            s1[4 * i + 0] = a[0]; s1[4 * i + 1] = a[1]; s1[4 * i + 2] = b[0]; s1[4 * i + 3] = b[1];
        }
    } else if constexpr (FMT == FMT_NVFP4) {
        // E2M1 pairs (one code byte each, low nibble first) by the hardware
        // converter at scale 1 (exact), times the block's E4M3 scale: the
        // product has at most 6 significant bits and lies in fp16's normal
        // range, so it is exact too
        const _Float16 sc0 = (_Float16)e4m3_to_float(w.s & 0xFFu);
        const _Float16 sc1 = (_Float16)e4m3_to_float(w.s >> 8);
        const half2_t k0 = {sc0, sc0}, k1 = {sc1, sc1};
        // (the byte selector must be a literal)
        const half2_t a[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.c0, 1.0f, 0) * k0,
                              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.c0, 1.0f, 1) * k0,
                              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.c0, 1.0f, 2) * k0,
                              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.c0, 1.0f, 3) * k0};
        const half2_t b[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.c1, 1.0f, 0) * k1,
                              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.c1, 1.0f, 1) * k1,
                              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.c1, 1.0f, 2) * k1,
                              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.c1, 1.0f, 3) * k1};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            s0[2 * k] = a[k][0]; s0[2 * k + 1] = a[k][1];
            s1[2 * k] = b[k][0]; s1[2 * k + 1] = b[k][1];
        }
    } else {
        const uint32_t a[4] = {w.v0.x, w.v0.y, w.v0.z, w.v0.w};
        const uint32_t b[4] = {w.v1.x, w.v1.y, w.v1.z, w.v1.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            s0[2 * j] = (_Float16)bf16lo(a[j]);
            s0[2 * j + 1] = (_Float16)bf16hi(a[j]);
            s1[2 * j] = (_Float16)bf16lo(b[j]);
            s1[2 * j + 1] = (_Float16)bf16hi(b[j]);
        }
    }
}

// Block -> (tile, weight-row block) with an XCD-aware order.  Blocks go
// round-robin to the 8 XCDs (block b to XCD b % 8).  XCD x takes a
// contiguous eighth of the full tiles, then a contiguous eighth of the partial
// tiles (the table lists the full tiles first, in expert order), the MT
// blocks of a tile back to back: an expert's full tiles then run on one or
// two XCDs, which fetch its weights into their L2 once, the MT blocks of a
// tile share its token rows in that L2, and every XCD gets as many full and
// as many partial tiles as the others (to one), the partial ones filling its
// tail.  Returns ti * MT + mt, or -1 past the XCD's last tile.
__device__ __forceinline__ int xcd_tile_block(int b, int MT, int n_tiles, int n_full) {
    const int x = b & 7, k = (b >> 3) / MT, mt = (b >> 3) % MT;
    const int f0 = x * n_full / 8, nf = (x + 1) * n_full / 8 - f0;
    if (k < nf) return (f0 + k) * MT + mt;
    const int n_part = n_tiles - n_full;
    const int p0 = x * n_part / 8, np = (x + 1) * n_part / 8 - p0;
    return k - nf < np ? (n_full + p0 + k - nf) * MT + mt : -1;
}

// LDS bytes between consecutive lanes of a 2-byte buffer-to-LDS copy: each
// lane's value lands zero-extended in a dword of its own (measured on gfx950)
constexpr int NV_DMA16_STRIDE = 4;

// Weight stage of pf_gemm: the raw fragments of the block's 256 weight rows
// for one 32-input step, copied to LDS as they are stored in HBM
//   q4_1:  codes [256][16 B], then {d, m} [256][4 B]
//   NVFP4: codes [256][16 B], then E4M3 pairs [256][2 B]
//   bf16:  values [256][64 B]
template <int FMT> struct WStage;
template <> struct WStage<FMT_Q4_1> { static constexpr int BYTES = 256 * 20, SCALE_OFF = 4096, DMA = 2; };
// (the NVFP4 scale region is sized for 4 bytes per row so that the 2-byte
// DMA stays inside it whichever lane stride the hardware uses)
template <> struct WStage<FMT_NVFP4> {
    static constexpr int BYTES = 256 * 20, SCALE_OFF = 4096, DMA = 2, SCALE_STRIDE = NV_DMA16_STRIDE;
};
template <> struct WStage<FMT_BF16> { static constexpr int BYTES = 256 * 64, DMA = 4; };

// DMA copies issued per thread per K-step (2 token chunks + the weight stage);
// the wait for a stage three steps back relies on this count
template <int FMT> constexpr int pf_loads_per_step() { return 2 + WStage<FMT>::DMA; }

// s_waitcnt with vmcnt(n) only (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

constexpr int PF_NS = 4;       // LDS stages in flight
constexpr int PF_UNROLL = 16;  // K-steps per loop trip (multiple of PF_NS)

// Workgroup barrier without the memory fence of __syncthreads (whose release
// half waits for every outstanding load, which would drain the prefetch
// pipeline).  Callers order the LDS traffic themselves: an explicit vmcnt
// wait for the DMA writes, and every LDS read of a stage is consumed before
// the barrier that lets it be overwritten.  The signal fences keep the
// compiler from moving memory operations across it.
__device__ __forceinline__ void pf_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// slot of (row, 16-byte chunk) in a stage of 64-byte rows: chunks XOR-
// swizzled by (row >> 2) & 3, so that a 16-lane group of 16-byte fragment
// reads (rows r .. r + 15, one chunk) covers all 64 banks (measured on
// gfx950: as fast as a contiguous read; swizzling by (row >> 1) & 3 costs 1.8x)
__device__ __forceinline__ int pf_swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int pf_slot(int r, int c) { return r * 4 + (c ^ pf_swz(r)); }

typedef __attribute__((address_space(3))) void lds_void;

// fragment of weight row `row` of a weight stage (lane group g)
template <int FMT>
__device__ __forceinline__ WRaw<FMT> wraw_from_lds(const uint8_t *ws, int row, int g) {
    WRaw<FMT> w;
    if constexpr (FMT == FMT_Q4_1) {
        w.c = *reinterpret_cast<const uint2 *>(ws + row * 16 + 8 * g);
        w.dm = *reinterpret_cast<const uint32_t *>(ws + WStage<FMT>::SCALE_OFF + row * 4);
    } else if constexpr (FMT == FMT_NVFP4) {
        w.c0 = *reinterpret_cast<const uint32_t *>(ws + row * 16 + 4 * g);
        w.c1 = *reinterpret_cast<const uint32_t *>(ws + row * 16 + 8 + 4 * g);
        w.s = *reinterpret_cast<const uint16_t *>(ws + WStage<FMT>::SCALE_OFF + row * WStage<FMT>::SCALE_STRIDE);
    } else {
        w.v0 = *reinterpret_cast<const uint4 *>(ws + row * 64 + 16 * g);
        w.v1 = *reinterpret_cast<const uint4 *>(ws + row * 64 + 32 + 16 * g);
    }
    return w;
}

// DMA sources of one thread in pf_gemm: token buffer and weight matrices
// (buffer resources) with this thread's byte offsets at step 0
template <int FMT> struct PfDma {
    __amdgpu_buffer_rsrc_t rx;
    uint32_t xo[2];
    __amdgpu_buffer_rsrc_t rw[WStage<FMT>::DMA];
    uint32_t wo[WStage<FMT>::DMA];
    int wave;
};

// copy step ks of the token tile and of the weight fragments into one stage
template <int FMT>
__device__ __forceinline__ void pf_issue(const PfDma<FMT> &d, uint4 *xs, uint8_t *wsb, int ks) {
#pragma unroll
    for (int i = 0; i < 2; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rx, (lds_void *)(xs + i * 256 + 64 * d.wave), 16, d.xo[i], 64 * ks,
                                                 0, 0);
    if constexpr (FMT == FMT_BF16) {
#pragma unroll
        for (int i = 0; i < 4; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rw[i], (lds_void *)(wsb + 16 * (i * 256 + 64 * d.wave)), 16,
                                                     d.wo[i], 64 * ks, 0, 0);
    } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rw[0], (lds_void *)(wsb + 16 * 64 * d.wave), 16, d.wo[0], 16 * ks,
                                                 0, 0);
        if constexpr (FMT == FMT_Q4_1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rw[1], (lds_void *)(wsb + WStage<FMT>::SCALE_OFF + 4 * 64 * d.wave),
                                                     4, d.wo[1], 4 * ks, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                d.rw[1], (lds_void *)(wsb + WStage<FMT>::SCALE_OFF + WStage<FMT>::SCALE_STRIDE * 64 * d.wave), 2,
                d.wo[1], 2 * ks, 0, 0);
    }
}
// DMA of one 32-input step of pf_router_gemm: this thread's token chunk and
// its 4 router chunks (offsets of step 0; the step goes in the scalar offset)
struct RgDma {
    __amdgpu_buffer_rsrc_t rx, rr;
    uint32_t xo, ro[4];
    int wave;
};

__device__ __forceinline__ void rg_issue(const RgDma &d, uint4 *xs, uint4 *rs, int k) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rx, (lds_void *)(xs + 64 * d.wave), 16, d.xo, 64 * k, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rr, (lds_void *)(rs + i * 256 + 64 * d.wave), 16, d.ro[i], 64 * k,
                                                 0, 0);
}
// Epilogue of the grouped GEMMs.  acc[a][b][j] = out[row m][token n] of
// the wave's row group a, m = 8 (j/4) + 4 g + j%4, n = 32 b + l32.
//   MODE 0: h = silu(gate) * up (gate in a = 0, up in a = 1), fp16 rows of H
//   MODE 1: O = coef * acc, fp16 rows of O
// silu(g) * u for the fp16 h of the grouped GEMM: the reciprocal instruction
// (within 1 ulp) in place of an IEEE division, whose correction steps cost
// several times more; the result is rounded to fp16 (2^-11) right after.
__device__ __forceinline__ float silu_mul_h(float g, float u) {
    return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

template <int MODE, int NBLK>
__device__ __forceinline__ void pf_epilogue(const PfParams &p, const PfTile &tile, const f32x16_t (&acc)[2][NBLK], int r0,
                                            const bool (&sub_ok)[2], int g, int l32) {
    if (MODE == 0) {
        if (!sub_ok[0]) return;
        const float ts_g = p.tscale ? p.tscale[3 * tile.e + 0] : 1.f;
        const float ts_u = p.tscale ? p.tscale[3 * tile.e + 1] : 1.f;
#pragma unroll
        for (int b = 0; b < NBLK; b++) {
            const int n = 32 * b + l32;
            if (n >= tile.rows) continue;
            _Float16 *hrow = p.h + (size_t)(tile.row0 + n) * p.F + r0 + 4 * g;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                uint32_t pk[2];
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    const float g0 = acc[0][b][4 * q + 2 * i] * ts_g, u0 = acc[1][b][4 * q + 2 * i] * ts_u;
                    const float g1 = acc[0][b][4 * q + 2 * i + 1] * ts_g, u1 = acc[1][b][4 * q + 2 * i + 1] * ts_u;
                    const _Float16 h0 = (_Float16)silu_mul_h(g0, u0), h1 = (_Float16)silu_mul_h(g1, u1);
                    pk[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                }
                *reinterpret_cast<uint2 *>(hrow + 8 * q) = make_uint2(pk[0], pk[1]);
            }
        }
    } else {
        const float ts_d = p.tscale ? p.tscale[3 * tile.e + 2] : 1.f;
#pragma unroll
        for (int b = 0; b < NBLK; b++) {
            const int n = 32 * b + l32;
            if (n >= tile.rows) continue;
            const float c = p.perm_w[tile.row0 + n] * ts_d;
            _Float16 *orow = p.o + (size_t)(tile.row0 + n) * p.D;
#pragma unroll
            for (int a = 0; a < 2; a++) {
                if (!sub_ok[a]) continue;
                const int dr = r0 + 32 * a + 4 * g;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const half2_t v01 = {(_Float16)(acc[a][b][4 * q + 0] * c), (_Float16)(acc[a][b][4 * q + 1] * c)};
                    const half2_t v23 = {(_Float16)(acc[a][b][4 * q + 2] * c), (_Float16)(acc[a][b][4 * q + 3] * c)};
                    *reinterpret_cast<uint2 *>(orow + dr + 8 * q) =
                        make_uint2(__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23));
                }
            }
        }
    }
}

// pf_epilogue through LDS, for tiles of up to 128 rows: each wave writes its
// results (the same fp32 arithmetic and fp16 rounding as pf_epilogue) to an
// 8 KB LDS region of its own, token-major, and reads them back so that every
// global store of a lane covers 16 contiguous bytes of one token's row and a
// wave's store covers whole 64- or 128-byte row segments.  Stored directly
// from the accumulator layout, one store instruction touches 32 rows of 16
// bytes each, and the address unit's cost of those stores dominated the end
// of every block.  The caller has waited for its copies into the region and
// passed a workgroup barrier after the main loop's last reads of it.
//   MODE 0: region [128 tokens][64 B]: the wave's 32 features of h; 16-byte
//           chunk c of row t at slot c ^ ((t >> 2) & 3)
//   MODE 1: region [64 tokens][128 B]: the wave's 64 output rows of O for
//           token blocks 2 hb, 2 hb + 1 (two halves); chunk c of row t at
//           slot c ^ (t & 7)
template <int MODE>
__device__ __forceinline__ void pf_epilogue_lds(const PfParams &p, const PfTile &tile, const f32x16_t (&acc)[2][4],
                                                int r0, const bool (&sub_ok)[2], int g, int l32, int lane,
                                                uint4 *region) {
    uint8_t *rb = reinterpret_cast<uint8_t *>(region);
    if (MODE == 0) {
        if (!sub_ok[0]) return;
        const float ts_g = p.tscale ? p.tscale[3 * tile.e + 0] : 1.f;
        const float ts_u = p.tscale ? p.tscale[3 * tile.e + 1] : 1.f;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int t = 32 * b + l32;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                uint32_t pk[2];
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    const float g0 = acc[0][b][4 * q + 2 * i] * ts_g, u0 = acc[1][b][4 * q + 2 * i] * ts_u;
                    const float g1 = acc[0][b][4 * q + 2 * i + 1] * ts_g, u1 = acc[1][b][4 * q + 2 * i + 1] * ts_u;
                    const _Float16 h0 = (_Float16)silu_mul_h(g0, u0), h1 = (_Float16)silu_mul_h(g1, u1);
                    pk[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                }
                if (t < tile.rows)
                    *reinterpret_cast<uint2 *>(rb + t * 64 + 16 * (q ^ ((t >> 2) & 3)) + 8 * g) = make_uint2(pk[0], pk[1]);
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int t = 16 * i + (lane >> 2), c = lane & 3;
            if (t < tile.rows) {
                const uint4 v = *reinterpret_cast<const uint4 *>(rb + t * 64 + 16 * (c ^ ((t >> 2) & 3)));
                *reinterpret_cast<uint4 *>(p.h + (size_t)(tile.row0 + t) * p.F + r0 + 8 * c) = v;
            }
        }
    } else {
        const float ts_d = p.tscale ? p.tscale[3 * tile.e + 2] : 1.f;
        const int ROWS_A = p.D;
#pragma unroll
        for (int hb = 0; hb < 2; hb++) {
#pragma unroll
            for (int bb = 0; bb < 2; bb++) {
                const int b = 2 * hb + bb, n = 32 * b + l32, t = 32 * bb + l32;
                if (n >= tile.rows) continue;
                const float c = p.perm_w[tile.row0 + n] * ts_d;
#pragma unroll
                for (int a = 0; a < 2; a++)
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const half2_t v01 = {(_Float16)(acc[a][b][4 * q + 0] * c), (_Float16)(acc[a][b][4 * q + 1] * c)};
                        const half2_t v23 = {(_Float16)(acc[a][b][4 * q + 2] * c), (_Float16)(acc[a][b][4 * q + 3] * c)};
                        *reinterpret_cast<uint2 *>(rb + t * 128 + 16 * ((4 * a + q) ^ (t & 7)) + 8 * g) =
                            make_uint2(__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23));
                    }
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int t = 8 * i + (lane >> 3), c = lane & 7, n = 64 * hb + t;
                if (n < tile.rows && r0 + 8 * c < ROWS_A) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(rb + t * 128 + 16 * (c ^ (t & 7)));
                    *reinterpret_cast<uint4 *>(p.o + (size_t)(tile.row0 + n) * p.D + r0 + 8 * c) = v;
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

#endif  // __HIP_DEVICE_COMPILE__ (helpers of pf_gemm)

// ---------------------------------------------------------------------------
// pf_gemm<MODE>: one block = one tile of <= 128 rows of one expert x 128
// (gate/up: features; MODE 0) or 256 (down: outputs; MODE 1) weight rows.
// Wave w owns 2 A-operand row groups of 32 (gate and up of the same 32
// features, or 2 x 32 down rows) against all 128 tile rows (4 x 32).
// Pipeline: the token tile and the block's raw weight fragments of step k
// are copied to LDS stage k % 4 by buffer-to-LDS DMA three steps ahead; the
// weights are dequantised from LDS into MFMA operands.
// ---------------------------------------------------------------------------
template <int FMT, int MODE>
__global__ void __launch_bounds__(PF_THREADS, 2) pf_gemm(PfParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    // one LDS object per stage: stage indices are compile-time after
    // unrolling, so alias analysis separates a stage's DMA writes from the
    // reads of the others (no conservative vmcnt waits before ds_read)
    __shared__ uint4 x0s[PF_BM * 4], x1s[PF_BM * 4], x2s[PF_BM * 4], x3s[PF_BM * 4];
    __shared__ __attribute__((aligned(16))) uint8_t w0s[WStage<FMT>::BYTES], w1s[WStage<FMT>::BYTES],
        w2s[WStage<FMT>::BYTES], w3s[WStage<FMT>::BYTES];
#define PF_XST(st) ((st) == 0 ? x0s : (st) == 1 ? x1s : (st) == 2 ? x2s : x3s)
#define PF_WST(st) ((st) == 0 ? w0s : (st) == 1 ? w1s : (st) == 2 ? w2s : w3s)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int MT = MODE == 0 ? (p.F + 127) / 128 : (p.D + 255) / 256;
    const int L = xcd_tile_block(blockIdx.x, MT, p.meta[0], p.meta[2]);
    if (L < 0) return;
    const int ti = L / MT, mt = L % MT;
    const PfTile tile = p.tiles[ti];
    const int K = MODE == 0 ? p.D : p.F;           // reduction length
    const int ROWS_A = MODE == 0 ? p.F : p.D;      // rows of the weight matrix
    const uint8_t *eb = p.experts + (size_t)tile.e * p.expert_bytes;
    const size_t mb_gu = mat_bytes<FMT>(p.F, p.D);
    const uint32_t mbytes = (uint32_t)mat_bytes<FMT>(ROWS_A, K);
    const int r0 = MODE == 0 ? mt * 128 + 32 * wave : mt * 256 + 64 * wave;  // first A row of sub 0
    const int r1 = MODE == 0 ? r0 : r0 + 32;
    const bool sub_ok[2] = {r0 < ROWS_A, r1 < ROWS_A};
    // this wave's two row groups inside a weight stage
    const int lrow0 = MODE == 0 ? 32 * wave + l32 : 64 * wave + l32;
    const int lrow1 = MODE == 0 ? 128 + 32 * wave + l32 : 64 * wave + 32 + l32;

    // token DMA: this thread fills slots (i * 256 + 64 * wave + lane) of a
    // stage, i = 0, 1, i.e. rows 64 i + 16 wave + lane / 4, one chunk each;
    // byte offsets inside the token buffer, the step goes in the scalar offset
    const __amdgpu_buffer_rsrc_t rx =
        MODE == 0 ? buf_rsrc(p.x16, (uint32_t)((size_t)p.T * p.D * 2))
                  : buf_rsrc(p.h + (size_t)tile.row0 * p.F, (uint32_t)tile.rows * p.F * 2);
    uint32_t xo[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int r = 64 * i + 16 * wave + (lane >> 2);
        const int c = (lane & 3) ^ pf_swz(r);
        const int rr = min(r, tile.rows - 1);
        const uint32_t row = MODE == 0 ? (uint32_t)p.perm_tok[tile.row0 + rr] * p.D : (uint32_t)rr * p.F;
        xo[i] = 2 * row + 16 * c;
    }
    // weight DMA: stage row q of the block -> weight row, matrix
    //   MODE 0: q < 128 gate row mt*128 + q, else up row mt*128 + q - 128
    //   MODE 1: down row mt*256 + q
    PfDma<FMT> dma;
    dma.rx = rx;
    dma.xo[0] = xo[0];
    dma.xo[1] = xo[1];
    dma.wave = wave;
    if constexpr (FMT == FMT_BF16) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int j = i * 256 + 64 * wave + lane;  // 16-byte chunk of the stage
            const int q = j >> 2;                       // row of the stage (uniform matrix per wave)
            const int qw = 64 * i + 16 * wave;          // first row of the wave's chunks
            const int rowA = min(MODE == 0 ? mt * 128 + (q & 127) : mt * 256 + q, ROWS_A - 1);
            const uint8_t *mat = MODE == 0 ? (qw < 128 ? eb : eb + mb_gu) : eb + 2 * mb_gu;
            dma.rw[i] = buf_rsrc(mat, mbytes);
            dma.wo[i] = (uint32_t)rowA * K * 2 + 16 * (j & 3);
        }
    } else {
        const int q = 64 * wave + lane;
        const int rowA = min(MODE == 0 ? mt * 128 + (q & 127) : mt * 256 + q, ROWS_A - 1);
        const uint8_t *mat = MODE == 0 ? (64 * wave < 128 ? eb : eb + mb_gu) : eb + 2 * mb_gu;
        dma.rw[0] = dma.rw[1] = buf_rsrc(mat, mbytes);
        dma.wo[0] = (uint32_t)rowA * (K / 2);
        dma.wo[1] = (uint32_t)ROWS_A * (K / 2) + (uint32_t)rowA * (FMT == FMT_Q4_1 ? (K / 32) * 4 : K / 16);
    }
    const int NK = K / 32;

    f32x16_t acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int j = 0; j < 16; j++) acc[a][b][j] = 0.f;

#pragma unroll
    for (int s = 0; s < PF_NS - 1; s++) pf_issue<FMT>(dma, PF_XST(s), PF_WST(s), min(s, NK - 1));

    // 16 steps per loop trip: the wait-count analysis is exact inside the
    // unrolled body but drains every load at a loop header
    for (int kb0 = 0; kb0 < NK; kb0 += PF_UNROLL) {
#pragma unroll
        for (int u = 0; u < PF_UNROLL; u++) {
            const int kb = kb0 + u;
            if (kb >= NK) break;
            // stage kb (issued 3 steps back) has landed for this wave; after
            // the barrier, for every wave, and stage kb - 1 is free
            wait_vmcnt<2 * pf_loads_per_step<FMT>()>();
            pf_barrier();
            // past the end: reload the last step (never read)
            pf_issue<FMT>(dma, PF_XST((u + PF_NS - 1) % PF_NS), PF_WST((u + PF_NS - 1) % PF_NS),
                          min(kb + PF_NS - 1, NK - 1));
            const uint8_t *wsb = PF_WST(u % PF_NS);
            half8_t af[2][2];
            dequant_frag<FMT>(wraw_from_lds<FMT>(wsb, lrow0, g), af[0][0], af[0][1]);
            dequant_frag<FMT>(wraw_from_lds<FMT>(wsb, lrow1, g), af[1][0], af[1][1]);
            const _Float16 *stg = reinterpret_cast<const _Float16 *>(PF_XST(u % PF_NS));
#pragma unroll
            for (int s = 0; s < 2; s++) {
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    const half8_t bf = *reinterpret_cast<const half8_t *>(stg + 8 * pf_slot(32 * b + l32, 2 * s + g));
                    acc[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[0][s], bf, acc[0][b], 0, 0, 0);
                    acc[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[1][s], bf, acc[1][b], 0, 0, 0);
                }
            }
        }
    }

    pf_epilogue<MODE, 4>(p, tile, acc, r0, sub_ok, g, l32);

#endif  // __HIP_DEVICE_COMPILE__
}
#undef PF_XST
#undef PF_WST

#if defined(__HIP_DEVICE_COMPILE__)
// MFMAs of one 32-input step against the first NB 32-row token blocks of a
// token stage (the tile's other blocks hold only padding rows)
template <int NB, int NBLK>
__device__ __forceinline__ void pf_mfma_tokens(const _Float16 *stg, const half8_t (&af)[2][2], f32x16_t (&acc)[2][NBLK],
                                               int l32, int g) {
#pragma unroll
    for (int s = 0; s < 2; s++) {
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const half8_t bf = *reinterpret_cast<const half8_t *>(stg + 8 * pf_slot(32 * b + l32, 2 * s + g));
            acc[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[0][s], bf, acc[0][b], 0, 0, 0);
            acc[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[1][s], bf, acc[1][b], 0, 0, 0);
        }
    }
}
#endif

// ---------------------------------------------------------------------------
// pq_gemm_body<FMT, MODE, BM, FUSED>: pf_gemm for the 4-bit formats (q4_1,
// NVFP4), run by pf_ffn_q4, on tiles of up to BM token rows (128: two blocks per CU; 256: one block per CU
// with the accumulators of 8 token blocks, so each dequantised weight feeds
// twice the MFMAs), with the weight fragments of 4 consecutive 32-input steps
// copied at once (per row 64 B of codes, and the 16 B of 4 q4_1 {d, m} pairs
// or the 8 B of 4 NVFP4 pairs of E4M3 block scales).  The address unit's cost of a wave-wide copy
// grows with the cache lines it touches: 16 rows x 64 B costs well under
// half of 64 rows x 16 B (measured on gfx950), and it dominated the
// one-step weight copies.  Weight macro-stages are double-buffered and
// copied one macro (4 steps) ahead; the token tile keeps pf_gemm's 4-stage
// per-step ring, and the weights are dequantised from LDS the same way.
// ---------------------------------------------------------------------------
constexpr int PQ_MS = 4;                                        // steps per weight macro-stage
constexpr int PQ_SOFF = 256 * 16 * PQ_MS;                       // scales inside a macro buffer
constexpr int PQ_WBYTES = PQ_SOFF + 256 * 4 * PQ_MS;
constexpr int PQ_UNROLL = 16;                                   // steps per loop trip

// chunk swizzle of a row in the code macro-stage (64-byte rows)
__device__ __forceinline__ int pq_swz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

#if defined(__HIP_DEVICE_COMPILE__)
// raw fragment of weight row `row`, step st of a macro buffer: the step's
// 16 code bytes sit at chunk st ^ pq_swz(row) of the row; sc = the row's
// scale word of that step (q4_1 {d, m}; NVFP4 the two E4M3 block scales)
template <int FMT>
__device__ __forceinline__ WRaw<FMT> pq_frag(const uint8_t *cb, int row, int st, int g, uint32_t sc) {
    const uint8_t *q = cb + row * 64 + 16 * (st ^ pq_swz(row));
    WRaw<FMT> w;
    if constexpr (FMT == FMT_Q4_1) {
        w.c = *reinterpret_cast<const uint2 *>(q + 8 * g);
        w.dm = sc;
    } else {
        w.c0 = *reinterpret_cast<const uint32_t *>(q + 4 * g);
        w.c1 = *reinterpret_cast<const uint32_t *>(q + 8 + 4 * g);
        w.s = sc;
    }
    return w;
}
#endif

#if defined(__HIP_DEVICE_COMPILE__)
// Handover of h from the gate/up blocks of a tile to its down blocks inside
// pf_ffn_q4.  Both run on the same XCD (see pf_ffn_q4), so h travels through
// that XCD's L2, which needs no cache maintenance: a gate/up block waits until
// its h stores have reached L2, then adds 1 + (its XCC id << 10) to the tile's
// counter with an L2 atomic.  A down block's thread 0 polls the counter with
// L1-bypassing loads for at most PF_SPIN_TICKS of the 100 MHz real-time
// counter, then checks that every producer ran on its own XCC (the id field
// must be target x its id).  A wait that gives up, or producers on another
// XCC (whose L2 this block cannot see), return nonzero in every thread: the
// block then writes NaN, so a broken handover shows as NaN outputs, never as
// stale values or a hang.
constexpr uint64_t PF_SPIN_TICKS = 2000000;  // 20 ms
constexpr int PF_DONE_COUNT_BITS = 10;
__device__ __forceinline__ int pf_xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15; }  // HW_REG_XCC_ID[3:0]
__device__ __forceinline__ int pf_wait_tile(const int32_t *done, int target) {
    int bad = 0;
    if (threadIdx.x == 0) {
        const int want_ids = target * pf_xcc_id();
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        int v;
        while (((v = __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) &
                ((1 << PF_DONE_COUNT_BITS) - 1)) < target) {
            if (__builtin_amdgcn_s_memrealtime() - t0 > PF_SPIN_TICKS) {
                bad = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if ((v >> PF_DONE_COUNT_BITS) != want_ids) bad = 1;
    }
    return __syncthreads_or(bad);
}
#endif

// Body of the 4-bit grouped GEMM for block `bid` of its role (MODE 0: gate/up,
// MODE 1: down), over LDS stages that the kernel declares.  FUSED: the block
// runs inside pf_ffn_q4, where a gate/up block counts its tile once its h
// rows are stored and a down block waits for that count before it copies h
// (its weight copies go out before the wait).
template <int FMT, int MODE, int BM, bool FUSED>
__device__ __forceinline__ void pq_gemm_body(const PfParams &p, int bid, uint4 *x0s, uint4 *x1s, uint4 *x2s,
                                             uint4 *x3s, uint8_t *c0s, uint8_t *c1s) {
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(FMT == FMT_Q4_1 || FMT == FMT_NVFP4, "4-bit formats");
    constexpr int NBLK = BM / 32;  // 32-row token blocks of a tile
    constexpr int XCH = BM / 64;   // token copies per thread per step
    // copies per thread of a weight macro's first part (W1: scales + 2 code
    // copies) and second part (W2: 2 code copies)
    constexpr int W1N = FMT == FMT_Q4_1 ? 3 : 4, W2N = 2;
#define PQ_XST(st) ((st) == 0 ? x0s : (st) == 1 ? x1s : (st) == 2 ? x2s : x3s)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int MT = MODE == 0 ? (p.F + 127) / 128 : (p.D + 255) / 256;
    const int L = xcd_tile_block(bid, MT, p.meta[0], p.meta[2]);
    if (L < 0) return;
    const int ti = L / MT, mt = L % MT;
    const PfTile tile = p.tiles[ti];
    const int K = MODE == 0 ? p.D : p.F;
    const int ROWS_A = MODE == 0 ? p.F : p.D;
    const uint8_t *eb = p.experts + (size_t)tile.e * p.expert_bytes;
    const uint32_t mb = (uint32_t)mat_bytes<FMT>(ROWS_A, K);  // bytes of one weight matrix
    // 32-row token blocks holding rows of the tile (the rest is padding)
    const int nb = __builtin_amdgcn_readfirstlane((tile.rows + 31) >> 5);
    const int r0 = MODE == 0 ? mt * 128 + 32 * wave : mt * 256 + 64 * wave;
    const int r1 = MODE == 0 ? r0 : r0 + 32;
    const bool sub_ok[2] = {r0 < ROWS_A, r1 < ROWS_A};
    const int lrow0 = MODE == 0 ? 32 * wave + l32 : 64 * wave + l32;
    const int lrow1 = MODE == 0 ? 128 + 32 * wave + l32 : 64 * wave + 32 + l32;

    // token DMA: this thread fills slots i * 256 + tid of a stage, i.e. rows
    // 64 i + 16 wave + lane / 4, one chunk each (the step goes in the scalar offset)
    const __amdgpu_buffer_rsrc_t rx = MODE == 0 ? buf_rsrc(p.x16, (uint32_t)((size_t)p.T * p.D * 2))
                                                : buf_rsrc(p.h + (size_t)tile.row0 * p.F, (uint32_t)tile.rows * p.F * 2);
    uint32_t xo[XCH];
#pragma unroll
    for (int i = 0; i < XCH; i++) {
        const int r = 64 * i + 16 * wave + (lane >> 2);
        const int c = (lane & 3) ^ pf_swz(r);
        const int rr = min(r, tile.rows - 1);
        const uint32_t row = MODE == 0 ? (uint32_t)p.perm_tok[tile.row0 + rr] * p.D : (uint32_t)rr * p.F;
        xo[i] = 2 * row + 16 * c;
    }
    // weight DMA over the block's matrices (gate then up, or down).  Stage
    // row q: MODE 0 gate row mt*128 + q (q < 128) or up row mt*128 + q - 128,
    // MODE 1 down row mt*256 + q.  Code slots i * 256 + tid hold row
    // q = 64 i + tid / 4, step (tid & 3) ^ pq_swz(q) (= pq_swz(tid / 4)).
    // q4_1 scale slot tid (16 B) holds row tid; NVFP4 scale dword slots
    // i * 256 + tid hold dword tid & 1 of row 128 i + tid / 2 (4-byte copies:
    // a row's 8 bytes of a macro are only 8-byte aligned in the matrix).
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc(MODE == 0 ? eb : eb + 2 * (size_t)mb, MODE == 0 ? 2 * mb : mb);
    auto wrow = [&](int q, uint32_t &mat) {
        mat = (MODE == 0 && q >= 128) ? mb : 0u;
        return (uint32_t)min(MODE == 0 ? mt * 128 + (q & 127) : mt * 256 + q, ROWS_A - 1);
    };
    uint32_t co[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t mat;
        const uint32_t ra = wrow(64 * i + (tid >> 2), mat);
        co[i] = mat + ra * (uint32_t)(K / 2) + 16 * ((tid & 3) ^ pq_swz(tid >> 2));
    }
    uint32_t so[FMT == FMT_Q4_1 ? 1 : 2];
    if constexpr (FMT == FMT_Q4_1) {
        uint32_t mat;
        const uint32_t ra = wrow(tid, mat);
        so[0] = mat + (uint32_t)ROWS_A * (K / 2) + ra * (uint32_t)(K / 32) * 4;
    } else {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            uint32_t mat;
            const uint32_t ra = wrow(128 * i + (tid >> 1), mat);
            so[i] = mat + (uint32_t)ROWS_A * (K / 2) + ra * (uint32_t)(K / 16) + 4 * (tid & 1);
        }
    }
    const int NK = K / 32, NM = (NK + PQ_MS - 1) / PQ_MS;
    uint32_t sc0[PQ_MS], sc1[PQ_MS];  // scale words of the current macro, rows lrow0 and lrow1

    f32x16_t acc[2][NBLK];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < NBLK; b++)
#pragma unroll
            for (int j = 0; j < 16; j++) acc[a][b][j] = 0.f;

    // weight macro m into buffer b, in two parts: W1 = the scale copy and
    // code copies 0, 1 (issued at the macro's first step), W2 = code copies
    // 2, 3 (at its second step), so no step queues all five
#define PQ_ISSUE_W1(b, m)                                                                                          \
    do {                                                                                                           \
        uint8_t *cb_ = (b) == 0 ? c0s : c1s;                                                                       \
        uint8_t *sb_ = ((b) == 0 ? c0s : c1s) + PQ_SOFF;                                                           \
        if constexpr (FMT == FMT_Q4_1) {                                                                           \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(sb_ + 16 * 64 * wave), 16, so[0],            \
                                                     4 * PQ_MS * (m), 0, 0);                                       \
        } else {                                                                                                   \
            _Pragma("unroll") for (int i_ = 0; i_ < 2; i_++) __builtin_amdgcn_raw_ptr_buffer_load_lds(             \
                rw, (lds_void *)(sb_ + 4 * (i_ * 256 + 64 * wave)), 4, so[i_], 2 * PQ_MS * (m), 0, 0);             \
        }                                                                                                          \
        _Pragma("unroll") for (int i_ = 0; i_ < 2; i_++) __builtin_amdgcn_raw_ptr_buffer_load_lds(                 \
            rw, (lds_void *)(cb_ + 16 * (i_ * 256 + 64 * wave)), 16, co[i_], 16 * PQ_MS * (m), 0, 0);              \
    } while (0)
#define PQ_ISSUE_W2(b, m)                                                                                          \
    do {                                                                                                           \
        uint8_t *cb_ = (b) == 0 ? c0s : c1s;                                                                       \
        _Pragma("unroll") for (int i_ = 2; i_ < 4; i_++) __builtin_amdgcn_raw_ptr_buffer_load_lds(                 \
            rw, (lds_void *)(cb_ + 16 * (i_ * 256 + 64 * wave)), 16, co[i_], 16 * PQ_MS * (m), 0, 0);              \
    } while (0)
#define PQ_ISSUE_X(st, ks)                                                                                         \
    do {                                                                                                           \
        _Pragma("unroll") for (int i_ = 0; i_ < XCH; i_++) __builtin_amdgcn_raw_ptr_buffer_load_lds(               \
            rx, (lds_void *)(PQ_XST(st) + i_ * 256 + 64 * wave), 16, xo[i_], 64 * (ks), 0, 0);                     \
    } while (0)
#define PQ_READ_SC(b)                                                                                              \
    do {                                                                                                           \
        const uint8_t *sb_ = ((b) == 0 ? c0s : c1s) + PQ_SOFF;                                                     \
        if constexpr (FMT == FMT_Q4_1) {                                                                           \
            const uint4 v0_ = *reinterpret_cast<const uint4 *>(sb_ + lrow0 * 16);                                  \
            const uint4 v1_ = *reinterpret_cast<const uint4 *>(sb_ + lrow1 * 16);                                  \
            sc0[0] = v0_.x; sc0[1] = v0_.y; sc0[2] = v0_.z; sc0[3] = v0_.w;                                        \
            sc1[0] = v1_.x; sc1[1] = v1_.y; sc1[2] = v1_.z; sc1[3] = v1_.w;                                        \
        } else {                                                                                                   \
            const uint2 v0_ = *reinterpret_cast<const uint2 *>(sb_ + lrow0 * 8);                                   \
            const uint2 v1_ = *reinterpret_cast<const uint2 *>(sb_ + lrow1 * 8);                                   \
            sc0[0] = v0_.x & 0xFFFFu; sc0[1] = v0_.x >> 16; sc0[2] = v0_.y & 0xFFFFu; sc0[3] = v0_.y >> 16;        \
            sc1[0] = v1_.x & 0xFFFFu; sc1[1] = v1_.x >> 16; sc1[2] = v1_.y & 0xFFFFu; sc1[3] = v1_.y >> 16;        \
        }                                                                                                          \
    } while (0)

    PQ_ISSUE_W1(0, 0);
    PQ_ISSUE_W2(0, 0);
    int gave_up = 0;
    if constexpr (FUSED && MODE == 1) gave_up = pf_wait_tile(p.tile_done + ti, (p.F + 127) / 128);
#pragma unroll
    for (int s = 0; s < PF_NS - 1; s++) PQ_ISSUE_X(s, min(s, NK - 1));
    // macro 0 has landed once only the 3 token stages are pending
    wait_vmcnt<XCH * (PF_NS - 1)>();
    pf_barrier();
    PQ_READ_SC(0);
    // weights of step 0 in MFMA operand form; each step then dequantises the
    // next step's weights while its own MFMAs run
    half8_t af[2][2];
    dequant_frag<FMT>(pq_frag<FMT>(c0s, lrow0, 0, g, sc0[0]), af[0][0], af[0][1]);
    dequant_frag<FMT>(pq_frag<FMT>(c0s, lrow1, 0, g, sc1[0]), af[1][0], af[1][1]);

    static_assert(PQ_UNROLL % (2 * PQ_MS) == 0 && PQ_UNROLL % PF_NS == 0 && PQ_MS == 4, "stage indices per trip");
    // The main loop, instantiated for tiles of at most 32 rows (the partial
    // tiles of most experts), of at most 128 and of up to BM rows: the
    // token-block count fixes the MFMAs of a step.  Step kb waits until
    // token stage kb has landed (only the copies of the two later steps may
    // be pending: XCH token copies each, plus W1 (W1N) after a macro's first
    // step and W2 (W2N) after its second); at a macro's last step it also waits
    // for the next macro's W2, whose codes it dequantises for the next step.
    // The next macro's scales are read at that step too (its W1 copy came
    // before this step's token stage).
#define PQ_MAIN_LOOP(NB_)                                                                                              \
    for (int kb0 = 0; kb0 < NK; kb0 += PQ_UNROLL) {                                                                    \
_Pragma("unroll")                                                                                                      \
        for (int u = 0; u < PQ_UNROLL; u++) {                                                                          \
            const int kb = kb0 + u;                                                                                    \
            if (kb >= NK) break;                                                                                       \
            const int st = u % PQ_MS;                                                                                  \
            if (st == 0)                                                                                               \
                wait_vmcnt<2 * XCH>();                                                                                 \
            else if (st == 1)                                                                                          \
                wait_vmcnt<2 * XCH + W1N>();                                                                           \
            else if (st == 2)                                                                                          \
                wait_vmcnt<2 * XCH + W1N + W2N>();                                                                     \
            else                                                                                                       \
                wait_vmcnt<2 * XCH>();                                                                                 \
            pf_barrier();                                                                                              \
            if (st == 0) PQ_ISSUE_W1((u / PQ_MS + 1) % 2, min(kb / PQ_MS + 1, NM - 1));                                \
            if (st == 1) PQ_ISSUE_W2((u / PQ_MS + 1) % 2, min(kb / PQ_MS + 1, NM - 1));                                \
            PQ_ISSUE_X((u + PF_NS - 1) % PF_NS, min(kb + PF_NS - 1, NK - 1));                                          \
            const _Float16 *stg = reinterpret_cast<const _Float16 *>(PQ_XST(u % PF_NS));                               \
            pf_mfma_tokens<NB_, NBLK>(stg, af, acc, l32, g);                                                           \
            const int un = u + 1, stn = un % PQ_MS;                                                                    \
            if (stn == 0) PQ_READ_SC((un / PQ_MS) % 2);                                                                \
            const uint8_t *cb = (un / PQ_MS) % 2 == 0 ? c0s : c1s;                                                     \
            dequant_frag<FMT>(pq_frag<FMT>(cb, lrow0, stn, g, sc0[stn]), af[0][0], af[0][1]);                          \
            dequant_frag<FMT>(pq_frag<FMT>(cb, lrow1, stn, g, sc1[stn]), af[1][0], af[1][1]);                          \
        }                                                                                                              \
    }
    if (nb == 1) {
        PQ_MAIN_LOOP(1);
    } else if (BM == 128 || nb <= 4) {
        PQ_MAIN_LOOP(4);
    } else {
        PQ_MAIN_LOOP(NBLK);
    }
#undef PQ_MAIN_LOOP
#undef PQ_ISSUE_W1
#undef PQ_ISSUE_W2
#undef PQ_ISSUE_X
#undef PQ_READ_SC
    if (gave_up) {
#pragma unroll
        for (int a = 0; a < 2; a++)
#pragma unroll
            for (int b = 0; b < NBLK; b++)
#pragma unroll
                for (int j = 0; j < 16; j++) acc[a][b][j] = __builtin_nanf("");
    }
    if constexpr (BM == 128) {
        // the stages are free once every copy has landed and every wave is
        // past its last step; wave w then takes token stage w as its region
        wait_vmcnt<0>();
        __syncthreads();
        pf_epilogue_lds<MODE>(p, tile, acc, r0, sub_ok, g, l32, lane, PQ_XST(wave));
    } else {
        pf_epilogue<MODE, NBLK>(p, tile, acc, r0, sub_ok, g, l32);
    }
    if constexpr (FUSED && MODE == 0) {
        // every wave's h stores have reached this XCD's L2 before the barrier;
        // then one thread counts the tile's block with its XCC id
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            __hip_atomic_fetch_add(p.tile_done + ti, 1 + (pf_xcc_id() << PF_DONE_COUNT_BITS), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
#endif  // __HIP_DEVICE_COMPILE__
}
#undef PQ_XST

// pf_ffn_q4: both grouped GEMMs of a layer in one dispatch.  Blocks below
// p.g1 are the gate/up GEMM's blocks, the rest the down GEMM's, each in the
// block -> tile order of its own kernel; p.g1 is a multiple of 8, so the down
// blocks of a tile run on the XCD that ran its gate/up blocks and read h
// from that XCD's L2.  A down block waits only for the gate/up blocks of its
// own tile, so the down GEMM fills the slots that the gate/up GEMM's last
// blocks leave idle, without a kernel boundary between the two.  The wait
// cannot deadlock: each XCD dispatches its blocks in order, so every gate/up
// block is resident before any down block of its XCD, and gate/up blocks
// never wait.
template <int FMT>
__global__ void __launch_bounds__(PF_THREADS, 2) pf_ffn_q4(PfParams p) {
    // token stages: [128 rows][4 x 16 B]; weight macro buffers: codes [256
    // rows][4 steps x 16 B], a row's step chunks XOR-swizzled by pq_swz(row)
    // (the 8-byte fragment reads of 32 rows then spread over the banks with
    // the least conflict measured), then scales at PQ_SOFF: [256 rows][4
    // steps x {d, m}] (q4_1) or [256 rows][4 steps x 2 E4M3] (NVFP4).  One
    // LDS object per stage and per macro buffer, so that the compiler's wait
    // analysis tells a stage's copies from another stage's reads.
    __shared__ uint4 x0s[PQ_BM * 4], x1s[PQ_BM * 4], x2s[PQ_BM * 4], x3s[PQ_BM * 4];
    __shared__ __attribute__((aligned(16))) uint8_t c0s[PQ_WBYTES], c1s[PQ_WBYTES];
    if ((int)blockIdx.x < p.g1)
        pq_gemm_body<FMT, 0, PQ_BM, true>(p, blockIdx.x, x0s, x1s, x2s, x3s, c0s, c1s);
    else
        pq_gemm_body<FMT, 1, PQ_BM, true>(p, blockIdx.x - p.g1, x0s, x1s, x2s, x3s, c0s, c1s);
}

// ---------------------------------------------------------------------------
// pf_router_gemm: router logits of bf16 tokens as a tiled GEMM on the matrix
// cores.  One block = 64 tokens x all experts (<= 256) x one of ksplit parts
// of the reduction; wave w owns experts 64w .. 64w + 63 (2 x 32) against the
// 64 tokens (2 x 32).  The tokens and router rows of each 32-input step are
// copied to a 4-stage LDS ring by buffer-to-LDS DMA three steps ahead, as in
// pf_gemm.  bf16 x bf16 products are exact in the fp32 accumulator.  Output:
// the part's partial logits (no bias; pf_topk sums the parts in order) and,
// when the expert GEMMs follow, the fp16 copy of the block's slice of x.
// The blocks of one part run on one XCD pair, whose L2 then holds only that
// part of the router.  X16: write the fp16 copy of x.
// ---------------------------------------------------------------------------
constexpr int RG_NS = 4;       // LDS stages (at most 6)
constexpr int RG_UNROLL = 16;  // steps per loop trip (multiple of RG_NS)
static_assert(RG_NS <= 6 && RG_UNROLL % RG_NS == 0, "router GEMM pipeline shape");

template <int X16>
__global__ void __launch_bounds__(PF_THREADS) pf_router_gemm(PfParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    // one LDS object per stage (unused ones are dropped)
    __shared__ uint4 x0s[RG_BT * 4], x1s[RG_BT * 4], x2s[RG_BT * 4], x3s[RG_BT * 4], x4s[RG_BT * 4], x5s[RG_BT * 4];
    __shared__ uint4 r0s[256 * 4], r1s[256 * 4], r2s[256 * 4], r3s[256 * 4], r4s[256 * 4], r5s[256 * 4];
#define RG_XST(st) ((st) == 0 ? x0s : (st) == 1 ? x1s : (st) == 2 ? x2s : (st) == 3 ? x3s : (st) == 4 ? x4s : x5s)
#define RG_RST(st) ((st) == 0 ? r0s : (st) == 1 ? r1s : (st) == 2 ? r2s : (st) == 3 ? r3s : (st) == 4 ? r4s : r5s)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int S = p.ksplit, T = p.T, D = p.D, E = p.E;
    const int xcd = blockIdx.x % 8;
    const int ks = xcd % S;
    const int t0 = ((blockIdx.x / 8) * (8 / S) + xcd / S) * RG_BT;
    if (t0 >= T) return;
    const int NK = D / 32;
    const int kb_lo = ks * NK / S, n = (ks + 1) * NK / S - kb_lo;

    // stage slot j holds row j / 4, 16-byte chunk (j & 3) ^ pf_swz(row);
    // this thread fills token slot tid and router slots i * 256 + tid, whose
    // rows 64 i + tid / 4 share the swizzle of row tid / 4
    const int xr = tid >> 2, xc = (tid & 3) ^ pf_swz(xr);
    RgDma dma;
    dma.wave = wave;
    dma.rx = buf_rsrc(p.x, (uint32_t)((size_t)T * D * 2));
    dma.rr = buf_rsrc(p.router, (uint32_t)E * D * 2);
    dma.xo = (uint32_t)min(t0 + xr, T - 1) * D * 2 + 16 * xc + 64 * kb_lo;
#pragma unroll
    for (int i = 0; i < 4; i++) dma.ro[i] = (uint32_t)min(64 * i + xr, E - 1) * D * 2 + 16 * xc + 64 * kb_lo;
    // rows past T hold row T - 1 (clamped DMA) and rewrite its identical values
    _Float16 *x16p = p.x16 + (size_t)min(t0 + xr, T - 1) * D + 32 * kb_lo + 8 * xc;

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
            for (int j = 0; j < 16; j++) acc[a][b][j] = 0.f;

#pragma unroll
    for (int s = 0; s < RG_NS - 1; s++) rg_issue(dma, RG_XST(s), RG_RST(s), min(s, n - 1));

    for (int kb0 = 0; kb0 < n; kb0 += RG_UNROLL) {
        _Float16 *x16b = x16p + 32 * kb0;
#pragma unroll
        for (int u = 0; u < RG_UNROLL; u++) {
            const int kb = kb0 + u;
            if (kb >= n) break;
            wait_vmcnt<(RG_NS - 2) * 5>();
            pf_barrier();
            rg_issue(dma, RG_XST((u + RG_NS - 1) % RG_NS), RG_RST((u + RG_NS - 1) % RG_NS), min(kb + RG_NS - 1, n - 1));
            const uint4 *xs = RG_XST(u % RG_NS);
            const uint4 *rs = RG_RST(u % RG_NS);
            if (X16) {  // this thread's own token chunk of the step (packed by
                        // hand: a half8 store here stops the unrolling)
                const uint4 v = xs[tid];
                const uint32_t ww[4] = {v.x, v.y, v.z, v.w};
                uint32_t hh[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const half2_t h2 = {(_Float16)bf16lo(ww[j]), (_Float16)bf16hi(ww[j])};
                    hh[j] = __builtin_bit_cast(uint32_t, h2);
                }
                *reinterpret_cast<uint4 *>(x16b + 32 * u) = make_uint4(hh[0], hh[1], hh[2], hh[3]);
            }
#pragma unroll
            for (int s = 0; s < 2; s++) {
                const bf16x8_t a0 = as_bf16x8(rs[pf_slot(64 * wave + l32, 2 * s + g)]);
                const bf16x8_t a1 = as_bf16x8(rs[pf_slot(64 * wave + 32 + l32, 2 * s + g)]);
                const bf16x8_t b0 = as_bf16x8(xs[pf_slot(l32, 2 * s + g)]);
                const bf16x8_t b1 = as_bf16x8(xs[pf_slot(32 + l32, 2 * s + g)]);
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
            }
        }
    }

    // acc[a][b][j] = partial logit of expert 64 w + 32 a + 8 (j/4) + 4 g + j%4, token t0 + 32 b + l32
    float *part = p.part + (size_t)ks * T * E;
#pragma unroll
    for (int b = 0; b < 2; b++) {
        const int t = t0 + 32 * b + l32;
        if (t >= T) continue;
        float *prow = part + (size_t)t * E;
#pragma unroll
        for (int a = 0; a < 2; a++) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int e = 64 * wave + 32 * a + 8 * q + 4 * g;
                if ((E & 3) == 0) {
                    if (e < E)
                        *reinterpret_cast<float4 *>(prow + e) =
                            make_float4(acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (e + i < E) prow[e + i] = acc[a][b][4 * q + i];
                }
            }
        }
    }
#undef RG_XST
#undef RG_RST
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// pf_combine: y[t, 8i..8i+7] = sum over t's slots (routed in top-k order,
// then shared) of O[pos] (fp16, already scaled by the slot's weight),
// accumulated in fp32.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(PF_THREADS) pf_combine(PfParams p) {
    const size_t i = (size_t)blockIdx.x * PF_THREADS + threadIdx.x;
    const int D8 = p.D / 8;
    if (i >= (size_t)p.T * D8) return;
    const int t = (int)(i / D8), c = (int)(i % D8);
    const int KS = p.K + p.S;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < KS; j++) {
        const int r = p.pos[(size_t)t * KS + j];
        if (r < 0) continue;
        const uint4 v = reinterpret_cast<const uint4 *>(p.o + (size_t)r * p.D)[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const half2_t h2 = __builtin_bit_cast(half2_t, w[k]);
            s[2 * k] += (float)h2[0];
            s[2 * k + 1] += (float)h2[1];
        }
    }
    float4 *yo = reinterpret_cast<float4 *>(p.y) + 2 * i;
    yo[0] = make_float4(s[0], s[1], s[2], s[3]);
    yo[1] = make_float4(s[4], s[5], s[6], s[7]);
}

// grid of the grouped GEMMs for at most tiles_max tiles of MT blocks (the
// block -> tile order of xcd_tile_block: an XCD takes at most
// ceil(full / 8) + ceil(partial / 8) <= ceil(tiles_max / 8) + 1 tiles)
unsigned pf_gemm_grid(int tiles_max, int MT) { return (unsigned)(8 * MT * ((tiles_max + 7) / 8 + 1)); }

template <int FMT>
void launch_gemms(const PfParams &p, hipStream_t st) {
    const int mt0 = (p.F + 127) / 128, mt1 = (p.D + 255) / 256;
    // pf_ffn_q4 copies a row's NVFP4 block scales of a macro-stage as two
    // dwords, which must be 4-byte aligned in the matrix: K / 16 a multiple
    // of 4 for both matrices (d_model and d_ff multiples of 64); other shapes
    // take the one-step pipeline of pf_gemm
    const bool macro = prefill_fused(FMT, p.D, p.F);
    if constexpr (FMT == FMT_Q4_1 || FMT == FMT_NVFP4) {
        if (macro) {
            // both GEMMs in one dispatch (pf_ffn_q4): gate/up blocks first
            PfParams q = p;
            q.g1 = (int)pf_gemm_grid(p.tiles_max, mt0);
            const unsigned grid = (unsigned)q.g1 + pf_gemm_grid(p.tiles_max, mt1);
            MOE_LAUNCH(4, pf_ffn_q4<FMT>, dim3(grid), dim3(PF_THREADS), st, q);
            return;
        }
    }
    if constexpr (FMT != FMT_Q4_1) {
        MOE_LAUNCH(4, (pf_gemm<FMT, 0>), dim3(pf_gemm_grid(p.tiles_max, mt0)), dim3(PF_THREADS), st, p);
        MOE_LAUNCH(5, (pf_gemm<FMT, 1>), dim3(pf_gemm_grid(p.tiles_max, mt1)), dim3(PF_THREADS), st, p);
    }
}

}  // namespace

bool prefill_fused(int fmt, int D, int F) {
    return fmt == FMT_Q4_1 || (fmt == FMT_NVFP4 && D % 64 == 0 && F % 64 == 0);
}

const char *prefill_names(int act, bool fused) {
    // with the GEMMs fused, slot 4 is the fused kernel and slot 5 does not run
    if (fused)
        return act == MOE_ACT_F32 ? "pf_logits;pf_topk;pf_scan;pf_scatter;pf_ffn;pf_gemm_down;pf_combine"
                                  : "pf_router_gemm;pf_topk;pf_scan;pf_scatter;pf_ffn;pf_gemm_down;pf_combine";
    return act == MOE_ACT_F32 ? "pf_logits;pf_topk;pf_scan;pf_scatter;pf_gemm_gateup;pf_gemm_down;pf_combine"
                              : "pf_router_gemm;pf_topk;pf_scan;pf_scatter;pf_gemm_gateup;pf_gemm_down;pf_combine";
}

size_t prefill_ws_bytes(int D, int F, int E, int S, int K, int T) { return pf_layout(D, F, E, S, K, T).total; }

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st) {
    if (a.E > 256 || a.K > PF_MAX_TOPK || a.D % 32 || a.F % 32) return hipErrorNotSupported;
    const PfWs L = pf_layout(a.D, a.F, a.E, a.S, a.K, a.T);
    PfParams p{};
    p.D = a.D; p.F = a.F; p.E = a.E; p.S = a.S; p.K = a.K; p.T = a.T; p.act = a.act;
    p.NW = L.NW; p.R = L.R; p.tiles_max = L.tiles_max;
    p.want_x16 = a.route_only ? 0 : 1;
    p.ev = a.ev;
    p.expert_bytes = a.expert_bytes;
    p.x = a.x; p.router = a.router; p.bias = a.bias; p.experts = a.experts; p.tscale = a.tscale;
    p.y = a.y; p.idx_out = a.idx_out; p.w_out = a.w_out; p.logits_out = a.logits_out;
    p.logits = a.logits_out ? a.logits_out : wsp<float>(a.ws, L.logits);
    p.part = wsp<float>(a.ws, L.part);
    p.ksplit = L.ksplit;
    p.BM = a.fmt == FMT_Q4_1 ? PQ_BM : PF_BM;
    p.x16 = wsp<_Float16>(a.ws, L.x16);
    p.idx = wsp<int32_t>(a.ws, L.idx);
    p.w = wsp<float>(a.ws, L.w);
    p.mask = wsp<unsigned long long>(a.ws, L.mask);
    p.wp = wsp<int32_t>(a.ws, L.wp);
    p.off = wsp<int32_t>(a.ws, L.off);
    p.tiles = wsp<PfTile>(a.ws, L.tiles);
    p.meta = wsp<int32_t>(a.ws, L.meta);
    p.tile_done = wsp<int32_t>(a.ws, L.done);
    p.perm_tok = wsp<int32_t>(a.ws, L.perm_tok);
    p.perm_w = wsp<float>(a.ws, L.perm_w);
    p.pos = wsp<int32_t>(a.ws, L.pos);
    p.h = wsp<_Float16>(a.ws, L.h);
    p.o = wsp<_Float16>(a.ws, L.o);
    const int nb64 = (a.T + 63) / 64;
    if (!a.given_idx) {
        const dim3 gk(4 * L.NW);  // pf_topk: 16-token blocks over whole mask words
        if (a.act == MOE_ACT_F32) {
            // fp32 tokens: the two-term bf16 split needs the pf_logits kernel
            MOE_LAUNCH(0, (pf_logits<0, 4>), dim3((a.T + 31) / 32, (a.E + 31) / 32), dim3(PF_THREADS), st, p);
            MOE_LAUNCH(1, pf_topk<0>, gk, dim3(PF_TOPK_THREADS), st, p);
        } else {
            const int ntt = (a.T + RG_BT - 1) / RG_BT;
            const dim3 gr((unsigned)((ntt * p.ksplit + 7) / 8 * 8));
            if (p.want_x16)
                MOE_LAUNCH(0, pf_router_gemm<1>, gr, dim3(PF_THREADS), st, p);
            else
                MOE_LAUNCH(0, pf_router_gemm<0>, gr, dim3(PF_THREADS), st, p);
            switch (p.ksplit) {
            case 1: MOE_LAUNCH(1, pf_topk<1>, gk, dim3(PF_TOPK_THREADS), st, p); break;
            case 2: MOE_LAUNCH(1, pf_topk<2>, gk, dim3(PF_TOPK_THREADS), st, p); break;
            case 4: MOE_LAUNCH(1, pf_topk<4>, gk, dim3(PF_TOPK_THREADS), st, p); break;
            default: MOE_LAUNCH(1, pf_topk<8>, gk, dim3(PF_TOPK_THREADS), st, p); break;
            }
        }
        if (a.route_only) return hipGetLastError();
    } else {
        p.idx = const_cast<int32_t *>(a.given_idx);
        p.w = const_cast<float *>(a.given_w);
        const size_t n8 = (size_t)a.T * a.D / 8;
        const dim3 gx((unsigned)((n8 + PF_THREADS - 1) / PF_THREADS));
        if (a.act == MOE_ACT_F32)
            hipLaunchKernelGGL((pf_x16<0>), gx, dim3(PF_THREADS), 0, st, p);
        else
            hipLaunchKernelGGL((pf_x16<1>), gx, dim3(PF_THREADS), 0, st, p);
        MOE_LAUNCH(1, pf_mask_given, dim3(nb64), dim3(PF_THREADS), st, p);
    }
    MOE_LAUNCH(2, pf_scan, dim3(1), dim3(PF_SCAN_THREADS), st, p);
    MOE_LAUNCH(3, pf_scatter, dim3((a.T * (a.K + a.S) + PF_THREADS - 1) / PF_THREADS), dim3(PF_THREADS), st, p);
    if (a.fmt == FMT_Q4_1)
        launch_gemms<FMT_Q4_1>(p, st);
    else if (a.fmt == FMT_NVFP4)
        launch_gemms<FMT_NVFP4>(p, st);
    else
        launch_gemms<FMT_BF16>(p, st);
    const size_t n8 = (size_t)a.T * a.D / 8;
    MOE_LAUNCH(6, pf_combine, dim3((unsigned)((n8 + PF_THREADS - 1) / PF_THREADS)), dim3(PF_THREADS), st, p);
    return hipGetLastError();
}


}  // namespace moe
