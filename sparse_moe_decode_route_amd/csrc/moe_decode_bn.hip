// Decode path for a small batch (1 <= T <= 32 tokens) of regular shape.
//
// The layer is the same as on the batch-1 path (the Flint 40B-A2.5B pages,
// "Recursive Flint 40B-A2.5B", orcarouter.ai blog, section "The architecture
// is a memory-bandwidth argument": 256 routed experts, 6 chosen per token,
// one shared expert; decode time is weight traffic).  Three kernels:
//
//   bn_router   router logits: one block per expert row, one wave per token
//               (the batch-1 router's reduction per wave); in a stack
//               x_t = y_t / rms(y_t) is never written: the router and gate/up
//               kernels apply each token's 1/rms, computed from the loads they
//               already make
//   bn_gateup   one wave per (item, 2-4 features).  Items: each shared expert
//               with a pair of tokens, then every (token t, selection j): the
//               wave finds token t's j-th expert itself from the logits (the
//               batch-1 selection rounds), so no selection kernel or work
//               list sits between the router and the weight stream.  A
//               routed expert chosen by several tokens is read once per token
//               (at 8 tokens and 256 experts, 48 selections hit ~45 experts;
//               repeats are served by L2)
//   bn_down     8 output rows per block; wave t takes token t's selections
//               (written by the gate/up wave of its first selection) and sums
//               its down terms (its
//               shared slots, then its selections in top-k order) in batches
//               of 4 with every load of a batch in flight
// h is kept per (token, slot of the token): [T][S + K][F].
// No floating-point atomics; every sum has a fixed order.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BN_WAVES = 4;     // waves per block in gate/up
constexpr int BN_RR = 2;        // output rows per lane group in down
constexpr int BN_PB = 4;        // list entries per load batch in down
constexpr int BN_MAXB = 3;      // batches per wave: a token's list has K + S <= 12 entries
constexpr int BN_ROUTER_WAVES = 16;  // tokens per router block

// ---------------------------------------------------------------------------
// bn_router: logits[t, e] = x_t . Wr[e] (+ bias[e]) for T <= 32 tokens.  One
// block per (expert row, group of up to 16 tokens), wave w = token
// 16 * blockIdx.y + w; each wave sums its lane's units in
// order and then across the wave (DPP butterfly), as the batch-1 router does,
// so the same fp32 rounding band holds.  SCALED: x_t = y_t / rms(y_t) from
// the previous layer's output, the sum of squares taken from the wave's own
// loads of y_t.  d_model = 512 * UPLR.
// ---------------------------------------------------------------------------
template <int UPLR, bool SCALED>
__global__ void __launch_bounds__(MOE_WAVE *BN_ROUTER_WAVES) bn_router(DecodeParams p) {
    const int lane = threadIdx.x & (MOE_WAVE - 1);
    const int t = blockIdx.y * BN_ROUTER_WAVES + threadIdx.x / MOE_WAVE;
    if (t >= p.T) return;  // a group's unused waves
    const int e = blockIdx.x;
    const float *xin = (SCALED ? p.x_prev : p.x) + (size_t)t * p.D;
    float4 yr[2 * UPLR];
    load_rms_part<UPLR>(yr, xin);
    Mat mr{(const uint8_t *)p.router, p.E, p.D, 1.f};
    WUnit w[UPLR];
#pragma unroll
    for (int i = 0; i < UPLR; i++) w[i] = load_unit<FMT_BF16>(mr, e, lane + MOE_WAVE * i);
    __builtin_amdgcn_sched_barrier(0);
    const float xs = SCALED ? inv_rms_from<UPLR>(yr) : 1.f;
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
    const float sum = wave_sum(acc);
    if (lane == 0) p.logits[(size_t)t * p.E + e] = p.bias ? sum + p.bias[e] : sum;
}

// h for one work item from weights and x in registers: the wave holds the
// tokens' whole rows, so 1/rms comes from them (1 outside a stack).
template <int FMT, int UPLD, int RG, bool TWO>
__device__ __forceinline__ void bn_gateup_finish(const DecodeParams &p, const WUnit (&wg)[RG][UPLD],
                                                 const WUnit (&wu)[RG][UPLD], const XUnit<FMT> (&xa)[UPLD],
                                                 const XUnit<FMT> (&xb)[UPLD], float tsg, float tsu, bool scaled,
                                                 int slot, int ta, int tb, int f0) {
    const int lane = threadIdx.x & 63;
    float inv[2] = {1.f, 1.f};
    if (scaled) {
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int i = 0; i < UPLD; i++)
#pragma unroll
            for (int k = 0; k < Unit<FMT>::E; k++) {
                sa = __builtin_fmaf(xa[i].v[k], xa[i].v[k], sa);
                if (TWO) sb = __builtin_fmaf(xb[i].v[k], xb[i].v[k], sb);
            }
        inv[0] = 1.0f / sqrtf(wave_sum(sa) / (float)p.D + 1e-6f);
        if (TWO) inv[1] = 1.0f / sqrtf(wave_sum(sb) / (float)p.D + 1e-6f);
    }
    float ag[RG][2], au[RG][2];
#pragma unroll
    for (int r = 0; r < RG; r++) {
        ag[r][0] = ag[r][1] = au[r][0] = au[r][1] = 0.f;
#pragma unroll
        for (int i = 0; i < UPLD; i++) {
            if (TWO) {
                float g0, g1, u0, u1;
                unit_dot2<FMT>(wg[r][i], xa[i], xb[i], tsg, g0, g1);
                unit_dot2<FMT>(wu[r][i], xa[i], xb[i], tsu, u0, u1);
                ag[r][0] += g0;
                ag[r][1] += g1;
                au[r][0] += u0;
                au[r][1] += u1;
            } else {
                ag[r][0] += unit_dot<FMT>(wg[r][i], xa[i], tsg);
                au[r][0] += unit_dot<FMT>(wu[r][i], xa[i], tsu);
            }
        }
    }
    // all RG x tokens x (gate, up) sums in one halving reduction: value
    // k = (RG * NT) * (0 gate, 1 up) + NT * r + j ends in lanes l % PV == k,
    // so lane NT * r + j holds the gate sum and its up sum sits PV / 2 lanes on
    constexpr int NT = TWO ? 2 : 1, PV = 2 * RG * NT;
    static_assert(PV == 4 || PV == 8 || PV == 16, "one exchange pairs the gate and up sums");
    float v[PV];
#pragma unroll
    for (int r = 0; r < RG; r++)
#pragma unroll
        for (int j = 0; j < NT; j++) {
            v[NT * r + j] = ag[r][j];
            v[RG * NT + NT * r + j] = au[r][j];
        }
    const float red = wave_reduce_rows<PV>(v, lane);
    const float up = xor_lane(red, PV == 16 ? 3 : PV == 8 ? 2 : 1);  // lane ^ (PV / 2)
    const int k = lane % PV;
    if (k < RG * NT) {
        const int r = k / NT, j = k % NT;
        const float sc = j == 0 ? inv[0] : inv[1];
        const int t = j == 0 ? ta : tb;
        if (lane == k) p.h[((size_t)t * (p.S + p.K) + slot) * p.F + f0 + r] = silu_mul(red * sc, up * sc);
    }
}

// ---------------------------------------------------------------------------
// bn_gateup: wave gw -> item gw / (F / RG), features f0 .. f0 + RG - 1.
// Items 0 .. S*ceil(T/2)-1: shared expert s with tokens 2i and 2i+1 (or 2i
// alone); then item S*ceil(T/2) + K t + j: token t's j-th selection.
// h[(t * (S + K) + slot) * F + f] = silu(Wg x_t)[f] * (Wu x_t)[f], slot = s
// for shared expert s, S + j for selection j.
// Weight loads first; the tokens' x rows go to LDS by contiguous loads of the
// whole block and are read back per lane unit.
// ---------------------------------------------------------------------------
template <int FMT, int UPLD, int RG>
__global__ void __launch_bounds__(MOE_WAVE *BN_WAVES) bn_gateup(DecodeParams p) {
    __shared__ uint4 xs[2][UPLD * MOE_WAVE * Unit<FMT>::E / 4];  // both tokens' x, 16-byte chunks
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int per_item = p.F / RG;
    const int gw = blockIdx.x * BN_WAVES + wave;
    const int item = gw / per_item, f0 = (gw % per_item) * RG;
    const int pairs = (p.T + 1) / 2, n_shared_items = p.S * pairs;
    int slot, ta, tb, expert;
    bool two, sel_wave = false;
    float sel_lv[4];
    if (item < n_shared_items) {
        const int s2 = item / pairs, i = item % pairs;
        slot = s2;
        ta = 2 * i;
        two = 2 * i + 1 < p.T;
        tb = two ? 2 * i + 1 : ta;
        expert = p.E + s2;
    } else {
        const int r = item - n_shared_items;
        const int t = r / p.K, j = r % p.K;
        if (t >= p.T) return;  // past the last item (uniform per block: its waves share the item)
        slot = p.S + j;
        ta = tb = t;
        two = false;
        if (p.route_given) {
            expert = p.idx[t * p.K + j];
            if (expert < 0 || expert >= p.E) return;  // an invalid given index selects nothing
        } else {
            float lv[4];
            wave_topk_load(p.logits + (size_t)t * p.E, p.E, lv);
            expert = wave_topk_nth(lv, p.E, j);
            if (j == 0 && f0 == 0) {
                // the item's first wave also writes token t's full selection
                // with its weights, for the down kernel and the caller (after
                // this wave's weight loads below are in flight)
                sel_wave = true;
                for (int k = 0; k < 4; k++) sel_lv[k] = lv[k];
            }
        }
    }
    const uint8_t *eb = p.experts + (size_t)expert * p.expert_bytes;
    Mat mg{eb, p.F, p.D, tensor_scale<FMT>(p.tscale, 3 * expert + 0)};
    Mat mu{eb + mat_bytes<FMT>(p.F, p.D), p.F, p.D, tensor_scale<FMT>(p.tscale, 3 * expert + 1)};
    const bool scaled = p.x_prev != nullptr;  // stack: x is the previous output, normalised here
    const float *xin = scaled ? p.x_prev : p.x;
    WUnit wg[RG][UPLD], wu[RG][UPLD];
    XUnit<FMT> xa[UPLD], xb[UPLD];
#pragma unroll
    for (int r = 0; r < RG; r++)
#pragma unroll
        for (int i = 0; i < UPLD; i++) {
            wg[r][i] = load_unit<FMT>(mg, f0 + r, lane + MOE_WAVE * i);
            wu[r][i] = load_unit<FMT>(mu, f0 + r, lane + MOE_WAVE * i);
        }
    if (sel_wave) {
        int es;
        float wi;
        wave_topk_regs(sel_lv, p.E, p.K, &es, &wi);
        if (lane < p.K) {
            p.idx[ta * p.K + lane] = es;
            p.w[ta * p.K + lane] = wi;
            if (p.idx_out) p.idx_out[ta * p.K + lane] = es;
            if (p.w_out) p.w_out[ta * p.K + lane] = wi;
        }
    }
    // the block's waves share the item (F / RG is a multiple of BN_WAVES):
    // its tokens' x rows are loaded once, 1 KB contiguous per wave-wide load
    const int nq = p.D / 4;  // 16-byte chunks per row
    for (int q = threadIdx.x; q < nq; q += MOE_WAVE * BN_WAVES) {
        xs[0][xs_slot<FMT>(q)] = *reinterpret_cast<const uint4 *>(xin + (size_t)ta * p.D + 4 * q);
        xs[1][xs_slot<FMT>(q)] = *reinterpret_cast<const uint4 *>(xin + (size_t)tb * p.D + 4 * q);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < UPLD; i++) {
        load_x_lds<FMT>(xa[i], xs[0], lane + MOE_WAVE * i);
        load_x_lds<FMT>(xb[i], xs[1], lane + MOE_WAVE * i);
    }
    // the second token's arithmetic only runs for items that have one
    // (uniform branch)
    if (two)
        bn_gateup_finish<FMT, UPLD, RG, true>(p, wg, wu, xa, xb, mg.ts, mu.ts, scaled, slot, ta, tb, f0);
    else
        bn_gateup_finish<FMT, UPLD, RG, false>(p, wg, wu, xa, xb, mg.ts, mu.ts, scaled, slot, ta, tb, f0);
}

// ---------------------------------------------------------------------------
// bn_down: y[t, r] = sum over token t's list (its shared slots, then its
// selections in top-k order) of coef * (Wd[slot] row r . h[slot, t]).  One
// block per (ROWS output rows, group of up to 8 tokens); wave w = token
// 8 * blockIdx.y + w, so each wave sums its own token's terms in list order
// and writes its rows (no cross-wave reduction).
// Lanes: LPR_F lanes per row (one unit each), row groups of BN_RR rows.
// ---------------------------------------------------------------------------
template <int FMT, int LPR_F>
__global__ void __launch_bounds__(MOE_WAVE *MAX_DECODE_T) bn_down(DecodeParams p) {
    constexpr int UE = Unit<FMT>::E;
    constexpr int G = MOE_WAVE / LPR_F;  // row groups per wave
    constexpr int ROWS = G * BN_RR;      // rows per block
    constexpr int HCH = LPR_F * UE / 4;  // 16-byte chunks of one h row (d_ff floats)
    constexpr int HLD = (HCH + MOE_WAVE - 1) / MOE_WAVE;  // wave-wide loads per h row
    // per wave: the h rows of one batch, each in the unit-swizzled chunk order
    __shared__ uint4 hs[MAX_DECODE_T][BN_PB * HCH];  // per wave
    const int lane = threadIdx.x & 63;
    const int tw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave within the block
    const int t = blockIdx.y * MAX_DECODE_T + tw;
    if (t >= p.T) return;  // a group's unused waves (no block-wide synchronisation below)
    const int grp = lane / LPR_F, sub = lane % LPR_F;
    const int D = p.D, F = p.F;
    const int r0 = blockIdx.x * ROWS + grp * BN_RR;
    const int KS = p.K + p.S;
    // the token's list (its shared slots, then its selections in top-k
    // order): lane i
    // holds entry i = {h row, valid, coef bits, expert}; every entry is then
    // read out as wave-uniform (scalar) values where it is used (no per-lane
    // array of entries: indexed by the batch loop, it would live in scratch)
    // (the given routing, or the selection the gate/up kernel wrote)
    const int es = lane < p.K ? p.idx[t * p.K + lane] : 0;
    const float wi = lane < p.K ? p.w[t * p.K + lane] : 0.f;
    int4 mine;
    {
        const int j = min(max(lane - p.S, 0), p.K - 1);
        const int ej = __shfl(es, j, 64);
        const float wj = __shfl(wi, j, 64);
        const bool shared = lane < p.S;
        const bool valid = shared || (ej >= 0 && ej < p.E);
        mine = make_int4(t * KS + min(lane, KS - 1), valid ? t : -1, __float_as_int(shared ? 1.f : wj),
                         shared ? p.E + lane : (valid ? ej : 0));
    }
    auto entry = [&](int i) {
        const int j = min(i, KS - 1);
        return make_int4(__builtin_amdgcn_readlane(mine.x, j), __builtin_amdgcn_readlane(mine.y, j),
                         __builtin_amdgcn_readlane(mine.z, j), __builtin_amdgcn_readlane(mine.w, j));
    };
    float acc[BN_RR];
#pragma unroll
    for (int r = 0; r < BN_RR; r++) acc[r] = 0.f;
#pragma unroll
    for (int bt = 0; bt < BN_MAXB; bt++) {
        if (bt * BN_PB >= KS) break;
        // one batch: BN_PB entries (past the list's end: weight 0)
        WUnit wd[BN_PB][BN_RR];
        XUnit<FMT> hv[BN_PB];
        float coef[BN_PB], ts[BN_PB];
        bool on[BN_PB];
#pragma unroll
        for (int q = 0; q < BN_PB; q++) {
            const int j = bt * BN_PB + q;
            const int4 pr = entry(j);
            // an entry past the list or of an invalid given index adds nothing
            // (its h row was never written: selected out, not multiplied by 0)
            on[q] = j < KS && pr.y >= 0;
            coef[q] = __int_as_float(pr.z);
            const uint8_t *eb = p.experts + (size_t)pr.w * p.expert_bytes;
            Mat md{eb + 2 * mat_bytes<FMT>(F, D), D, F, tensor_scale<FMT>(p.tscale, 3 * pr.w + 2)};
            ts[q] = md.ts;
#pragma unroll
            for (int r = 0; r < BN_RR; r++) wd[q][r] = load_unit<FMT>(md, min(r0 + r, D - 1), sub);
        }
        // the batch's h rows: contiguous 16-byte loads (1 KB per wave-wide
        // load) into this wave's LDS region, then per-lane units from LDS
        uint4 hc[BN_PB][HLD];
#pragma unroll
        for (int q = 0; q < BN_PB; q++) {
            const uint4 *hsrc = reinterpret_cast<const uint4 *>(p.h + (size_t)entry(bt * BN_PB + q).x * F);
#pragma unroll
            for (int i = 0; i < HLD; i++) hc[q][i] = hsrc[min(lane + MOE_WAVE * i, HCH - 1)];
        }
        // (a wave's LDS accesses complete in issue order, so these writes do
        // not overtake the previous batch's reads of the same region)
#pragma unroll
        for (int q = 0; q < BN_PB; q++)
#pragma unroll
            for (int i = 0; i < HLD; i++)
                if (lane + MOE_WAVE * i < HCH) hs[tw][q * HCH + xs_slot<FMT>(lane + MOE_WAVE * i)] = hc[q][i];
#pragma unroll
        for (int q = 0; q < BN_PB; q++) {
            load_x_lds<FMT>(hv[q], &hs[tw][q * HCH], sub);
#pragma unroll
            for (int r = 0; r < BN_RR; r++) {
                const float v = acc[r] + coef[q] * unit_dot<FMT>(wd[q][r], hv[q], ts[q]);
                acc[r] = on[q] ? v : acc[r];
            }
        }
    }
#pragma unroll
    for (int r = 0; r < BN_RR; r++) {
        const float y = group_sum<LPR_F>(acc[r]);
        if (sub == 0 && r0 + r < D) p.y[(size_t)t * D + r0 + r] = y;
    }
}

template <int FMT, int UPLD, int LPR_F>
hipError_t launch_bn_fmt(const DecodeParams &p, hipStream_t st) {
    const int S = p.S;
    constexpr int RG = UPLD == 1 ? 4 : 2;  // features per wave (register budget)
    const int max_items = S * ((p.T + 1) / 2) + p.T * p.K;
    const int waves_g = max_items * (p.F / RG);
    MOE_LAUNCH(1, (bn_gateup<FMT, UPLD, RG>), dim3((waves_g + BN_WAVES - 1) / BN_WAVES), dim3(MOE_WAVE * BN_WAVES),
               st, p);
    const int rows = (MOE_WAVE / LPR_F) * BN_RR;
    const int tg = (p.T + MAX_DECODE_T - 1) / MAX_DECODE_T;  // token groups of up to 8 waves
    MOE_LAUNCH(2, (bn_down<FMT, LPR_F>), dim3((p.D + rows - 1) / rows, tg), dim3(MOE_WAVE * min(p.T, MAX_DECODE_T)),
               st, p);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_bn_shape(const DecodeParams &p, hipStream_t st) {
    constexpr int UE = Unit<FMT>::E;
    if (p.D % (MOE_WAVE * UE)) return hipErrorNotSupported;
    const int upld = p.D / (MOE_WAVE * UE), lpr_f = p.F / UE;
    if (p.F % UE || p.F % 4) return hipErrorNotSupported;
    if (upld == 1 && lpr_f == 16) return launch_bn_fmt<FMT, 1, 16>(p, st);
    if (upld == 1 && lpr_f == 32) return launch_bn_fmt<FMT, 1, 32>(p, st);
    if (upld == 2 && lpr_f == 16) return launch_bn_fmt<FMT, 2, 16>(p, st);
    if (upld == 2 && lpr_f == 32) return launch_bn_fmt<FMT, 2, 32>(p, st);
    return hipErrorNotSupported;
}

template <int FMT>
bool bn_shape_ok(const DecodeParams &p) {
    constexpr int UE = Unit<FMT>::E;
    if (p.D % (MOE_WAVE * UE) || p.F % UE || p.F % 4) return false;
    const int upld = p.D / (MOE_WAVE * UE), lpr_f = p.F / UE;
    const int rg = upld == 1 ? 4 : 2;  // features per gate/up wave: a block's waves share one item
    return (upld == 1 || upld == 2) && (lpr_f == 16 || lpr_f == 32) && (p.F / rg) % BN_WAVES == 0;
}

}  // namespace

bool decode_bn_supported(int fmt, int D, int F, int E, int S) {
    DecodeParams p{};
    p.D = D;
    p.F = F;
    const bool shape = fmt == FMT_Q4_1 ? bn_shape_ok<FMT_Q4_1>(p)
                       : fmt == FMT_NVFP4 ? bn_shape_ok<FMT_NVFP4>(p)
                                          : bn_shape_ok<FMT_BF16>(p);
    const int u = D / 512;  // router units per lane
    return shape && E <= 256 && S <= 4 && D % 512 == 0 && (u == 1 || u == 2 || u == 4 || u == 8);
}

// Kernel slots: 0 logits, 1 gate/up, 2 down.
hipError_t launch_decode_bn(const DecodeParams &p, hipStream_t st) {
    if (p.T < 1 || p.T > MAX_BN_T || p.E > 256 || p.S > 4 || !p.want_shared) return hipErrorNotSupported;
    const bool ok = p.fmt == FMT_Q4_1 ? bn_shape_ok<FMT_Q4_1>(p)
                    : p.fmt == FMT_NVFP4 ? bn_shape_ok<FMT_NVFP4>(p)
                                         : bn_shape_ok<FMT_BF16>(p);
    if (!ok) return hipErrorNotSupported;
    if (!p.route_given) {
        if (!p.want_router || p.D % 512) return hipErrorNotSupported;
        const dim3 gr(p.E, (p.T + BN_ROUTER_WAVES - 1) / BN_ROUTER_WAVES), br(MOE_WAVE * min(p.T, BN_ROUTER_WAVES));
#define BN_ROUTER(U)                                                                  \
    if (p.x_prev)                                                                     \
        MOE_LAUNCH(0, (bn_router<U, true>), gr, br, st, p);                           \
    else                                                                              \
        MOE_LAUNCH(0, (bn_router<U, false>), gr, br, st, p);
        switch (p.D / 512) {
        case 1: BN_ROUTER(1) break;
        case 2: BN_ROUTER(2) break;
        case 4: BN_ROUTER(4) break;
        case 8: BN_ROUTER(8) break;
        default: return hipErrorNotSupported;
        }
#undef BN_ROUTER
    }
    if (p.fmt == FMT_Q4_1) return launch_bn_shape<FMT_Q4_1>(p, st);
    if (p.fmt == FMT_NVFP4) return launch_bn_shape<FMT_NVFP4>(p, st);
    return launch_bn_shape<FMT_BF16>(p, st);
}

}  // namespace moe
