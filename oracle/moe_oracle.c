/*
 * CPU oracle for the sparse mixture-of-experts FFN layer at token decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg do.  It shares no source with
 * the HIP library.
 *
 * What it computes follows the Flint 40B-A2.5B pages:
 *   - "Recursive Flint 40B-A2.5B" (orcarouter.ai blog), section "The
 *     architecture is a memory-bandwidth argument", sparsity bullet: per MoE
 *     layer 256 routed experts, 6 selected per token, plus one always-active
 *     shared expert; decode reads only the selected experts' weights.
 *   - the same page, sections "What shipped" and "The quantisation recipe is
 *     the most transferable part": 4-bit q4_1 and NVFP4 weight files.
 *   - "Flint ... published as GGUF" (648news.com), section "MoE structure and
 *     recommended settings": 47 of 49 layers are MoE, 6 of 256 experts.
 * The pages leave the gating function, the expert activation, the block
 * layouts and the tie-break open; the readings taken are:
 *   router logits l_e = sum_k x_k * Wr[e,k] (+ bias_e); p = softmax(l) over
 *   all routed experts; S = the top_k experts after a stable sort on
 *   (logit descending, index ascending); w_i = p_i / sum_{j in S} p_j;
 *   expert FFN h = silu(Wg x) * (Wu x), o = Wd h, silu(z) = z / (1 + e^-z);
 *   y = sum of shared outputs (weight 1) + sum_{i in S, ascending index} w_i o_i;
 *   between stacked layers x_next = y / sqrt(mean(y^2) + 1e-6).
 *
 * Arithmetic is fp64 throughout, in plain loops, with no blocking or
 * reordering beyond the definitions above.  Every decoded weight is exact in
 * fp64 (4-bit code times an fp16/E4M3 scale plus an fp16 min, times an fp32
 * tensor scale), so the only roundings are those of the fp64 sums.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FMT_BF16 0
#define ORC_FMT_Q4_1 1
#define ORC_FMT_NVFP4 2

typedef struct {
    int32_t d_model, d_ff, n_routed, n_shared, top_k, wfmt;
} orc_dims;

/* ------------------------------------------------------------------------ */
/* scalar decoders: each field of the format read out and scaled by hand     */
/* ------------------------------------------------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
double orc_fp16(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + m, e - 25);
    return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
double orc_bf16(uint16_t b) {
    int s = (b >> 15) & 1, e = (b >> 7) & 255, m = b & 127;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(128.0 + m, e - 134);
    return s ? -v : v;
}

/* OCP FP8 E4M3 ("FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 * subnormals, no infinities, S.1111.111 is NaN, largest finite 448. */
double orc_e4m3(uint8_t c) {
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(8.0 + m, e - 10);
    return s ? -v : v;
}

/* OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit, no inf/NaN. */
double orc_e2m1(uint8_t c) {
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v;
    if (e == 0)
        v = 0.5 * m;
    else
        v = ldexp(2.0 + m, e - 2);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* matrix decoding: one row at a time into fp64                              */
/* ------------------------------------------------------------------------ */

static size_t mat_bytes(int fmt, int rows, int k) {
    if (fmt == ORC_FMT_BF16) return (size_t)rows * k * 2;
    if (fmt == ORC_FMT_Q4_1) return (size_t)rows * (k / 32) * 20;
    return (size_t)rows * (k / 2) + (size_t)rows * (k / 16);
}

size_t orc_expert_bytes(const orc_dims *dm) {
    return 2 * mat_bytes(dm->wfmt, dm->d_ff, dm->d_model) + mat_bytes(dm->wfmt, dm->d_model, dm->d_ff);
}

/* q4_1 block of 20 bytes: fp16 d, fp16 m, 16 bytes of codes; element j in the
 * low nibble of byte j, element j+16 in the high nibble; value d*q + m. */
void orc_dequant_q4_1_block(const uint8_t *blk, double out[32]) {
    double d = orc_fp16((uint16_t)(blk[0] | (blk[1] << 8)));
    double m = orc_fp16((uint16_t)(blk[2] | (blk[3] << 8)));
    for (int j = 0; j < 16; j++) {
        int lo = blk[4 + j] & 15, hi = blk[4 + j] >> 4;
        out[j] = d * lo + m;
        out[j + 16] = d * hi + m;
    }
}

/* Decode row r of a [rows, k] matrix stored in format fmt at base. */
void orc_dequant_row(int fmt, const uint8_t *base, int rows, int k, int r, double s_t, double *out) {
    if (fmt == ORC_FMT_BF16) {
        const uint8_t *p = base + (size_t)r * k * 2;
        for (int c = 0; c < k; c++) out[c] = orc_bf16((uint16_t)(p[2 * c] | (p[2 * c + 1] << 8)));
    } else if (fmt == ORC_FMT_Q4_1) {
        const uint8_t *p = base + (size_t)r * (k / 32) * 20;
        for (int b = 0; b < k / 32; b++) orc_dequant_q4_1_block(p + 20 * b, out + 32 * b);
    } else {
        const uint8_t *nib = base + (size_t)r * (k / 2);
        const uint8_t *sc = base + (size_t)rows * (k / 2) + (size_t)r * (k / 16);
        for (int c = 0; c < k; c++) {
            uint8_t byte = nib[c / 2];
            uint8_t code = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
            out[c] = orc_e2m1(code) * orc_e4m3(sc[c / 16]) * s_t;
        }
    }
}

/* Decode a whole [rows, k] matrix (tests use this to pin the decoders). */
void orc_dequant_matrix(int fmt, const uint8_t *base, int rows, int k, double s_t, double *out) {
    for (int r = 0; r < rows; r++) orc_dequant_row(fmt, base, rows, k, r, s_t, out + (size_t)r * k);
}

/* ------------------------------------------------------------------------ */
/* routing                                                                   */
/* ------------------------------------------------------------------------ */

/* logits[e] = sum_k x[k] * Wr[e,k] (+ bias[e]), Wr bf16 [n_routed, d]. */
void orc_router_logits(const orc_dims *dm, const double *x, const uint16_t *wr, const double *bias,
                       double *logits) {
    for (int e = 0; e < dm->n_routed; e++) {
        double acc = 0.0;
        for (int k = 0; k < dm->d_model; k++) acc += x[k] * orc_bf16(wr[(size_t)e * dm->d_model + k]);
        logits[e] = bias ? acc + bias[e] : acc;
    }
}

/* Full softmax over n logits. */
void orc_softmax(int n, const double *l, double *p) {
    double mx = l[0];
    for (int i = 1; i < n; i++)
        if (l[i] > mx) mx = l[i];
    double sum = 0.0;
    for (int i = 0; i < n; i++) {
        p[i] = exp(l[i] - mx);
        sum += p[i];
    }
    for (int i = 0; i < n; i++) p[i] /= sum;
}

/* Stable insertion sort of 0..n-1 by (logit descending, index ascending);
 * the first k entries are the selected experts. */
void orc_sort_experts(int n, const double *l, int32_t *order) {
    for (int i = 0; i < n; i++) order[i] = i;
    for (int i = 1; i < n; i++) {
        int32_t cur = order[i];
        int j = i - 1;
        while (j >= 0 && l[order[j]] < l[cur]) { /* strict: equal keys keep index order */
            order[j + 1] = order[j];
            j--;
        }
        order[j + 1] = cur;
    }
}

/* Route one token: selected indices (sorted order) and renormalised weights. */
void orc_route(const orc_dims *dm, const double *logits, const int32_t *forced, int32_t *idx, double *w,
               double *probs) {
    int E = dm->n_routed, K = dm->top_k;
    double *p = (double *)malloc(sizeof(double) * E);
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * E);
    orc_softmax(E, logits, p);
    if (forced) {
        for (int i = 0; i < K; i++) idx[i] = forced[i];
    } else {
        orc_sort_experts(E, logits, order);
        for (int i = 0; i < K; i++) idx[i] = order[i];
    }
    double den = 0.0;
    for (int i = 0; i < K; i++) den += p[idx[i]];
    for (int i = 0; i < K; i++) w[i] = p[idx[i]] / den;
    if (probs) memcpy(probs, p, sizeof(double) * E);
    free(p);
    free(order);
}

/* ------------------------------------------------------------------------ */
/* expert FFN                                                                */
/* ------------------------------------------------------------------------ */

/* o = Wd (silu(Wg x) * (Wu x)) for expert e; weights decoded row by row. */
void orc_expert_ffn(const orc_dims *dm, const uint8_t *experts, const float *tscale, int e, const double *x,
                    double *o) {
    int D = dm->d_model, F = dm->d_ff, fmt = dm->wfmt;
    const uint8_t *base = experts + (size_t)e * orc_expert_bytes(dm);
    const uint8_t *wg = base;
    const uint8_t *wu = wg + mat_bytes(fmt, F, D);
    const uint8_t *wd = wu + mat_bytes(fmt, F, D);
    double sg = tscale ? tscale[3 * e + 0] : 1.0;
    double su = tscale ? tscale[3 * e + 1] : 1.0;
    double sd = tscale ? tscale[3 * e + 2] : 1.0;
    double *row = (double *)malloc(sizeof(double) * (D > F ? D : F));
    double *h = (double *)malloc(sizeof(double) * F);
    for (int f = 0; f < F; f++) {
        double g = 0.0, u = 0.0;
        orc_dequant_row(fmt, wg, F, D, f, sg, row);
        for (int k = 0; k < D; k++) g += row[k] * x[k];
        orc_dequant_row(fmt, wu, F, D, f, su, row);
        for (int k = 0; k < D; k++) u += row[k] * x[k];
        h[f] = g / (1.0 + exp(-g)) * u;
    }
    for (int r = 0; r < D; r++) {
        double acc = 0.0;
        orc_dequant_row(fmt, wd, D, F, r, sd, row);
        for (int f = 0; f < F; f++) acc += row[f] * h[f];
        o[r] = acc;
    }
    free(row);
    free(h);
}

/* ------------------------------------------------------------------------ */
/* layer                                                                     */
/* ------------------------------------------------------------------------ */

/*
 * One MoE layer over T tokens.
 *   x        [T, d_model] inputs (fp64 copies of the fp32/bf16 values)
 *   wr       bf16 router [n_routed, d_model]; bias [n_routed] or NULL
 *   experts  canonical bytes of n_routed + n_shared experts
 *   tscale   NVFP4 tensor scales [(n_routed+n_shared)*3] or NULL
 *   forced   [T, top_k] expert indices to use instead of the selection
 *            (teacher forcing), or NULL
 *   dense    0: evaluate only the selected experts;
 *            1: evaluate every routed expert and weight the unselected by 0
 *   outputs  idx [T, top_k], w [T, top_k], logits [T, n_routed] (nullable),
 *            y [T, d_model]
 * Returns 0, or -1 on bad dimensions.
 */
int orc_layer_forward(const orc_dims *dm, int32_t T, const double *x, const uint16_t *wr, const double *bias,
                      const uint8_t *experts, const float *tscale, const int32_t *forced, int32_t dense,
                      int32_t *idx, double *w, double *logits_out, double *y) {
    int D = dm->d_model, E = dm->n_routed, K = dm->top_k;
    if (D <= 0 || dm->d_ff <= 0 || E <= 0 || K <= 0 || K > E || dm->n_shared < 0) return -1;
    if (dm->wfmt == ORC_FMT_Q4_1 && (D % 32 || dm->d_ff % 32)) return -1;
    if (dm->wfmt == ORC_FMT_NVFP4 && (D % 16 || dm->d_ff % 16)) return -1;
    double *logits = (double *)malloc(sizeof(double) * E);
    double *o = (double *)malloc(sizeof(double) * D);
    for (int t = 0; t < T; t++) {
        const double *xt = x + (size_t)t * D;
        double *yt = y + (size_t)t * D;
        int32_t *it = idx + (size_t)t * K;
        double *wt = w + (size_t)t * K;
        orc_router_logits(dm, xt, wr, bias, logits);
        if (logits_out) memcpy(logits_out + (size_t)t * E, logits, sizeof(double) * E);
        orc_route(dm, logits, forced ? forced + (size_t)t * K : NULL, it, wt, NULL);
        for (int r = 0; r < D; r++) yt[r] = 0.0;
        for (int s = 0; s < dm->n_shared; s++) {
            orc_expert_ffn(dm, experts, tscale, E + s, xt, o);
            for (int r = 0; r < D; r++) yt[r] += o[r];
        }
        for (int e = 0; e < E; e++) {
            double we = 0.0;
            int sel = 0;
            for (int i = 0; i < K; i++)
                if (it[i] == e) {
                    we = wt[i];
                    sel = 1;
                }
            if (!sel && !dense) continue;
            orc_expert_ffn(dm, experts, tscale, e, xt, o);
            for (int r = 0; r < D; r++) yt[r] += we * o[r];
        }
    }
    free(logits);
    free(o);
    return 0;
}

/*
 * Expert FFN over a given routing: y = sum_shared expert_s(x) +
 * sum_i w[i] * expert_{idx[i]}(x), slots taken in the order given.
 */
int orc_experts_given(const orc_dims *dm, int32_t T, const double *x, const uint8_t *experts, const float *tscale,
                      const int32_t *idx, const double *w, double *y) {
    int D = dm->d_model, K = dm->top_k;
    double *o = (double *)malloc(sizeof(double) * D);
    for (int t = 0; t < T; t++) {
        const double *xt = x + (size_t)t * D;
        double *yt = y + (size_t)t * D;
        for (int r = 0; r < D; r++) yt[r] = 0.0;
        for (int s = 0; s < dm->n_shared; s++) {
            orc_expert_ffn(dm, experts, tscale, dm->n_routed + s, xt, o);
            for (int r = 0; r < D; r++) yt[r] += o[r];
        }
        for (int i = 0; i < K; i++) {
            orc_expert_ffn(dm, experts, tscale, idx[(size_t)t * K + i], xt, o);
            for (int r = 0; r < D; r++) yt[r] += w[(size_t)t * K + i] * o[r];
        }
    }
    free(o);
    return 0;
}

/* x_next = y / sqrt(mean(y^2) + eps), one token of length n. */
void orc_rmsnorm(int n, const double *y, double eps, double *out) {
    double ss = 0.0;
    for (int i = 0; i < n; i++) ss += y[i] * y[i];
    double r = sqrt(ss / n + eps);
    for (int i = 0; i < n; i++) out[i] = y[i] / r;
}

/*
 * A stack of n_layers independent layers, one token at a time:
 * x_0 = input, y_l = layer_l(x_l), x_{l+1} = rmsnorm(y_l).  layers_* are
 * host arrays of per-layer pointers.  y_trace [n_layers, T, d] receives every
 * y_l (nullable); y receives y_{n_layers-1}.  idx_trace [n_layers, T, top_k]
 * (nullable).
 */
int orc_stack_forward(const orc_dims *dm, int32_t n_layers, int32_t T, const double *x0,
                      const uint16_t *const *layers_wr, const uint8_t *const *layers_experts,
                      const float *const *layers_tscale, double *y, double *y_trace, int32_t *idx_trace) {
    int D = dm->d_model, K = dm->top_k;
    double *x = (double *)malloc(sizeof(double) * (size_t)T * D);
    double *yl = (double *)malloc(sizeof(double) * (size_t)T * D);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * K);
    double *w = (double *)malloc(sizeof(double) * (size_t)T * K);
    memcpy(x, x0, sizeof(double) * (size_t)T * D);
    int rc = 0;
    for (int l = 0; l < n_layers && rc == 0; l++) {
        rc = orc_layer_forward(dm, T, x, layers_wr[l], NULL, layers_experts[l],
                               layers_tscale ? layers_tscale[l] : NULL, NULL, 0, idx, w, NULL, yl);
        if (y_trace) memcpy(y_trace + (size_t)l * T * D, yl, sizeof(double) * (size_t)T * D);
        if (idx_trace) memcpy(idx_trace + (size_t)l * T * K, idx, sizeof(int32_t) * (size_t)T * K);
        for (int t = 0; t < T; t++) orc_rmsnorm(D, yl + (size_t)t * D, 1e-6, x + (size_t)t * D);
    }
    memcpy(y, yl, sizeof(double) * (size_t)T * D);
    free(x);
    free(yl);
    free(idx);
    free(w);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* 4-bit output layer (lm_head)                                              */
/* ------------------------------------------------------------------------ */

/*
 * Output-layer logits: logits[t, i] = sum_k x[t, k] * W[rows[i], k] for the
 * listed vocabulary rows (all rows 0..vocab-1 when rows is NULL and
 * n_rows == vocab).  W is [vocab, d] in format fmt, canonical layout, with
 * tensor scale s_t (NVFP4).  "Recursive Flint 40B-A2.5B" (orcarouter.ai
 * blog), section "The quantisation recipe is the most transferable part":
 * the output layer ships in 4 bits, since with 2.5 B active parameters it
 * is a large part of the weights every decoded token reads.  Each row is
 * decoded exactly into fp64 and summed over k in order.  logits is
 * [T, n_rows].  Returns -1 on a row index outside [0, vocab).
 */
int orc_lm_head(int fmt, const uint8_t *w, int32_t vocab, int32_t d, double s_t, int32_t T, const double *x,
                const int32_t *rows, int32_t n_rows, double *logits) {
    double *wr = (double *)malloc(sizeof(double) * (size_t)d);
    int rc = 0;
    for (int i = 0; i < n_rows && rc == 0; i++) {
        int r = rows ? rows[i] : i;
        if (r < 0 || r >= vocab) {
            rc = -1;
            break;
        }
        orc_dequant_row(fmt, w, vocab, d, r, s_t, wr);
        for (int t = 0; t < T; t++) {
            const double *xt = x + (size_t)t * d;
            double acc = 0.0;
            for (int k = 0; k < d; k++) acc += xt[k] * wr[k];
            logits[(size_t)t * n_rows + i] = acc;
        }
    }
    free(wr);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* decode attention (the step before the MoE FFN in every layer)             */
/* ------------------------------------------------------------------------ */

/* bfloat16 bits of v as a 32-bit producer stores it: v cast to float, then
 * rounded to nearest even (v finite). */
static uint16_t orc_to_bf16(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(r >> 16);
}

/* y = x / sqrt(mean(x^2) + eps) * w over one head of n values. */
static void orc_head_rmsnorm(int n, const double *x, const double *w, double eps, double *y) {
    double ss = 0.0;
    for (int i = 0; i < n; i++) ss += x[i] * x[i];
    double r = sqrt(ss / n + eps);
    for (int i = 0; i < n; i++) y[i] = x[i] / r * w[i];
}

/* Rotary embedding at position p, pairs (i, i + n/2) rotated by the angle
 * p * base^(-2i/n). */
static void orc_rope(int n, double *x, int p, double base) {
    int h = n / 2;
    for (int i = 0; i < h; i++) {
        double ang = (double)p * pow(base, -2.0 * i / n);
        double c = cos(ang), s = sin(ang);
        double a = x[i], b = x[i + h];
        x[i] = a * c - b * s;
        x[i + h] = a * s + b * c;
    }
}

/*
 * One decode step of attention for B sequences.  "Recursive Flint
 * 40B-A2.5B" (orcarouter.ai blog), section "The architecture is a
 * memory-bandwidth argument", attention and positional-encoding bullets:
 * 32 query heads share 4 key/value heads (head size 128); sliding-window
 * layers see the current token and the 512 before it and use rotary
 * embeddings, full layers see every earlier token and use none; each head's
 * queries and keys are RMS-normalised, and every head has a learned sink.
 * For sequence b with new position P = pos[b]:
 *   q_h = rope(rmsnorm(q[b,h]) * qw) (rope only when window > 0), likewise
 *   k for each key/value head; k and v are stored in the caches at P in
 *   bfloat16;
 *   head h reads key/value head g = h / (Hq / Hkv) at positions
 *   j in [max(0, P - window + 1), P] (all j <= P when window == 0);
 *   s_j = q_h . K[j] / sqrt(D); the sink logit z_h joins the softmax
 *   denominator only: out = sum_j e^{s_j} V[j] / (sum_j e^{s_j} + e^{z_h}).
 * Caches are bfloat16 [B, Hkv, max_len, D]; q, out [B, Hq, D]; k_new, v_new
 * [B, Hkv, D].  The stored k and v are rounded to bfloat16 from fp32 (the
 * fp64 value cast to float, then round to nearest even).  Returns -1 on a
 * position outside [0, max_len).
 */
int orc_attn_decode(int Hq, int Hkv, int D, int window, double rope_base, double eps, int B, const double *q,
                    const double *k_new, const double *v_new, const double *qw, const double *kw,
                    const double *sinks, uint16_t *k_cache, uint16_t *v_cache, int max_len, const int32_t *pos,
                    double *out) {
    double *qh = (double *)malloc(sizeof(double) * D);
    double *kh = (double *)malloc(sizeof(double) * D);
    double *sc = (double *)malloc(sizeof(double) * (size_t)max_len);
    int grp = Hq / Hkv, rc = 0;
    for (int b = 0; b < B && rc == 0; b++) {
        int P = pos[b];
        if (P < 0 || P >= max_len) {
            rc = -1;
            break;
        }
        for (int g = 0; g < Hkv; g++) {
            orc_head_rmsnorm(D, k_new + ((size_t)b * Hkv + g) * D, kw, eps, kh);
            if (window > 0) orc_rope(D, kh, P, rope_base);
            uint16_t *kc = k_cache + (((size_t)b * Hkv + g) * max_len + P) * D;
            uint16_t *vc = v_cache + (((size_t)b * Hkv + g) * max_len + P) * D;
            for (int d = 0; d < D; d++) {
                kc[d] = orc_to_bf16(kh[d]);
                vc[d] = orc_to_bf16(v_new[((size_t)b * Hkv + g) * D + d]);
            }
        }
        int lo = window > 0 ? (P - window + 1 > 0 ? P - window + 1 : 0) : 0;
        for (int h = 0; h < Hq; h++) {
            int g = h / grp;
            orc_head_rmsnorm(D, q + ((size_t)b * Hq + h) * D, qw, eps, qh);
            if (window > 0) orc_rope(D, qh, P, rope_base);
            const uint16_t *K = k_cache + ((size_t)b * Hkv + g) * max_len * D;
            const uint16_t *V = v_cache + ((size_t)b * Hkv + g) * max_len * D;
            double m = sinks[h];
            for (int j = lo; j <= P; j++) {
                double s = 0.0;
                for (int d = 0; d < D; d++) s += qh[d] * orc_bf16(K[(size_t)j * D + d]);
                s /= sqrt((double)D);
                sc[j] = s;
                if (s > m) m = s;
            }
            double den = exp(sinks[h] - m);
            for (int j = lo; j <= P; j++) den += exp(sc[j] - m);
            double *o = out + ((size_t)b * Hq + h) * D;
            for (int d = 0; d < D; d++) o[d] = 0.0;
            for (int j = lo; j <= P; j++) {
                double w = exp(sc[j] - m) / den;
                for (int d = 0; d < D; d++) o[d] += w * orc_bf16(V[(size_t)j * D + d]);
            }
        }
    }
    free(qh);
    free(kh);
    free(sc);
    return rc;
}
