"""Comparison helpers shared by the GPU parity tests and the smoke check.

Routing: the GPU takes its top-k decision on fp32 logits, the oracle on fp64
logits.  Both are correct selections whenever no two logits around the cut
are closer than the fp32 rounding error of the GPU's dot products, so the GPU
set is checked for validity against the fp64 logits with a band derived from
that error bound; outside the band the sets must be identical.  Outputs are
compared with the oracle run on the GPU's own selection (teacher forcing),
which equals the oracle's own result whenever the sets match.
"""
from __future__ import annotations

import numpy as np

REL_L2_TOL = 2e-3  # layer-output tolerance on the relative L2 error per token
U32 = 2.0 ** -24


def router_band(x: np.ndarray, router_f64: np.ndarray) -> np.ndarray:
    """Per-token bound on |fp32 logit - exact logit|, doubled (two logits compared).

    The router kernel gives each lane d_model/512 units of 8 products,
    accumulated in order by FMA, then a 6-level butterfly: every product
    passes through at most n = d_model/64 + 8 roundings, so
    |err| <= n * 2^-24 * sum_k |x_k W_ek| (first order).
    """
    d = x.shape[1]
    n = d / 64 + 8
    mag = np.abs(x) @ np.abs(router_f64).T  # [T, E]
    return 2.0 * n * U32 * mag.max(axis=1) * 1.01


def check_routing(gpu_idx: np.ndarray, gpu_w: np.ndarray, logits64: np.ndarray, orc_idx: np.ndarray,
                  orc_w: np.ndarray, band: np.ndarray, w_atol: float = 2e-6):
    """Returns (n_exact, n_ambiguous).  Raises AssertionError on an invalid selection."""
    T, K = gpu_idx.shape
    E = logits64.shape[1]
    n_exact = n_amb = 0
    for t in range(T):
        sg = gpu_idx[t].tolist()
        assert len(set(sg)) == K, f"token {t}: repeated experts {sg}"
        assert all(0 <= e < E for e in sg), f"token {t}: index out of range {sg}"
        rest = np.setdiff1d(np.arange(E), sg)
        lo_sel = logits64[t, sg].min()
        hi_rest = logits64[t, rest].max() if rest.size else -np.inf
        assert lo_sel >= hi_rest - band[t], (
            f"token {t}: selection {sg} invalid: min selected {lo_sel} < max unselected {hi_rest} - {band[t]}")
        srt = np.sort(logits64[t])[::-1]
        gap = srt[K - 1] - srt[K] if E > K else np.inf
        if gap > band[t]:
            assert sorted(sg) == sorted(orc_idx[t].tolist()), f"token {t}: {sg} vs oracle {orc_idx[t]}"
            if gpu_w is not None:
                ow = dict(zip(orc_idx[t].tolist(), orc_w[t].tolist()))
                for e, wv in zip(sg, gpu_w[t].tolist()):
                    assert abs(wv - ow[e]) <= w_atol, f"token {t} expert {e}: w {wv} vs {ow[e]}"
            n_exact += 1
        else:
            n_amb += 1
        if gpu_w is not None:
            assert abs(float(np.sum(gpu_w[t])) - 1.0) < 1e-5
    return n_exact, n_amb


def rel_l2(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-row relative L2 error of a against reference b."""
    a = np.asarray(a, dtype=np.float64).reshape(len(b), -1)
    b = np.asarray(b, dtype=np.float64).reshape(len(b), -1)
    return np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-300)


def router_band_mfma(x: np.ndarray, router_f64: np.ndarray, f32_input: bool) -> np.ndarray:
    """Per-token bound on |GPU logit - exact logit| for the matrix-core router, doubled.

    Products of bf16 operands are exact in fp32.  Each MFMA instruction adds
    16 products into the fp32 accumulator; over d_model/16 instructions a
    product passes through at most n = d_model/16 + 16 roundings.  An fp32
    input is split x = hi + lo into two bf16 parts (residual <= 2^-18 |x|)
    and both halves are accumulated, doubling n."""
    d = x.shape[1]
    n = d / 16 + 16
    rel = 2 * n * U32 + 2.0 ** -18 if f32_input else n * U32
    mag = np.abs(x) @ np.abs(router_f64).T
    return 2.0 * rel * mag.max(axis=1) * 1.01


def decode_band(x: np.ndarray, router_f64: np.ndarray) -> np.ndarray:
    """Band for a decode call (1 to 8 tokens): every decode path computes the
    router as an fp32 GEMV, lane-sequential partial sums then a wave butterfly."""
    return router_band(x, router_f64)


def lm_head_band(x: np.ndarray, w_dec: np.ndarray, block: int = 32) -> np.ndarray:
    """Bound on |fp32 logit - exact logit| for the output-layer kernel, [T, V].

    A lane multiplies its columns' decoded weights into fp32 sums (at most
    32 terms per unit of a 4-bit format, in order), scales and adds the unit
    sums, and the wave adds its 64 lane sums in 6 levels: every product
    passes through fewer than n = 48 roundings.  For q4_1 a unit's sum is
    d * sum(q x) + m * sum(x), whose terms are bounded by |w| + 2 max|w| of
    the block (m is itself a decoded value of the block, the one with
    q = 0), so the bound uses that magnitude for every format."""
    V, D = w_dec.shape
    a = np.abs(w_dec)
    bmax = a.reshape(V, D // block, block).max(axis=2)
    mag = a + 2.0 * np.repeat(bmax, block, axis=1)
    n = 48
    return 2.0 * n * U32 * (np.abs(x) @ mag.T)


def check_chain_divergence(orc, layer, x_gpu_in: np.ndarray, x_orc_in: np.ndarray, band: float, top_k: int):
    """At the first layer where a free-running oracle chain (fp64 from x_0) and
    the GPU chain (fp32) select different experts, the difference must come
    from the drift between their inputs to that layer: the oracle's own gap
    between its k-th and (k+1)-th logit must lie within twice the largest
    logit change that the drift causes, plus the fp32 band.  Returns
    (gap, logit drift)."""
    lg = orc.router_logits(layer, x_gpu_in)[0]
    lo = orc.router_logits(layer, x_orc_in)[0]
    drift = float(np.abs(lg - lo).max())
    srt = np.sort(lo)[::-1]
    gap = float(srt[top_k - 1] - srt[top_k])
    assert gap <= 2.0 * drift + band, f"selection differs at a gap {gap} the input drift {drift} does not explain"
    return gap, drift
