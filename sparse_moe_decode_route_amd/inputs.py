"""Seeded synthetic inputs for the sparse MoE decode layer.

This module is shared by the HIP path and by the CPU checker.  It draws
weights and hidden states and encodes the weights into the canonical 4-bit
block formats.  It computes none of the layer itself: no router product, no
softmax, no top-k, no decoding of blocks, no expert projection.

Workload recipe (the pages print no layer values, so every input is synthetic):

* expert and router weights ~ N(0, 0.02), hidden states ~ N(0, 1);
* router weights are stored as bf16 [n_routed, d_model] (nn.Linear order);
* expert e (0 <= e < n_routed routed, then the shared expert(s)) holds three
  matrices in the order gate [d_ff, d_model], up [d_ff, d_model],
  down [d_model, d_ff]; quantisation blocks run along the input dimension;
* the output layer (lm_head) W [vocab, d_model] ~ N(0, 0.02), encoded in the
  same block formats as the experts (blocks along d_model); its input is a
  final-normed hidden state ~ N(0, 1);
* decode attention: raw q, new k and v ~ N(0, 1); QK-norm gains 1 + 0.1 N(0, 1);
  sink logits ~ N(0, 1); cached keys and values bf16(N(0, 1)) (a stored key is a
  normalised vector, unit RMS);
* a skewed router prior (prefill workload) adds bias_e = ln(Zipf(s) pmf at the
  expert's rank), ranks given by a seeded permutation.

Canonical byte layouts (what the generator writes and what both sides read):

* bf16:   row-major uint16.
* q4_1:   per matrix, rows x (K/32) blocks of 20 bytes
          {fp16 d, fp16 m, u8 qs[16]}; element j of a block sits in the low
          nibble of qs[j], element j+16 in the high nibble; value = d*q + m.
* NVFP4:  per matrix, nibbles [rows, K/2] (element 2i in the low nibble of
          byte i, 2i+1 in the high nibble), then E4M3 block scales
          [rows, K/16]; one fp32 tensor scale per (expert, matrix) held in a
          separate array; value = e2m1(q) * e4m3(s_b) * s_t.

Random streams: numpy PCG64 seeded with SeedSequence([0xF1147, cfg_id, layer,
tensor_id]); tensor_id 0 = router, 1 + 3*e + m = expert e matrix m,
9997 = output layer, 9998 = Zipf permutation, 9999 + draw = hidden states.  A device-side variant
(``device="cuda"``) draws the same shapes with torch's Philox generator seeded
from the same SeedSequence, for workloads too large to draw on the host; its
values differ from the host stream but follow the same recipe.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

WFMT_CODES = {"bf16": 0, "q4_1": 1, "nvfp4": 2}
ROOT_SEED = 0xF1147
TID_ROUTER = 0
TID_ATTN = 9000
TID_LM_HEAD = 9997
TID_ZIPF = 9998
TID_HIDDEN = 9999


@dataclasses.dataclass(frozen=True)
class LayerDims:
    d_model: int
    d_ff: int
    n_routed: int = 256
    n_shared: int = 1
    top_k: int = 6
    wfmt: str = "q4_1"

    @property
    def n_experts(self) -> int:
        return self.n_routed + self.n_shared

    @property
    def wfmt_code(self) -> int:
        return WFMT_CODES[self.wfmt]

    def matrix_shapes(self):
        """(rows, K) of gate, up, down."""
        return [(self.d_ff, self.d_model), (self.d_ff, self.d_model), (self.d_model, self.d_ff)]


def matrix_bytes(rows: int, k: int, wfmt: str) -> int:
    if wfmt == "bf16":
        return rows * k * 2
    if wfmt == "q4_1":
        assert k % 32 == 0
        return rows * (k // 32) * 20
    if wfmt == "nvfp4":
        assert k % 16 == 0
        return rows * (k // 2) + rows * (k // 16)
    raise ValueError(wfmt)


def expert_bytes(dims: LayerDims) -> int:
    return sum(matrix_bytes(r, k, dims.wfmt) for r, k in dims.matrix_shapes())


def matrix_offsets(dims: LayerDims):
    offs, o = [], 0
    for r, k in dims.matrix_shapes():
        offs.append(o)
        o += matrix_bytes(r, k, dims.wfmt)
    return offs


@dataclasses.dataclass
class Layer:
    dims: LayerDims
    router: torch.Tensor                  # uint16-as-int16 bits of bf16 [E, d]
    router_bias: Optional[torch.Tensor]   # fp32 [E] or None
    experts: torch.Tensor                 # uint8 canonical blocks [n_experts * expert_bytes]
    tensor_scale: Optional[torch.Tensor]  # fp32 [n_experts * 3] (NVFP4) or None


def _rng(cfg_id: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, cfg_id, layer, tensor_id])))


def _torch_seed(cfg_id: int, layer: int, tensor_id: int) -> int:
    ss = np.random.SeedSequence([ROOT_SEED, cfg_id, layer, tensor_id])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF)


def _normal(shape, std, cfg_id, layer, tensor_id, device) -> torch.Tensor:
    if device is None or str(device) == "cpu":
        a = _rng(cfg_id, layer, tensor_id).standard_normal(size=shape, dtype=np.float32)
        t = torch.from_numpy(a)
    else:
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(cfg_id, layer, tensor_id))
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t * std if std != 1.0 else t


# ---------------------------------------------------------------------------
# encoders (inverse direction of the formats; data preparation only)
# ---------------------------------------------------------------------------

def bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 bit patterns (round to nearest even), as int16 tensor."""
    return x.to(torch.float32).to(torch.bfloat16).view(torch.int16)


def encode_q4_1(w: torch.Tensor) -> torch.Tensor:
    """fp32 [rows, K] -> canonical q4_1 bytes [rows, K/32*20] (uint8).

    Block of 32: m = fp16(min), d = fp16((max - min) / 15),
    q = clamp(round_half_even((x - m) / d), 0, 15); q = 0 where d == 0.
    """
    rows, k = w.shape
    b = w.reshape(rows, k // 32, 32).to(torch.float32)
    mn = b.amin(dim=2)
    mx = b.amax(dim=2)
    d16 = ((mx - mn) / 15.0).to(torch.float16)
    m16 = mn.to(torch.float16)
    d = d16.to(torch.float32).unsqueeze(2)
    m = m16.to(torch.float32).unsqueeze(2)
    safe_d = torch.where(d == 0, torch.ones_like(d), d)
    q = torch.round((b - m) / safe_d).clamp_(0, 15)
    q = torch.where(d == 0, torch.zeros_like(q), q).to(torch.uint8)
    qs = q[:, :, :16] | (q[:, :, 16:] << 4)                       # [rows, nb, 16]
    dm = torch.stack([d16.view(torch.int16), m16.view(torch.int16)], dim=2)  # [rows, nb, 2]
    dm_bytes = dm.contiguous().view(torch.uint8).reshape(rows, k // 32, 4)
    blk = torch.cat([dm_bytes, qs], dim=2)                         # [rows, nb, 20]
    return blk.reshape(rows, (k // 32) * 20).contiguous()


_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_ODD_LOWER = (False, True, False, True, False, True, False)


def _e2m1_code(v: torch.Tensor) -> torch.Tensor:
    """fp32 -> E2M1 code (sign bit 3), round to nearest, ties to even code, saturating at 6."""
    a = v.abs()
    code = torch.zeros_like(a, dtype=torch.int32)
    for mid, odd in zip(_E2M1_MIDS, _E2M1_ODD_LOWER):
        code += (a > mid).to(torch.int32)
        if odd:
            code += (a == mid).to(torch.int32)
    sign = ((v < 0) & (code > 0)).to(torch.int32) << 3
    return (code | sign).to(torch.uint8)


def encode_nvfp4(w: torch.Tensor):
    """fp32 [rows, K] -> (canonical bytes [rows*K/2 + rows*K/16] uint8, s_t fp32 scalar tensor).

    s_t = amax / (6 * 448); s_b = e4m3(amax_b / (6 * s_t)) with round to
    nearest even; q = e2m1(x / (s_b * s_t)).
    """
    rows, k = w.shape
    w = w.to(torch.float32)
    amax = w.abs().amax()
    s_t = (amax / (6.0 * 448.0)).reshape(1)
    if float(s_t) == 0.0:
        s_t = torch.ones_like(s_t)
    b = w.reshape(rows, k // 16, 16)
    amax_b = b.abs().amax(dim=2)
    sb_val = torch.clamp(amax_b / (6.0 * s_t), max=448.0)
    sb8 = sb_val.to(torch.float8_e4m3fn)
    sb = sb8.to(torch.float32).unsqueeze(2) * s_t
    safe = torch.where(sb == 0, torch.ones_like(sb), sb)
    q = _e2m1_code(b / safe)
    q = torch.where(sb == 0, torch.zeros_like(q), q)
    q = q.reshape(rows, k)
    nib = (q[:, 0::2] | (q[:, 1::2] << 4)).contiguous()            # [rows, K/2]
    scales = sb8.view(torch.uint8).contiguous()                     # [rows, K/16]
    return torch.cat([nib.reshape(-1), scales.reshape(-1)]), s_t.to(torch.float32)


def encode_matrix(w: torch.Tensor, wfmt: str):
    if wfmt == "bf16":
        return bf16_bits(w).contiguous().view(torch.uint8).reshape(-1), None
    if wfmt == "q4_1":
        return encode_q4_1(w).reshape(-1), None
    if wfmt == "nvfp4":
        return encode_nvfp4(w)
    raise ValueError(wfmt)


# ---------------------------------------------------------------------------
# layers and hidden states
# ---------------------------------------------------------------------------

def zipf_bias(n_routed: int, s: float, cfg_id: int, layer: int) -> torch.Tensor:
    """bias_e = ln(r_e^-s / H_s), ranks r_e = perm(e) + 1 from a seeded permutation."""
    perm = _rng(cfg_id, layer, TID_ZIPF).permutation(n_routed)
    ranks = perm.astype(np.float64) + 1.0
    h = np.sum(np.arange(1, n_routed + 1, dtype=np.float64) ** (-s))
    return torch.from_numpy((-s * np.log(ranks) - np.log(h)).astype(np.float32))


def make_expert(dims: LayerDims, cfg_id: int, layer: int, e: int, device=None):
    """Canonical bytes of expert e and its three tensor scales (NVFP4) or None."""
    parts, scales = [], []
    for m, (rows, k) in enumerate(dims.matrix_shapes()):
        w = _normal((rows, k), 0.02, cfg_id, layer, 1 + 3 * e + m, device)
        blob, s_t = encode_matrix(w, dims.wfmt)
        parts.append(blob)
        if s_t is not None:
            scales.append(s_t)
    return torch.cat(parts), (torch.cat(scales) if scales else None)


def make_layer(dims: LayerDims, cfg_id: int, layer: int = 0, zipf_s: Optional[float] = None,
               device=None, router_zero: bool = False) -> Layer:
    if router_zero:
        router = torch.zeros((dims.n_routed, dims.d_model), dtype=torch.int16, device=device)
    else:
        router = bf16_bits(_normal((dims.n_routed, dims.d_model), 0.02, cfg_id, layer, TID_ROUTER, device))
    bias = None
    if zipf_s is not None:
        bias = zipf_bias(dims.n_routed, zipf_s, cfg_id, layer)
        if device is not None:
            bias = bias.to(device)
    eb = expert_bytes(dims)
    experts = torch.empty(dims.n_experts * eb, dtype=torch.uint8, device=device)
    tscale = torch.empty(dims.n_experts * 3, dtype=torch.float32, device=device) if dims.wfmt == "nvfp4" else None
    for e in range(dims.n_experts):
        blob, s = make_expert(dims, cfg_id, layer, e, device)
        experts[e * eb:(e + 1) * eb] = blob
        if tscale is not None:
            tscale[3 * e:3 * e + 3] = s
    return Layer(dims, router.contiguous(), bias, experts, tscale)


def make_lm_head(vocab: int, d_model: int, wfmt: str, cfg_id: int, device=None):
    """Canonical bytes of the output layer [vocab, d_model] and its tensor scale
    (fp32 [1], NVFP4) or None.  Drawn in slabs of rows so that a full
    vocabulary does not hold a second fp32 copy of the matrix."""
    w = _normal((vocab, d_model), 0.02, cfg_id, 0, TID_LM_HEAD, device)
    if wfmt == "nvfp4":
        return encode_nvfp4(w)
    slab = 16384
    parts = [encode_matrix(w[r:r + slab], wfmt)[0] for r in range(0, vocab, slab)]
    return torch.cat(parts), None


@dataclasses.dataclass
class AttnInputs:
    q: torch.Tensor        # fp32 [B, Hq, D]
    k_new: torch.Tensor    # fp32 [B, Hkv, D]
    v_new: torch.Tensor    # fp32 [B, Hkv, D]
    q_norm_w: torch.Tensor  # fp32 [D]
    k_norm_w: torch.Tensor  # fp32 [D]
    sinks: torch.Tensor    # fp32 [Hq]
    k_cache: torch.Tensor  # bf16 bits int16 [B, Hkv, max_len, D]
    v_cache: torch.Tensor  # bf16 bits int16 [B, Hkv, max_len, D]


def make_attn(B: int, Hq: int, Hkv: int, D: int, max_len: int, cfg_id: int, draw: int = 0,
              device=None) -> AttnInputs:
    """Inputs of one decode-attention step (seeded; tensor ids 9000 + 8 * draw + i)."""
    t = TID_ATTN + 8 * draw
    return AttnInputs(
        q=_normal((B, Hq, D), 1.0, cfg_id, 0, t, device).contiguous(),
        k_new=_normal((B, Hkv, D), 1.0, cfg_id, 0, t + 1, device).contiguous(),
        v_new=_normal((B, Hkv, D), 1.0, cfg_id, 0, t + 2, device).contiguous(),
        q_norm_w=(1.0 + _normal((D,), 0.1, cfg_id, 0, t + 3, device)).contiguous(),
        k_norm_w=(1.0 + _normal((D,), 0.1, cfg_id, 0, t + 4, device)).contiguous(),
        sinks=_normal((Hq,), 1.0, cfg_id, 0, t + 5, device).contiguous(),
        k_cache=bf16_bits(_normal((B, Hkv, max_len, D), 1.0, cfg_id, 0, t + 6, device)).contiguous(),
        v_cache=bf16_bits(_normal((B, Hkv, max_len, D), 1.0, cfg_id, 0, t + 7, device)).contiguous())


def make_hidden(cfg_id: int, n_tokens: int, d_model: int, layer: int = 0, draw: int = 0,
                device=None) -> torch.Tensor:
    """Hidden states ~ N(0, 1), fp32 [n_tokens, d_model]."""
    return _normal((n_tokens, d_model), 1.0, cfg_id, layer, TID_HIDDEN + draw, device).contiguous()


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 hidden states to bf16 (activations of the prefill workload)."""
    return x.to(torch.bfloat16)


# Named workloads: (dims, tokens, extra).  Sizes as the layer is specified.
WORKLOADS = {
    # one CPU-sized layer: d 512, d_ff 128, bf16 weights, 4 tokens
    "c1_small_bf16": dict(cfg_id=1, dims=LayerDims(512, 128, wfmt="bf16"), tokens=4),
    # one full-size layer, q4_1, batch-1 decode
    "c2_layer_q4_1": dict(cfg_id=2, dims=LayerDims(2048, 512, wfmt="q4_1"), tokens=1),
    # 47 independent full-size q4_1 layers, one token, RMS-normalised between layers
    "c3_stack47_q4_1": dict(cfg_id=3, dims=LayerDims(2048, 512, wfmt="q4_1"), tokens=1, layers=47),
    # one full-size layer, NVFP4, batch 1 and batch 8
    "c4_layer_nvfp4": dict(cfg_id=4, dims=LayerDims(2048, 512, wfmt="nvfp4"), tokens=8),
    # prefill: 4096 bf16 tokens, Zipf(1.1) router prior, q4_1
    "c5_prefill_q4_1": dict(cfg_id=5, dims=LayerDims(2048, 512, wfmt="q4_1"), tokens=4096, zipf_s=1.1),
}

# Output layer at decode: the vocabulary is not on the pages; 0.3 B output
# parameters over d_model 2048 gives 146,484 rows (a reading, not a figure
# from the pages).  Not a multiple of any tile, so the last rows are ragged.
LM_HEAD_VOCAB = 146_484
LM_HEAD_CFG = 6

# Decode attention: 32 query heads over 4 key/value heads of 128; sliding
# window of 513 positions (rotary embeddings) or full attention (none).
ATTN_HQ, ATTN_HKV, ATTN_D, ATTN_WINDOW = 32, 4, 128, 513
ATTN_ROPE_BASE = 10000.0  # not on the pages (a reading)
ATTN_CFG = 7
