"""CPU oracle for the sparse MoE decode layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``moe_oracle.c`` (plain loops, fp64) through
ctypes and shares no code with the HIP library; the only thing both sides
share is the seeded input generator.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_SO = os.path.join(_HERE, "libmoe_oracle.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC"]

_lib = None


class OrcDims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_routed", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("top_k", ctypes.c_int32), ("wfmt", ctypes.c_int32)]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (building the checker is not using it)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_SO)
        for name in ("orc_fp16", "orc_bf16"):
            getattr(L, name).restype = ctypes.c_double
            getattr(L, name).argtypes = [ctypes.c_uint16]
        for name in ("orc_e4m3", "orc_e2m1"):
            getattr(L, name).restype = ctypes.c_double
            getattr(L, name).argtypes = [ctypes.c_uint8]
        L.orc_expert_bytes.restype = ctypes.c_size_t
        L.orc_expert_bytes.argtypes = [ctypes.POINTER(OrcDims)]
        L.orc_layer_forward.restype = ctypes.c_int
        L.orc_stack_forward.restype = ctypes.c_int
        L.orc_lm_head.restype = ctypes.c_int
        L.orc_attn_decode.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def dims_struct(dims) -> OrcDims:
    return OrcDims(dims.d_model, dims.d_ff, dims.n_routed, dims.n_shared, dims.top_k, dims.wfmt_code)


# --------------------------------------------------------------------------- scalar decoders

def fp16(bits: int) -> float:
    return lib().orc_fp16(bits)


def bf16(bits: int) -> float:
    return lib().orc_bf16(bits)


def e4m3(code: int) -> float:
    return lib().orc_e4m3(code)


def e2m1(code: int) -> float:
    return lib().orc_e2m1(code)


def bf16_array(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp64 through the oracle's decoder."""
    flat = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    table = np.array([lib().orc_bf16(i) for i in range(65536)], dtype=np.float64)
    return table[flat].reshape(np.shape(bits))


def dequant_q4_1_block(block: bytes) -> np.ndarray:
    buf = np.frombuffer(bytes(block), dtype=np.uint8).copy()
    out = np.zeros(32, dtype=np.float64)
    lib().orc_dequant_q4_1_block(_p(buf, ctypes.c_uint8), _p(out, ctypes.c_double))
    return out


def dequant_matrix(wfmt_code: int, blob: np.ndarray, rows: int, k: int, s_t: float = 1.0) -> np.ndarray:
    buf = np.ascontiguousarray(blob, dtype=np.uint8)
    out = np.zeros((rows, k), dtype=np.float64)
    lib().orc_dequant_matrix(ctypes.c_int(wfmt_code), _p(buf, ctypes.c_uint8), ctypes.c_int(rows),
                             ctypes.c_int(k), ctypes.c_double(s_t), _p(out, ctypes.c_double))
    return out


# --------------------------------------------------------------------------- routing pieces

def softmax(logits: np.ndarray) -> np.ndarray:
    l = np.ascontiguousarray(logits, dtype=np.float64)
    p = np.zeros_like(l)
    lib().orc_softmax(ctypes.c_int(l.size), _p(l, ctypes.c_double), _p(p, ctypes.c_double))
    return p


def sort_experts(logits: np.ndarray) -> np.ndarray:
    l = np.ascontiguousarray(logits, dtype=np.float64)
    order = np.zeros(l.size, dtype=np.int32)
    lib().orc_sort_experts(ctypes.c_int(l.size), _p(l, ctypes.c_double), _p(order, ctypes.c_int32))
    return order


def route(dims, logits: np.ndarray, forced: Optional[np.ndarray] = None):
    l = np.ascontiguousarray(logits, dtype=np.float64)
    d = dims_struct(dims)
    idx = np.zeros(dims.top_k, dtype=np.int32)
    w = np.zeros(dims.top_k, dtype=np.float64)
    probs = np.zeros(dims.n_routed, dtype=np.float64)
    f = None if forced is None else _p(np.ascontiguousarray(forced, dtype=np.int32), ctypes.c_int32)
    lib().orc_route(ctypes.byref(d), _p(l, ctypes.c_double), f, _p(idx, ctypes.c_int32), _p(w, ctypes.c_double),
                    _p(probs, ctypes.c_double))
    return idx, w, probs


def rmsnorm(y: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.zeros_like(y)
    lib().orc_rmsnorm(ctypes.c_int(y.size), _p(y, ctypes.c_double), ctypes.c_double(eps), _p(out, ctypes.c_double))
    return out


# --------------------------------------------------------------------------- layer / stack

def _layer_arrays(layer):
    wr = np.ascontiguousarray(layer.router.cpu().numpy().view(np.uint16))
    ex = np.ascontiguousarray(layer.experts.cpu().numpy())
    ts = None if layer.tensor_scale is None else np.ascontiguousarray(layer.tensor_scale.cpu().numpy(), dtype=np.float32)
    bias = None if layer.router_bias is None else np.ascontiguousarray(layer.router_bias.cpu().numpy(), dtype=np.float64)
    return wr, ex, ts, bias


def router_logits(layer, x: np.ndarray) -> np.ndarray:
    """Router logits only, [T, E] fp64 (x W_r^T + bias), token by token."""
    dims = layer.dims
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(-1, dims.d_model)
    wr, _, _, bias = _layer_arrays(layer)
    out = np.zeros((x.shape[0], dims.n_routed), dtype=np.float64)
    d = dims_struct(dims)
    bp = None if bias is None else _p(bias, ctypes.c_double)
    for t in range(x.shape[0]):
        lib().orc_router_logits(ctypes.byref(d), _p(x[t], ctypes.c_double), _p(wr, ctypes.c_uint16), bp,
                                _p(out[t], ctypes.c_double))
    return out


def layer_forward(layer, x: np.ndarray, forced: Optional[np.ndarray] = None, dense: bool = False):
    """Returns (idx [T,k] int32, w [T,k] f64, logits [T,E] f64, y [T,d] f64)."""
    dims = layer.dims
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(-1, dims.d_model)
    T = x.shape[0]
    wr, ex, ts, bias = _layer_arrays(layer)
    idx = np.zeros((T, dims.top_k), dtype=np.int32)
    w = np.zeros((T, dims.top_k), dtype=np.float64)
    logits = np.zeros((T, dims.n_routed), dtype=np.float64)
    y = np.zeros((T, dims.d_model), dtype=np.float64)
    fz = None
    if forced is not None:
        fz = np.ascontiguousarray(forced, dtype=np.int32).reshape(T, dims.top_k)
    d = dims_struct(dims)
    rc = lib().orc_layer_forward(
        ctypes.byref(d), ctypes.c_int32(T), _p(x, ctypes.c_double), _p(wr, ctypes.c_uint16),
        None if bias is None else _p(bias, ctypes.c_double), _p(ex, ctypes.c_uint8),
        None if ts is None else _p(ts, ctypes.c_float), None if fz is None else _p(fz, ctypes.c_int32),
        ctypes.c_int32(1 if dense else 0), _p(idx, ctypes.c_int32), _p(w, ctypes.c_double),
        _p(logits, ctypes.c_double), _p(y, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle rejected dims {dims}")
    return idx, w, logits, y


def experts_given(layer, x: np.ndarray, idx: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = shared experts + sum_i w[t, i] * expert_{idx[t, i]}(x_t), in fp64."""
    dims = layer.dims
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(-1, dims.d_model)
    T = x.shape[0]
    _, ex, ts, _ = _layer_arrays(layer)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(T, dims.top_k)
    w = np.ascontiguousarray(w, dtype=np.float64).reshape(T, dims.top_k)
    y = np.zeros((T, dims.d_model), dtype=np.float64)
    d = dims_struct(dims)
    lib().orc_experts_given(ctypes.byref(d), ctypes.c_int32(T), _p(x, ctypes.c_double), _p(ex, ctypes.c_uint8),
                            None if ts is None else _p(ts, ctypes.c_float), _p(idx, ctypes.c_int32),
                            _p(w, ctypes.c_double), _p(y, ctypes.c_double))
    return y


def stack_forward(layers: Sequence, x0: np.ndarray):
    """Returns (y_last [T,d], y_trace [L,T,d], idx_trace [L,T,k])."""
    dims = layers[0].dims
    x0 = np.ascontiguousarray(x0, dtype=np.float64).reshape(-1, dims.d_model)
    T, L = x0.shape[0], len(layers)
    arrs = [_layer_arrays(l) for l in layers]
    wr_ptrs = (ctypes.POINTER(ctypes.c_uint16) * L)(*[_p(a[0], ctypes.c_uint16) for a in arrs])
    ex_ptrs = (ctypes.POINTER(ctypes.c_uint8) * L)(*[_p(a[1], ctypes.c_uint8) for a in arrs])
    ts_ptrs = None
    if arrs[0][2] is not None:
        ts_ptrs = (ctypes.POINTER(ctypes.c_float) * L)(*[_p(a[2], ctypes.c_float) for a in arrs])
    y = np.zeros((T, dims.d_model), dtype=np.float64)
    y_trace = np.zeros((L, T, dims.d_model), dtype=np.float64)
    idx_trace = np.zeros((L, T, dims.top_k), dtype=np.int32)
    d = dims_struct(dims)
    rc = lib().orc_stack_forward(ctypes.byref(d), ctypes.c_int32(L), ctypes.c_int32(T), _p(x0, ctypes.c_double),
                                 wr_ptrs, ex_ptrs, ts_ptrs, _p(y, ctypes.c_double), _p(y_trace, ctypes.c_double),
                                 _p(idx_trace, ctypes.c_int32))
    if rc != 0:
        raise ValueError("oracle rejected the stack")
    return y, y_trace, idx_trace


# --------------------------------------------------------------------------- output layer

def lm_head(wfmt_code: int, blob: np.ndarray, vocab: int, d: int, x: np.ndarray, s_t: float = 1.0,
            rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Output-layer logits [T, n_rows] in fp64: x W^T over the listed rows of
    the canonical [vocab, d] matrix (every row when rows is None)."""
    buf = np.ascontiguousarray(blob, dtype=np.uint8).reshape(-1)
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(-1, d)
    T = x.shape[0]
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32).reshape(-1)
    n = vocab if r is None else r.size
    out = np.zeros((T, n), dtype=np.float64)
    rc = lib().orc_lm_head(ctypes.c_int(wfmt_code), _p(buf, ctypes.c_uint8), ctypes.c_int32(vocab),
                           ctypes.c_int32(d), ctypes.c_double(s_t), ctypes.c_int32(T), _p(x, ctypes.c_double),
                           None if r is None else _p(r, ctypes.c_int32), ctypes.c_int32(n),
                           _p(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle: row index outside the vocabulary")
    return out


# --------------------------------------------------------------------------- decode attention

def attn_decode(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, qw: np.ndarray, kw: np.ndarray,
                sinks: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos: np.ndarray, window: int,
                rope_base: float = 10000.0, eps: float = 1e-6):
    """One decode step of attention.  q [B, Hq, D], k_new / v_new [B, Hkv, D],
    caches bf16 bits uint16 [B, Hkv, max_len, D] (copied, not modified), pos
    [B].  Returns (out [B, Hq, D] fp64, k_cache, v_cache with the new entries)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    k_new = np.ascontiguousarray(k_new, dtype=np.float64)
    Hkv = k_new.shape[1]
    v_new = np.ascontiguousarray(v_new, dtype=np.float64)
    qw = np.ascontiguousarray(qw, dtype=np.float64)
    kw = np.ascontiguousarray(kw, dtype=np.float64)
    sinks = np.ascontiguousarray(sinks, dtype=np.float64)
    kc = np.array(k_cache, dtype=np.uint16, copy=True, order="C")
    vc = np.array(v_cache, dtype=np.uint16, copy=True, order="C")
    max_len = kc.shape[2]
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    rc = lib().orc_attn_decode(
        ctypes.c_int(Hq), ctypes.c_int(Hkv), ctypes.c_int(D), ctypes.c_int(window), ctypes.c_double(rope_base),
        ctypes.c_double(eps), ctypes.c_int(B), _p(q, ctypes.c_double), _p(k_new, ctypes.c_double),
        _p(v_new, ctypes.c_double), _p(qw, ctypes.c_double), _p(kw, ctypes.c_double), _p(sinks, ctypes.c_double),
        _p(kc, ctypes.c_uint16), _p(vc, ctypes.c_uint16), ctypes.c_int(max_len), _p(pos, ctypes.c_int32),
        _p(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle: position outside the cache")
    return out, kc, vc
