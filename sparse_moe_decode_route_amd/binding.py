"""Thin Python binding over libmoe's C ABI (argument marshalling only).

Every step of the layer runs in libmoe's HIP kernels; torch provides device
memory and the current HIP stream.  If libmoe.so is missing the import of any
entry point raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

from . import inputs as gen

_HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
ACT_F32, ACT_BF16 = 0, 1
ENTRY_POINTS = (
    "moe_packed_expert_bytes", "moe_workspace_size", "moe_repack_weights", "moe_route_topk",
    "moe_expert_ffn_q4", "moe_layer_forward", "moe_layer_forward_noalloc", "moe_layer_forward_prefill",
    "moe_stack_decode",
    "moe_stack_decode_timed", "moe_layer_forward_prefill_timed", "moe_lm_head_bytes", "moe_lm_head_repack",
    "moe_lm_head", "moe_lm_head_timed", "moe_attn_workspace_size", "moe_attn_chunk_plan", "moe_attn_decode", "moe_attn_decode_timed",
    "moe_set_decode_path", "moe_decode_check", "moe_status_string", "moe_last_error",
)

PATH_KERNELS, PATH_PERSISTENT, PATH_XCD = 0, 1, 2


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmoe status {status}: {msg}")
        self.status = status


class CAttnDims(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float)]


class CDims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_routed", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("top_k", ctypes.c_int32), ("wfmt", ctypes.c_int32)]


class CLayerWeights(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("experts", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(SO_PATH):
            raise RuntimeError(f"libmoe.so not built at {SO_PATH}; run sparse_moe_decode_route_amd/build.py")
        L = ctypes.CDLL(SO_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        pd = ctypes.POINTER(CDims)
        L.moe_packed_expert_bytes.restype = sz
        L.moe_packed_expert_bytes.argtypes = [pd]
        L.moe_workspace_size.restype = ctypes.c_int
        L.moe_workspace_size.argtypes = [pd, i32, ctypes.POINTER(sz)]
        L.moe_repack_weights.restype = ctypes.c_int
        L.moe_repack_weights.argtypes = [pd, vp, vp, i32, vp]
        L.moe_route_topk.restype = ctypes.c_int
        L.moe_route_topk.argtypes = [pd, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_expert_ffn_q4.restype = ctypes.c_int
        L.moe_expert_ffn_q4.argtypes = [pd, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_layer_forward.restype = ctypes.c_int
        L.moe_layer_forward.argtypes = [pd, ctypes.POINTER(CLayerWeights), vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.moe_layer_forward_prefill.restype = ctypes.c_int
        L.moe_layer_forward_prefill.argtypes = L.moe_layer_forward.argtypes
        L.moe_layer_forward_noalloc.restype = ctypes.c_int
        L.moe_layer_forward_noalloc.argtypes = [pd, ctypes.POINTER(CLayerWeights), vp, i32, i32, vp, vp, vp, vp]
        L.moe_stack_decode.restype = ctypes.c_int
        L.moe_stack_decode.argtypes = [pd, i32, ctypes.POINTER(CLayerWeights), vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_stack_decode_timed.restype = ctypes.c_int
        L.moe_stack_decode_timed.argtypes = [pd, i32, ctypes.POINTER(CLayerWeights), vp, i32, vp, vp, vp, sz,
                                             ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32), ctypes.c_char_p,
                                             sz, vp]
        L.moe_layer_forward_prefill_timed.restype = ctypes.c_int
        L.moe_layer_forward_prefill_timed.argtypes = [pd, ctypes.POINTER(CLayerWeights), vp, i32, i32, vp, vp, sz,
                                                      ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32),
                                                      ctypes.c_char_p, sz, vp]
        L.moe_lm_head_bytes.restype = sz
        L.moe_lm_head_bytes.argtypes = [i32, i32, i32]
        L.moe_lm_head_repack.restype = ctypes.c_int
        L.moe_lm_head_repack.argtypes = [i32, i32, i32, vp, vp, vp]
        L.moe_lm_head.restype = ctypes.c_int
        L.moe_lm_head.argtypes = [i32, i32, i32, vp, vp, vp, i32, i32, vp, vp]
        L.moe_lm_head_timed.restype = ctypes.c_int
        L.moe_lm_head_timed.argtypes = [i32, i32, i32, vp, vp, vp, i32, i32, vp, ctypes.POINTER(ctypes.c_float), vp]
        pa = ctypes.POINTER(CAttnDims)
        L.moe_attn_workspace_size.restype = ctypes.c_int
        L.moe_attn_workspace_size.argtypes = [pa, i32, i32, ctypes.POINTER(sz)]
        L.moe_attn_chunk_plan.restype = ctypes.c_int
        L.moe_attn_chunk_plan.argtypes = [pa, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.moe_attn_decode.restype = ctypes.c_int
        L.moe_attn_decode.argtypes = [pa, i32, i32] + [vp] * 11 + [sz, vp]
        L.moe_attn_decode_timed.restype = ctypes.c_int
        L.moe_attn_decode_timed.argtypes = [pa, i32, i32] + [vp] * 11 + [sz, ctypes.POINTER(ctypes.c_float), vp]
        L.moe_set_decode_path.restype = ctypes.c_int
        L.moe_set_decode_path.argtypes = [i32]
        L.moe_decode_check.restype = ctypes.c_int
        L.moe_decode_check.argtypes = [pd, i32, vp, sz, vp]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status: int):
    if status != MOE_OK:
        L = lib()
        raise MoeError(status, f"{L.moe_status_string(status).decode()}: {L.moe_last_error().decode()}")


def cdims(dims: gen.LayerDims) -> CDims:
    return CDims(dims.d_model, dims.d_ff, dims.n_routed, dims.n_shared, dims.top_k, dims.wfmt_code)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _act(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return ACT_F32
    if x.dtype == torch.bfloat16:
        return ACT_BF16
    raise TypeError(f"activations must be fp32 or bf16, got {x.dtype}")


# --------------------------------------------------------------------------- sizes / workspace

def packed_expert_bytes(dims: gen.LayerDims) -> int:
    d = cdims(dims)
    return int(lib().moe_packed_expert_bytes(ctypes.byref(d)))


def workspace_size(dims: gen.LayerDims, n_tokens: int) -> int:
    d = cdims(dims)
    out = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(d), n_tokens, ctypes.byref(out)))
    return int(out.value)


def workspace(dims: gen.LayerDims, n_tokens: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_size(dims, n_tokens), 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------- weights

@dataclasses.dataclass
class DeviceLayer:
    dims: gen.LayerDims
    router: torch.Tensor
    router_bias: Optional[torch.Tensor]
    experts: torch.Tensor          # device layout
    tensor_scale: Optional[torch.Tensor]

    def cstruct(self) -> CLayerWeights:
        return CLayerWeights(self.router.data_ptr(), 0 if self.router_bias is None else self.router_bias.data_ptr(),
                             self.experts.data_ptr(), 0 if self.tensor_scale is None else self.tensor_scale.data_ptr())


def repack_weights(dims: gen.LayerDims, canonical: torch.Tensor, packed: torch.Tensor, n_experts: int, stream=None):
    d = cdims(dims)
    _check(lib().moe_repack_weights(ctypes.byref(d), _ptr(canonical), _ptr(packed), n_experts, _stream(stream)))


def upload_layer(layer: gen.Layer, device="cuda") -> DeviceLayer:
    """Copy a generated layer to the device and repack its experts."""
    dims = layer.dims
    canon = layer.experts.to(device)
    packed = torch.empty_like(canon)
    repack_weights(dims, canon, packed, dims.n_experts)
    torch.cuda.current_stream().synchronize()
    del canon
    return DeviceLayer(dims, layer.router.to(device).contiguous(),
                       None if layer.router_bias is None else layer.router_bias.to(device).contiguous(), packed,
                       None if layer.tensor_scale is None else layer.tensor_scale.to(device).contiguous())


# --------------------------------------------------------------------------- entry points

def route_topk(dims: gen.LayerDims, x: torch.Tensor, router: torch.Tensor, router_bias: Optional[torch.Tensor] = None,
               want_logits: bool = True, ws: Optional[torch.Tensor] = None, stream=None):
    T = x.shape[0]
    dev = x.device
    idx = torch.empty((T, dims.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, dims.top_k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, dims.n_routed), dtype=torch.float32, device=dev) if want_logits else None
    ws = ws if ws is not None else workspace(dims, T, dev)
    d = cdims(dims)
    _check(lib().moe_route_topk(ctypes.byref(d), _ptr(x), _act(x), T, _ptr(router), _ptr(router_bias), _ptr(idx),
                                _ptr(w), _ptr(logits), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, w, logits


def expert_ffn_q4(dims: gen.LayerDims, x: torch.Tensor, experts: torch.Tensor, tensor_scale: Optional[torch.Tensor],
                  topk_idx: torch.Tensor, topk_w: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None):
    T = x.shape[0]
    y = torch.empty((T, dims.d_model), dtype=torch.float32, device=x.device)
    ws = ws if ws is not None else workspace(dims, T, x.device)
    d = cdims(dims)
    _check(lib().moe_expert_ffn_q4(ctypes.byref(d), _ptr(x), _act(x), T, _ptr(experts), _ptr(tensor_scale),
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
    return y


def layer_forward(layer: DeviceLayer, x: torch.Tensor, ws: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                  want_routing: bool = True, stream=None, prefill: bool = False):
    dims = layer.dims
    T = x.shape[0]
    dev = x.device
    y = y if y is not None else torch.empty((T, dims.d_model), dtype=torch.float32, device=dev)
    idx = torch.empty((T, dims.top_k), dtype=torch.int32, device=dev) if want_routing else None
    w = torch.empty((T, dims.top_k), dtype=torch.float32, device=dev) if want_routing else None
    ws = ws if ws is not None else workspace(dims, T, dev)
    d = cdims(dims)
    cw = layer.cstruct()
    fn = lib().moe_layer_forward_prefill if prefill else lib().moe_layer_forward
    _check(fn(ctypes.byref(d), ctypes.byref(cw), _ptr(x), _act(x), T, _ptr(y), _ptr(idx), _ptr(w), _ptr(ws),
              ws.numel(), _stream(stream)))
    return y, idx, w


def layer_forward_prefill(layer: DeviceLayer, x: torch.Tensor, **kw):
    return layer_forward(layer, x, prefill=True, **kw)


def layer_forward_noalloc(layer: DeviceLayer, x: torch.Tensor, y: torch.Tensor, idx: Optional[torch.Tensor] = None,
                          w: Optional[torch.Tensor] = None, stream=None):
    """moe_layer_forward_noalloc: the layer with the library's static scratch as
    workspace; the caller passes every output buffer."""
    d = cdims(layer.dims)
    cw = layer.cstruct()
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(d), ctypes.byref(cw), _ptr(x), _act(x), x.shape[0], _ptr(y),
                                           _ptr(idx), _ptr(w), _stream(stream)))
    return y, idx, w


def set_decode_path(path: int):
    """PATH_KERNELS (default: three kernels per layer), PATH_PERSISTENT (the
    persistent batch-1 kernel where built) or PATH_XCD (one kernel per layer,
    one expert per XCD, where built)."""
    _check(lib().moe_set_decode_path(path))


def decode_check(dims: gen.LayerDims, n_tokens: int, ws: torch.Tensor, stream=None):
    """Raises MoeError if the last persistent-kernel call on ws gave up a wait."""
    d = cdims(dims)
    _check(lib().moe_decode_check(ctypes.byref(d), n_tokens, _ptr(ws), ws.numel(), _stream(stream)))


class StackHandle:
    """Host array of per-layer weight structs, kept alive for repeated calls."""

    def __init__(self, layers: Sequence[DeviceLayer]):
        self.layers = list(layers)
        self.dims = layers[0].dims
        self.carr = (CLayerWeights * len(layers))(*[l.cstruct() for l in layers])


def stack_decode(stack: StackHandle, x0: torch.Tensor, ws: Optional[torch.Tensor] = None,
                 y: Optional[torch.Tensor] = None, trace: bool = False, stream=None):
    dims = stack.dims
    T = x0.shape[0]
    L = len(stack.layers)
    dev = x0.device
    y = y if y is not None else torch.empty((T, dims.d_model), dtype=torch.float32, device=dev)
    y_trace = torch.empty((L, T, dims.d_model), dtype=torch.float32, device=dev) if trace else None
    idx_trace = torch.empty((L, T, dims.top_k), dtype=torch.int32, device=dev) if trace else None
    ws = ws if ws is not None else workspace(dims, T, dev)
    d = cdims(dims)
    _check(lib().moe_stack_decode(ctypes.byref(d), L, stack.carr, _ptr(x0), T, _ptr(y), _ptr(y_trace),
                                  _ptr(idx_trace), _ptr(ws), ws.numel(), _stream(stream)))
    return y, y_trace, idx_trace


def stack_decode_timed(stack: StackHandle, x0: torch.Tensor, ws: Optional[torch.Tensor] = None,
                       y: Optional[torch.Tensor] = None, trace: bool = False, stream=None):
    """moe_stack_decode_timed: returns (y, idx_trace or None, {kernel name: mean us per launch}).

    Synchronises the stream (the call waits for its own events)."""
    dims = stack.dims
    T = x0.shape[0]
    L = len(stack.layers)
    dev = x0.device
    y = y if y is not None else torch.empty((T, dims.d_model), dtype=torch.float32, device=dev)
    idx_trace = torch.empty((L, T, dims.top_k), dtype=torch.int32, device=dev) if trace else None
    ws = ws if ws is not None else workspace(dims, T, dev)
    d = cdims(dims)
    us = (ctypes.c_float * 8)()
    nk = ctypes.c_int32(0)
    names = ctypes.create_string_buffer(256)
    _check(lib().moe_stack_decode_timed(ctypes.byref(d), L, stack.carr, _ptr(x0), T, _ptr(y), _ptr(idx_trace),
                                        _ptr(ws), ws.numel(), us, ctypes.byref(nk), names, 256, _stream(stream)))
    keys = names.value.decode().split(";")
    return y, idx_trace, {keys[k]: float(us[k]) for k in range(nk.value)}


def layer_forward_prefill_timed(layer: DeviceLayer, x: torch.Tensor, ws: Optional[torch.Tensor] = None,
                                y: Optional[torch.Tensor] = None, stream=None):
    """moe_layer_forward_prefill_timed: returns (y, {kernel name: us}).  Synchronises the stream."""
    dims = layer.dims
    T = x.shape[0]
    y = y if y is not None else torch.empty((T, dims.d_model), dtype=torch.float32, device=x.device)
    ws = ws if ws is not None else workspace(dims, T, x.device)
    d = cdims(dims)
    cw = layer.cstruct()
    us = (ctypes.c_float * 8)()
    nk = ctypes.c_int32(0)
    names = ctypes.create_string_buffer(256)
    _check(lib().moe_layer_forward_prefill_timed(ctypes.byref(d), ctypes.byref(cw), _ptr(x), _act(x), T, _ptr(y),
                                                 _ptr(ws), ws.numel(), us, ctypes.byref(nk), names, 256,
                                                 _stream(stream)))
    keys = names.value.decode().split(";")
    return y, {keys[k]: float(us[k]) for k in range(nk.value)}


# --------------------------------------------------------------------------- output layer (lm_head)

@dataclasses.dataclass
class LmHead:
    """Output-layer weights on the device: W [vocab, d_model] in the device layout."""
    vocab: int
    d_model: int
    wfmt: str
    weights: torch.Tensor                 # uint8, device layout
    tensor_scale: Optional[torch.Tensor]  # fp32 [1] (NVFP4) or None

    @property
    def wfmt_code(self) -> int:
        return gen.WFMT_CODES[self.wfmt]


def lm_head_bytes(vocab: int, d_model: int, wfmt: str) -> int:
    return int(lib().moe_lm_head_bytes(vocab, d_model, gen.WFMT_CODES[wfmt]))


def lm_head_repack(vocab: int, d_model: int, wfmt: str, canonical: torch.Tensor, packed: torch.Tensor, stream=None):
    _check(lib().moe_lm_head_repack(vocab, d_model, gen.WFMT_CODES[wfmt], _ptr(canonical), _ptr(packed),
                                    _stream(stream)))


def upload_lm_head(vocab: int, d_model: int, wfmt: str, canonical: torch.Tensor, tensor_scale: Optional[torch.Tensor],
                   device="cuda") -> LmHead:
    """Copy canonical output-layer bytes to the device and convert them to the device layout."""
    canon = canonical.to(device)
    packed = torch.empty_like(canon)
    lm_head_repack(vocab, d_model, wfmt, canon, packed)
    torch.cuda.current_stream().synchronize()
    del canon
    ts = None if tensor_scale is None else tensor_scale.to(device=device, dtype=torch.float32).reshape(1).contiguous()
    return LmHead(vocab, d_model, wfmt, packed, ts)


def lm_head(head: LmHead, x: torch.Tensor, logits: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_lm_head: fp32 logits [T, vocab] of the tokens x [T, d_model] (fp32 or bf16)."""
    T = x.shape[0]
    logits = logits if logits is not None else torch.empty((T, head.vocab), dtype=torch.float32, device=x.device)
    _check(lib().moe_lm_head(head.vocab, head.d_model, head.wfmt_code, _ptr(head.weights), _ptr(head.tensor_scale),
                             _ptr(x), _act(x), T, _ptr(logits), _stream(stream)))
    return logits


def lm_head_timed(head: LmHead, x: torch.Tensor, logits: Optional[torch.Tensor] = None, stream=None):
    """moe_lm_head_timed: (logits, kernel microseconds).  Synchronises the stream."""
    T = x.shape[0]
    logits = logits if logits is not None else torch.empty((T, head.vocab), dtype=torch.float32, device=x.device)
    us = ctypes.c_float(0.0)
    _check(lib().moe_lm_head_timed(head.vocab, head.d_model, head.wfmt_code, _ptr(head.weights),
                                   _ptr(head.tensor_scale), _ptr(x), _act(x), T, _ptr(logits), ctypes.byref(us),
                                   _stream(stream)))
    return logits, float(us.value)


# --------------------------------------------------------------------------- decode attention

def attn_dims(n_q_heads: int, n_kv_heads: int, window: int, rope_base: float = 10000.0,
              norm_eps: float = 1e-6) -> CAttnDims:
    return CAttnDims(n_q_heads, n_kv_heads, 128, window, rope_base, norm_eps)


def attn_workspace(dims: CAttnDims, n_seqs: int, max_len: int, device="cuda") -> torch.Tensor:
    n = ctypes.c_size_t(0)
    _check(lib().moe_attn_workspace_size(ctypes.byref(dims), n_seqs, max_len, ctypes.byref(n)))
    return torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=device)


def attn_chunk_plan(dims: CAttnDims, n_seqs: int, max_len: int) -> tuple[int, int]:
    """(positions per chunk, chunk partial slots per query head) for these sizes."""
    c, n = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().moe_attn_chunk_plan(ctypes.byref(dims), n_seqs, max_len, ctypes.byref(c), ctypes.byref(n)))
    return int(c.value), int(n.value)


def _attn_args(dims, a, pos, out, ws):
    B, _, _ = a.q.shape
    max_len = a.k_cache.shape[2]
    out = out if out is not None else torch.empty_like(a.q)
    ws = ws if ws is not None else attn_workspace(dims, B, max_len, a.q.device)
    args = [ctypes.byref(dims), B, max_len, _ptr(a.q), _ptr(a.k_new), _ptr(a.v_new), _ptr(a.q_norm_w),
            _ptr(a.k_norm_w), _ptr(a.sinks), _ptr(pos), _ptr(a.k_cache), _ptr(a.v_cache), _ptr(out), _ptr(ws),
            ws.numel()]
    return args, out


def attn_decode(dims: CAttnDims, a: gen.AttnInputs, pos: torch.Tensor, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_attn_decode: writes the new keys/values into a.k_cache / a.v_cache
    (device tensors) and returns out [B, Hq, 128]."""
    args, out = _attn_args(dims, a, pos, out, ws)
    _check(lib().moe_attn_decode(*args, _stream(stream)))
    return out


def attn_decode_timed(dims: CAttnDims, a: gen.AttnInputs, pos: torch.Tensor, out: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, stream=None):
    """moe_attn_decode_timed: (out, {kernel: us}).  Synchronises the stream."""
    args, out = _attn_args(dims, a, pos, out, ws)
    us = (ctypes.c_float * 2)()
    _check(lib().moe_attn_decode_timed(*args, us, _stream(stream)))
    return out, dict(zip(("attn_chunk", "attn_combine"), (float(v) for v in us)))
