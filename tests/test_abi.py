"""C-ABI checks that need no GPU: the library loads, exports every entry
point declared in include/moe.h, and rejects bad arguments on the host with
the documented status codes before anything is enqueued."""
import ctypes
import os
import re

import pytest

from sparse_moe_decode_route_amd import binding as B
from sparse_moe_decode_route_amd import inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, ALIGNMENT = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.SO_PATH):
        from sparse_moe_decode_route_amd import build
        build.build()
    return B.lib()


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("moe_route_topk", "moe_expert_ffn_q4", "moe_layer_forward"):
        assert required in names
    assert set(names) == set(B.ENTRY_POINTS)


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name


def _d(**kw):
    base = dict(d_model=2048, d_ff=512, n_routed=256, n_shared=1, top_k=6, wfmt=1)
    base.update(kw)
    return B.CDims(**base)


def test_sizes(L):
    d = _d()
    assert L.moe_packed_expert_bytes(ctypes.byref(d)) == 1_966_080
    d4 = _d(wfmt=2)
    assert L.moe_packed_expert_bytes(ctypes.byref(d4)) == 1_769_472
    db = _d(d_model=512, d_ff=128, wfmt=0)
    assert L.moe_packed_expert_bytes(ctypes.byref(db)) == 393_216
    n = ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n)) == OK and n.value > 0
    assert L.moe_workspace_size(ctypes.byref(d), 4096, ctypes.byref(n)) == OK


@pytest.mark.parametrize("bad", [dict(d_model=48), dict(d_model=0), dict(d_ff=8200), dict(n_routed=300),
                                 dict(top_k=0), dict(top_k=9), dict(n_routed=4, top_k=6), dict(n_shared=5)])
def test_bad_dims_rejected(L, bad):
    d = _d(**bad)
    n = ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n)) == INVALID
    assert L.moe_packed_expert_bytes(ctypes.byref(d)) == 0
    assert L.moe_last_error()


def test_unknown_format_rejected(L):
    d = _d(wfmt=7)
    n = ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n)) == UNSUPPORTED


def test_entry_points_validate_before_enqueue(L):
    d = _d()
    fake = ctypes.c_void_p(0x10000)       # never dereferenced: every call below fails validation
    odd = ctypes.c_void_p(0x10004)        # misaligned
    w = B.CLayerWeights(0x10000, 0, 0x20000, 0)
    wnull = B.CLayerWeights(0, 0, 0x20000, 0)
    # NULL x
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), None, 0, 1, fake, None, None, fake, 1 << 30, None) == INVALID
    # NULL router
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(wnull), fake, 0, 1, fake, None, None, fake, 1 << 30, None) == INVALID
    # misaligned y
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), fake, 0, 1, odd, None, None, fake, 1 << 30, None) == ALIGNMENT
    # workspace too small / missing
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), fake, 0, 1, fake, None, None, fake, 16, None) == WORKSPACE
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), fake, 0, 1, fake, None, None, None, 0, None) == WORKSPACE
    # bad token counts and activation type
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), fake, 0, 0, fake, None, None, fake, 1 << 30, None) == INVALID
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), fake, 5, 1, fake, None, None, fake, 1 << 30, None) == UNSUPPORTED
    assert L.moe_expert_ffn_q4(ctypes.byref(d), fake, 0, 70000, fake, None, fake, fake, fake, fake, 1 << 30, None) == INVALID
    # NVFP4 needs tensor scales
    d4 = _d(wfmt=2)
    assert L.moe_expert_ffn_q4(ctypes.byref(d4), fake, 0, 1, fake, None, fake, fake, fake, fake, 1 << 30, None) == INVALID
    assert L.moe_route_topk(ctypes.byref(d), fake, 0, 70000, fake, None, fake, fake, None, fake, 1 << 30, None) == INVALID
    assert L.moe_stack_decode(ctypes.byref(d), 0, ctypes.byref(w), fake, 1, fake, None, None, fake, 1 << 30, None) == INVALID
    assert L.moe_stack_decode(ctypes.byref(d), 1, ctypes.byref(w), fake, 9, fake, None, None, fake, 1 << 30, None) == INVALID
    # overlapping repack buffers
    assert L.moe_repack_weights(ctypes.byref(d), fake, fake, 1, None) == INVALID
    assert L.moe_repack_weights(ctypes.byref(d), fake, ctypes.c_void_p(0x90000000), 0, None) == INVALID
    assert b"n_experts" in L.moe_last_error()


def test_timed_entry_points_validate_before_enqueue(L):
    # the timed calls check their arguments before anything (the stream hold
    # included) is enqueued: every call below fails validation on the host
    d = _d()
    fake = ctypes.c_void_p(0x10000)
    w = B.CLayerWeights(0x10000, 0, 0x20000, 0)
    us = (ctypes.c_float * 8)()
    nk = ctypes.c_int32(0)
    names = ctypes.create_string_buffer(64)
    # no timing outputs
    assert L.moe_stack_decode_timed(ctypes.byref(d), 1, ctypes.byref(w), fake, 1, fake, None, fake, 1 << 30,
                                    None, ctypes.byref(nk), names, 64, None) == INVALID
    # too many tokens for the stack, and no layers
    assert L.moe_stack_decode_timed(ctypes.byref(d), 1, ctypes.byref(w), fake, 9, fake, None, fake, 1 << 30,
                                    us, ctypes.byref(nk), names, 64, None) == INVALID
    assert L.moe_stack_decode_timed(ctypes.byref(d), 0, ctypes.byref(w), fake, 1, fake, None, fake, 1 << 30,
                                    us, ctypes.byref(nk), names, 64, None) == INVALID
    # workspace too small
    assert L.moe_stack_decode_timed(ctypes.byref(d), 1, ctypes.byref(w), fake, 1, fake, None, fake, 16,
                                    us, ctypes.byref(nk), names, 64, None) == WORKSPACE
    # prefill: NULL x, bad activation type, no timing outputs
    assert L.moe_layer_forward_prefill_timed(ctypes.byref(d), ctypes.byref(w), None, 0, 64, fake, fake, 1 << 30,
                                             us, ctypes.byref(nk), names, 64, None) == INVALID
    assert L.moe_layer_forward_prefill_timed(ctypes.byref(d), ctypes.byref(w), fake, 7, 64, fake, fake, 1 << 30,
                                             us, ctypes.byref(nk), names, 64, None) == UNSUPPORTED
    assert L.moe_layer_forward_prefill_timed(ctypes.byref(d), ctypes.byref(w), fake, 0, 64, fake, fake, 1 << 30,
                                             None, ctypes.byref(nk), names, 64, None) == INVALID


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, -5):
        assert L.moe_status_string(s)


def test_binding_error_carries_message(L):
    dims = gen.LayerDims(48, 64)
    with pytest.raises(B.MoeError) as e:
        B.workspace_size(dims, 1)
    assert "d_model" in str(e.value)


def test_lm_head_sizes_and_checks(L):
    V, D = 146_484, 2048
    assert L.moe_lm_head_bytes(V, D, 1) == V * D // 32 * 20
    assert L.moe_lm_head_bytes(V, D, 2) == V * D // 2 + V * D // 16
    assert L.moe_lm_head_bytes(V, D, 0) == V * D * 2
    assert B.lm_head_bytes(V, D, "q4_1") == gen.matrix_bytes(V, D, "q4_1")
    for v, d, f in ((0, D, 1), (V, 48, 1), (V, 8192, 1), (V, D, 7), (1 << 25, D, 1)):
        assert L.moe_lm_head_bytes(v, d, f) == 0
    fake = ctypes.c_void_p(0x10000)
    out = ctypes.c_void_p(0x90000000)
    odd = ctypes.c_void_p(0x10004)
    # shapes, formats, token counts
    assert L.moe_lm_head(V, 48, 1, fake, None, fake, 0, 1, out, None) == INVALID
    assert L.moe_lm_head(0, D, 1, fake, None, fake, 0, 1, out, None) == INVALID
    assert L.moe_lm_head(V, D, 9, fake, None, fake, 0, 1, out, None) == UNSUPPORTED
    assert L.moe_lm_head(V, D, 1, fake, None, fake, 3, 1, out, None) == UNSUPPORTED
    assert L.moe_lm_head(V, D, 1, fake, None, fake, 0, 0, out, None) == INVALID
    assert L.moe_lm_head(V, D, 1, fake, None, fake, 0, 9, out, None) == INVALID
    # pointers: NULL, misaligned, NVFP4 tensor scale, overlap of logits with an input
    assert L.moe_lm_head(V, D, 1, None, None, fake, 0, 1, out, None) == INVALID
    assert L.moe_lm_head(V, D, 1, fake, None, odd, 0, 1, out, None) == ALIGNMENT
    assert L.moe_lm_head(V, D, 2, fake, None, fake, 0, 1, out, None) == INVALID
    assert b"tensor_scale" in L.moe_last_error()
    assert L.moe_lm_head(V, D, 2, ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x10002), fake, 0, 1, out, None) == ALIGNMENT
    assert L.moe_lm_head(V, D, 1, fake, None, ctypes.c_void_p(0x90000400), 0, 1, out, None) == INVALID
    assert b"overlap" in L.moe_last_error()
    assert L.moe_lm_head(V, D, 1, ctypes.c_void_p(0x8F000000), None, fake, 0, 1, out, None) == INVALID
    # repack: overlap and shape
    assert L.moe_lm_head_repack(V, D, 1, fake, fake, None) == INVALID
    assert L.moe_lm_head_repack(V, 40, 1, fake, out, None) == INVALID
    kus = ctypes.c_float()
    assert L.moe_lm_head_timed(V, D, 1, fake, None, fake, 0, 1, out, None, None) == INVALID
    assert L.moe_lm_head_timed(V, D, 1, fake, None, fake, 0, 0, out, ctypes.byref(kus), None) == INVALID


def test_attn_checks(L):
    d = B.attn_dims(32, 4, 513)
    n = ctypes.c_size_t()
    assert L.moe_attn_workspace_size(ctypes.byref(d), 1, 8192, ctypes.byref(n)) == OK and n.value > 0
    full = B.attn_dims(32, 4, 0)
    n2 = ctypes.c_size_t()
    assert L.moe_attn_workspace_size(ctypes.byref(full), 1, 8192, ctypes.byref(n2)) == OK and n2.value > n.value
    for bad, code in ((B.CAttnDims(32, 4, 64, 513, 1e4, 1e-6), UNSUPPORTED), (B.CAttnDims(30, 4, 128, 513, 1e4, 1e-6), INVALID),
                      (B.CAttnDims(48, 4, 128, 513, 1e4, 1e-6), UNSUPPORTED), (B.CAttnDims(32, 4, 128, -1, 1e4, 1e-6), INVALID),
                      (B.CAttnDims(32, 4, 128, 513, 0.0, 1e-6), INVALID), (B.CAttnDims(32, 4, 128, 513, 1e4, -1.0), INVALID)):
        assert L.moe_attn_workspace_size(ctypes.byref(bad), 1, 8192, ctypes.byref(n)) == code
    assert L.moe_attn_workspace_size(ctypes.byref(d), 0, 8192, ctypes.byref(n)) == INVALID
    assert L.moe_attn_workspace_size(ctypes.byref(d), 1, 0, ctypes.byref(n)) == INVALID
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(10)]
    ws = ctypes.c_void_p(0x40000000)
    args = lambda **kw: [ctypes.byref(d), 1, 8192] + [kw.get(str(i), p[i]) for i in range(10)] + [kw.get("ws", ws), kw.get("wsb", 1 << 30), None]
    assert L.moe_attn_decode(*args(**{"0": None})) == INVALID                         # NULL q
    assert L.moe_attn_decode(*args(**{"6": ctypes.c_void_p(0x700004)})) == ALIGNMENT  # misaligned pos
    assert L.moe_attn_decode(*args(wsb=16)) == WORKSPACE
    # the k cache (2 MiB at 0x800000) overlapping the v cache
    assert L.moe_attn_decode(*args(**{"8": ctypes.c_void_p(0x810000)})) == INVALID
    assert b"overlaps" in L.moe_last_error()
    kus = (ctypes.c_float * 2)()
    assert L.moe_attn_decode_timed(*(args(**{"0": None})[:-1] + [kus, None])) == INVALID


def test_attn_chunk_plan(L):
    """Chunk plan: windows in 64-position chunks for groups of 8 (matrix-core
    kernel), 32 otherwise; for full layers the smallest
    power of two in [64, 1024] keeping a call near 512 blocks for groups of 8
    (matrix-core kernel), near 1024 otherwise; the workspace
    holds one (max, sum, 128-value) partial per slot and query head."""
    cases = (((32, 4, 513), 1, 8192, 64, 9), ((32, 4, 513), 1, 100, 64, 2), ((16, 4, 513), 1, 8192, 32, 17), ((32, 4, 0), 1, 131072, 1024, 128),
             ((32, 4, 0), 1, 8192, 64, 128), ((32, 4, 0), 8, 131072, 1024, 128), ((32, 4, 0), 1, 1, 64, 1),
             ((16, 4, 0), 1, 131072, 512, 256), ((16, 4, 0), 1, 16384, 64, 256), ((32, 4, 0), 1, 16384, 128, 128))
    for (hq, hkv, win), nseq, ml, chunk, slots in cases:
        d = B.attn_dims(hq, hkv, win)
        assert B.attn_chunk_plan(d, nseq, ml) == (chunk, slots)
        n = ctypes.c_size_t()
        assert L.moe_attn_workspace_size(ctypes.byref(d), nseq, ml, ctypes.byref(n)) == OK
        need = nseq * hq * slots * 130 * 4
        assert need <= n.value < need + 3 * 256
    c = ctypes.c_int32()
    assert L.moe_attn_chunk_plan(ctypes.byref(B.attn_dims(32, 4, 0)), 1, 8192, ctypes.byref(c), None) == INVALID
    assert L.moe_attn_chunk_plan(ctypes.byref(B.attn_dims(32, 4, 0)), 0, 8192, ctypes.byref(c), ctypes.byref(c)) == INVALID


def test_decode_path_switch(L):
    # the three batch-1 paths are accepted, anything else is refused (host only)
    try:
        for path in (B.PATH_PERSISTENT, B.PATH_XCD, B.PATH_KERNELS):
            assert L.moe_set_decode_path(path) == OK
        for bad in (-1, 3):
            assert L.moe_set_decode_path(bad) == INVALID
            assert b"MOE_PATH_XCD" in L.moe_last_error()
    finally:
        L.moe_set_decode_path(B.PATH_KERNELS)
