"""moe_layer_forward_noalloc: the layer with the library's static device
scratch as workspace, for callers that cannot allocate.  It must reject a
call whose workspace would not fit before touching the device, and on the
GPU give exactly what moe_layer_forward gives (same kernels, same order) on
consecutive calls of different sizes, the later one smaller, so that a
stale part of the shared scratch cannot leak into a result."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_moe_decode_route_amd import binding as B
from sparse_moe_decode_route_amd import inputs as gen

WORKSPACE = -3


def _cd(**kw):
    base = dict(d_model=2048, d_ff=512, n_routed=256, n_shared=1, top_k=6, wfmt=1)
    base.update(kw)
    return B.CDims(**base)


def test_noalloc_rejects_oversized_workspace_before_enqueue():
    L = B.lib()
    d = _cd()
    need = ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(d), 4096, ctypes.byref(need)) == 0
    assert need.value > (16 << 20)
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: the size check fails first
    w = B.CLayerWeights(0x10000, 0, 0x20000, 0)
    assert L.moe_layer_forward_noalloc(ctypes.byref(d), ctypes.byref(w), fake, 0, 4096, fake, None, None,
                                       None) == WORKSPACE
    assert b"static scratch" in L.moe_last_error()


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def _check_pair(dl, x):
    T = x.shape[0]
    dims = dl.dims
    y_ref, i_ref, w_ref = B.layer_forward(dl, x)
    y = torch.full((T, dims.d_model), float("nan"), device=x.device)
    idx = torch.full((T, dims.top_k), -7, dtype=torch.int32, device=x.device)
    w = torch.full((T, dims.top_k), float("nan"), device=x.device)
    B.layer_forward_noalloc(dl, x, y, idx, w)
    torch.cuda.synchronize()
    assert torch.equal(i_ref, idx), (T, i_ref, idx)
    assert torch.equal(w_ref, w), T
    assert torch.equal(y_ref, y), (T, float((y_ref - y).abs().max()))


@pytest.mark.gpu
@pytest.mark.parametrize("wfmt,sizes", [("q4_1", (8, 1)), ("nvfp4", (32, 3)), ("q4_1", (4, 2))])
def test_noalloc_matches_layer_forward_on_consecutive_calls(wfmt, sizes):
    dims = gen.LayerDims(2048, 512, wfmt=wfmt)
    host = gen.make_layer(dims, cfg_id=60, layer=0)
    dl = B.upload_layer(host, _dev())
    for k, T in enumerate(sizes):  # the second call is smaller than the first
        x = gen.make_hidden(60, T, 2048, draw=k).to(_dev())
        _check_pair(dl, x)


@pytest.mark.gpu
def test_noalloc_small_bf16_layer_and_bf16_tokens():
    w = gen.WORKLOADS["c1_small_bf16"]
    host = gen.make_layer(w["dims"], cfg_id=w["cfg_id"])
    dl = B.upload_layer(host, _dev())
    for k, T in enumerate((6, 2)):
        x = gen.to_bf16(gen.make_hidden(w["cfg_id"], T, 512, draw=20 + k)).to(_dev())
        _check_pair(dl, x)
