"""GPU parity of the batch-1 decode path with one kernel per layer and one
active expert per XCD (moe_set_decode_path(MOE_PATH_XCD)): full-size q4_1 and
NVFP4 layers against the oracle, agreement with the three-kernel path, a
Zipf-biased router, stacks across the 64-layer clear of the barrier counters
(teacher-forced against the oracle), graph replays, and the fallback for shapes
the path is not built for."""
import functools

import numpy as np
import pytest
import torch

import oracle
from sparse_moe_decode_route_amd import binding as B
from sparse_moe_decode_route_amd import inputs as gen
from tests.helpers import REL_L2_TOL, check_routing, decode_band, rel_l2

pytestmark = pytest.mark.gpu

FP32_PATH_TOL = 5e-5


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=None)
def _layer(dims, cfg_id, layer=0, zipf_s=None, router_zero=False):
    host = gen.make_layer(dims, cfg_id=cfg_id, layer=layer, zipf_s=zipf_s, router_zero=router_zero)
    return host, B.upload_layer(host, _dev())


def _router64(host):
    return oracle.bf16_array(host.router.numpy().view(np.uint16))


@pytest.fixture
def xcd():
    B.set_decode_path(B.PATH_XCD)
    yield
    B.set_decode_path(B.PATH_KERNELS)


def _one(host, dl, x, label, check=True):
    ws = B.workspace(host.dims, 1)
    y, idx, w = B.layer_forward(dl, x.to(_dev()), ws=ws)
    torch.cuda.synchronize()
    if check:
        # the workspace's error word is written only by the paths with waits
        B.decode_check(host.dims, 1, ws)
    y, idx, w = y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    x64 = x.double().numpy()
    oi, ow, ol, _ = oracle.layer_forward(host, x64)
    n_exact, n_amb = check_routing(idx, w, ol, oi, ow, decode_band(x64, _router64(host)))
    _, _, _, oy = oracle.layer_forward(host, x64, forced=idx)
    err = float(rel_l2(y, oy).max())
    print(f"[{label}] exact={n_exact} ambiguous={n_amb} rel-L2 {err:.3e}")
    assert err <= REL_L2_TOL and err <= FP32_PATH_TOL, err
    return y, idx, w


@pytest.mark.parametrize("wfmt,cfg", [("q4_1", 2), ("nvfp4", 4)])
def test_xcd_full_layer_batch1(xcd, wfmt, cfg):
    dims = gen.LayerDims(2048, 512, wfmt=wfmt)
    host, dl = _layer(dims, cfg)
    for draw in range(8):
        _one(host, dl, gen.make_hidden(cfg, 1, 2048, draw=200 + draw), f"xcd {wfmt} draw {draw}")


def test_xcd_zipf_biased_router(xcd):
    host, dl = _layer(gen.LayerDims(2048, 512, wfmt="q4_1"), 63, zipf_s=1.1)
    for draw in range(3):
        _one(host, dl, gen.make_hidden(61, 1, 2048, draw=draw), f"xcd zipf draw {draw}")


def test_xcd_agrees_with_three_kernels():
    dims = gen.LayerDims(2048, 512, wfmt="q4_1")
    host, dl = _layer(dims, 2)
    for draw in range(4):
        x = gen.make_hidden(2, 1, 2048, draw=300 + draw).to(_dev())
        outs = {}
        for name, code in (("xcd", B.PATH_XCD), ("kernels", B.PATH_KERNELS)):
            B.set_decode_path(code)
            outs[name] = B.layer_forward(dl, x)
        B.set_decode_path(B.PATH_KERNELS)
        torch.cuda.synchronize()
        (yx, ix, wx), (yk, ik, wk) = outs["xcd"], outs["kernels"]
        assert torch.equal(ix, ik)
        assert float((wx - wk).abs().max()) <= 2e-6
        assert float(rel_l2(yx.cpu().numpy(), yk.cpu().numpy()).max()) <= FP32_PATH_TOL


def test_xcd_unsupported_shape_falls_back(xcd):
    """64 routed experts: the path is not built for it, the call takes the
    three-kernel path and stays correct."""
    host, dl = _layer(gen.LayerDims(2048, 512, n_routed=64, n_shared=1, top_k=6, wfmt="q4_1"), 61)
    _one(host, dl, gen.make_hidden(61, 1, 2048, draw=5), "xcd fallback e64", check=False)


@pytest.mark.parametrize("wfmt,L", [("q4_1", 5), ("nvfp4", 66)])
def test_xcd_stack_teacher_forced(xcd, wfmt, L):
    """L layers on the path (66: across the clear of the barrier counters every
    64 layers; the oracle checks layers 0-2 and 62-65 teacher-forced)."""
    dims = gen.LayerDims(2048, 512, wfmt=wfmt)
    checked = set(range(L)) if L <= 8 else {0, 1, 2, L - 4, L - 3, L - 2, L - 1}
    lays = [gen.make_layer(dims, cfg_id=65, layer=l, device="cuda") for l in range(L)]
    devs = []
    for lay in lays:
        packed = torch.empty_like(lay.experts)
        B.repack_weights(dims, lay.experts, packed, dims.n_experts)
        devs.append(B.DeviceLayer(dims, lay.router, None, packed, lay.tensor_scale))
    torch.cuda.synchronize()
    stack = B.StackHandle(devs)
    x0 = gen.make_hidden(65, 1, 2048)
    ws = B.workspace(dims, 1)
    y, ytr, itr = B.stack_decode(stack, x0.to(_dev()), ws=ws, trace=True)
    torch.cuda.synchronize()
    B.decode_check(dims, 1, ws)
    y, ytr, itr = y.cpu().numpy(), ytr.cpu().numpy(), itr.cpu().numpy()
    assert np.array_equal(y, ytr[-1])
    for l in sorted(checked):
        x = x0.double().numpy() if l == 0 else oracle.rmsnorm(ytr[l - 1][0])[None]
        lay = lays[l]
        host = gen.Layer(dims, lay.router.cpu(), None, lay.experts.cpu(),
                         None if lay.tensor_scale is None else lay.tensor_scale.cpu())
        oi, ow, ol, _ = oracle.layer_forward(host, x)
        check_routing(itr[l], None, ol, oi, ow, decode_band(x, _router64(host)) + 1e-5)
        _, _, _, oy = oracle.layer_forward(host, x, forced=itr[l])
        err = float(rel_l2(ytr[l], oy).max())
        print(f"[xcd stack {wfmt} L={L}] layer {l} rel-L2 {err:.3e}")
        assert err <= FP32_PATH_TOL, (l, err)


def test_xcd_stack_graph_replays_match_eager(xcd):
    dims = gen.LayerDims(2048, 512, wfmt="q4_1")
    devs = [_layer(dims, 66, layer=l)[1] for l in range(3)]
    stack = B.StackHandle(devs)
    xs = gen.make_hidden(66, 4, 2048, device=_dev())
    x_static = torch.empty((1, 2048), device=_dev())
    y_static = torch.empty((1, 2048), device=_dev())
    ws = B.workspace(dims, 1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.stack_decode(stack, x_static, ws=ws, y=y_static)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.stack_decode(stack, x_static, ws=ws, y=y_static)
    for i in range(4):
        x_static.copy_(xs[i:i + 1])
        g.replay()
        torch.cuda.synchronize()
        got = y_static.clone()
        ref, _, _ = B.stack_decode(stack, xs[i:i + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(got, ref), i
        B.decode_check(dims, 1, ws)


def test_xcd_give_up_path_sets_error_and_nan(xcd):
    """A barrier limit of 0 ticks makes every XCD barrier that is not complete
    at its first poll give up: the call must end (no hang) with NaN outputs and
    an error from moe_decode_check; the next call with the normal limit is
    correct."""
    import os
    dims = gen.LayerDims(2048, 512, wfmt="q4_1")
    host, dl = _layer(dims, 2)
    x = gen.make_hidden(2, 1, 2048, draw=400).to(_dev())
    ws = B.workspace(dims, 1)
    os.environ["MOE_XCD_SPIN_TICKS"] = "0"
    try:
        y, _, _ = B.layer_forward(dl, x, ws=ws)
        torch.cuda.synchronize()
    finally:
        del os.environ["MOE_XCD_SPIN_TICKS"]
    try:
        B.decode_check(dims, 1, ws)
        gave_up = False
    except B.MoeError as e:
        gave_up = True
        assert "gave up" in str(e)
    if gave_up:
        assert torch.isnan(y).any()
    y2, _, _ = B.layer_forward(dl, x, ws=ws)
    torch.cuda.synchronize()
    B.decode_check(dims, 1, ws)
    assert not torch.isnan(y2).any()
    print(f"[xcd give-up] first call gave up: {gave_up}")
