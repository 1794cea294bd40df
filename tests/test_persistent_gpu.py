"""GPU parity of the persistent batch-1 decode kernel (one dispatch per 64
layers, one block per CU, mailbox exchanges) and of the three-kernel path it
replaces, on the same seeded inputs; the oracle decides both.  Covers the
full-size q4_1 and NVFP4 layers, fewer routed experts than blocks, equal
logits, a router bias, stacks across the 32-layer launch boundary, graph
replays, and the give-up path of its bounded waits (forced from the host by
a spin limit of zero, every kernel still ending normally)."""
import functools
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_moe_decode_route_amd import binding as B
from sparse_moe_decode_route_amd import inputs as gen
from tests.helpers import REL_L2_TOL, check_routing, decode_band, rel_l2

pytestmark = pytest.mark.gpu

FP32_PATH_TOL = 5e-5
PATHS = {"persistent": B.PATH_PERSISTENT, "kernels": B.PATH_KERNELS}


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=None)
def _layer(dims, cfg_id, layer=0, zipf_s=None, router_zero=False):
    host = gen.make_layer(dims, cfg_id=cfg_id, layer=layer, zipf_s=zipf_s, router_zero=router_zero)
    return host, B.upload_layer(host, _dev())


def _router64(host):
    return oracle.bf16_array(host.router.numpy().view(np.uint16))


@pytest.fixture(params=list(PATHS))
def path(request):
    B.set_decode_path(PATHS[request.param])
    yield request.param
    B.set_decode_path(B.PATH_KERNELS)


def _one(host, dl, x, label):
    ws = B.workspace(host.dims, 1)
    y, idx, w = B.layer_forward(dl, x.to(_dev()), ws=ws)
    torch.cuda.synchronize()
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
def test_full_layer_batch1_both_paths(path, wfmt, cfg):
    dims = gen.LayerDims(2048, 512, wfmt=wfmt)
    host, dl = _layer(dims, cfg)
    for draw in range(8):
        _one(host, dl, gen.make_hidden(cfg, 1, 2048, draw=200 + draw), f"{path} {wfmt} draw {draw}")


def test_paths_agree_on_routing_and_output():
    dims = gen.LayerDims(2048, 512, wfmt="q4_1")
    host, dl = _layer(dims, 2)
    for draw in range(4):
        x = gen.make_hidden(2, 1, 2048, draw=300 + draw).to(_dev())
        outs = {}
        for name, code in PATHS.items():
            B.set_decode_path(code)
            outs[name] = B.layer_forward(dl, x)
        B.set_decode_path(B.PATH_KERNELS)
        torch.cuda.synchronize()
        (yp, ip, wp), (yk, ik, wk) = outs["persistent"], outs["kernels"]
        assert torch.equal(ip, ik)
        assert float((wp - wk).abs().max()) <= 2e-6
        assert float(rel_l2(yp.cpu().numpy(), yk.cpu().numpy()).max()) <= FP32_PATH_TOL


@pytest.fixture
def persistent():
    B.set_decode_path(B.PATH_PERSISTENT)
    yield
    B.set_decode_path(B.PATH_KERNELS)


@pytest.mark.parametrize("case", ["e64", "e64_equal_logits", "zipf_bias", "top4"])
def test_persistent_shapes(persistent, case):
    if case == "e64":
        host, dl = _layer(gen.LayerDims(2048, 512, n_routed=64, n_shared=1, top_k=6, wfmt="q4_1"), 61)
    elif case == "e64_equal_logits":
        host, dl = _layer(gen.LayerDims(2048, 512, n_routed=64, n_shared=1, top_k=6, wfmt="q4_1"), 62,
                          router_zero=True)
    elif case == "zipf_bias":
        host, dl = _layer(gen.LayerDims(2048, 512, wfmt="q4_1"), 63, zipf_s=1.1)
    else:
        host, dl = _layer(gen.LayerDims(2048, 512, n_routed=128, n_shared=1, top_k=4, wfmt="nvfp4"), 64)
    for draw in range(3):
        x = gen.make_hidden(61, 1, 2048, draw=draw)
        y, idx, w = _one(host, dl, x, f"persistent {case} draw {draw}")
        if case == "e64_equal_logits":
            assert idx.tolist() == [[0, 1, 2, 3, 4, 5]]
            np.testing.assert_allclose(w, np.full((1, 6), 1 / 6), rtol=1e-6)


@pytest.mark.parametrize("wfmt,L", [("nvfp4", 5), ("nvfp4", 66)])
def test_persistent_stack_teacher_forced(persistent, wfmt, L):
    """L layers through the persistent path (66: two launches, 64 + 2 layers;
    the oracle checks layers 0-2 and 62-65 teacher-forced)."""
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
        host = gen.Layer(dims, lay.router.cpu(), None, lay.experts.cpu(), lay.tensor_scale.cpu())
        oi, ow, ol, _ = oracle.layer_forward(host, x)
        check_routing(itr[l], None, ol, oi, ow, decode_band(x, _router64(host)) + 1e-5)
        _, _, _, oy = oracle.layer_forward(host, x, forced=itr[l])
        err = float(rel_l2(ytr[l], oy).max())
        print(f"[persistent stack {wfmt} L={L}] layer {l} rel-L2 {err:.3e}")
        assert err <= FP32_PATH_TOL, (l, err)


def test_persistent_stack_graph_replays_match_eager(persistent):
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


def test_persistent_give_up_path_sets_error_and_nan(persistent):
    """A spin limit of 0 makes every wait that is not satisfied at its first
    poll give up: the call must end (no hang) with NaN outputs and an error
    from moe_decode_check; the next call with the normal limit is correct."""
    dims = gen.LayerDims(2048, 512, wfmt="q4_1")
    host, dl = _layer(dims, 2)
    x = gen.make_hidden(2, 1, 2048, draw=400).to(_dev())
    ws = B.workspace(dims, 1)
    os.environ["MOE_PERSISTENT_SPIN_LIMIT"] = "0"
    try:
        y, _, _ = B.layer_forward(dl, x, ws=ws)
        torch.cuda.synchronize()
    finally:
        del os.environ["MOE_PERSISTENT_SPIN_LIMIT"]
    try:
        B.decode_check(dims, 1, ws)
        gave_up = False
    except B.MoeError as e:
        gave_up = True
        assert "gave up" in str(e)
    if gave_up:
        assert torch.isnan(y).all()
    y2, _, _ = B.layer_forward(dl, x, ws=ws)
    torch.cuda.synchronize()
    B.decode_check(dims, 1, ws)
    assert not torch.isnan(y2).any()
    print(f"[give-up] first call gave up: {gave_up}")
