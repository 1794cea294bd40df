"""GPU parity: libmoe's HIP path against the CPU oracle on the same seeded bytes.

Selected experts must match exactly (outside the fp32 rounding band around
the top-k cut, see helpers.check_routing) and the layer output must be within
relative L2 error 2e-3 per token of the oracle's fp64 result."""
import functools

import numpy as np
import pytest
import torch

import oracle
from sparse_moe_decode_route_amd import binding as B
from sparse_moe_decode_route_amd import inputs as gen
from tests.helpers import REL_L2_TOL, check_chain_divergence, check_routing, decode_band, rel_l2, router_band

pytestmark = pytest.mark.gpu

# fp32 accumulation of 4-bit-decoded weights lands far inside the contract;
# this tighter guard catches a dropped term or a wrong scale early.
FP32_PATH_TOL = 5e-5


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=None)
def _layer(name_or_dims, cfg_id, layer=0, zipf_s=None, router_zero=False):
    dims = gen.WORKLOADS[name_or_dims]["dims"] if isinstance(name_or_dims, str) else name_or_dims
    host = gen.make_layer(dims, cfg_id=cfg_id, layer=layer, zipf_s=zipf_s, router_zero=router_zero)
    return host, B.upload_layer(host, _dev())


def _router64(host):
    return oracle.bf16_array(host.router.numpy().view(np.uint16))


def _run_layer_case(host, dev_layer, x32: torch.Tensor, label: str, prefill=False, band_extra=0.0):
    dims = host.dims
    T = x32.shape[0]
    xin = x32.to(_dev())
    y, idx, w = B.layer_forward(dev_layer, xin, prefill=prefill)
    torch.cuda.synchronize()
    y, idx, w = y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    x64 = x32.double().numpy()
    oi, ow, ol, oy = oracle.layer_forward(host, x64)
    band = decode_band(x64, _router64(host)) + band_extra
    n_exact, n_amb = check_routing(idx, w, ol, oi, ow, band)
    # outputs against the oracle on the GPU's own selection
    _, _, _, oy_forced = oracle.layer_forward(host, x64, forced=idx)
    err = rel_l2(y, oy_forced)
    print(f"[{label}] T={T} exact={n_exact} ambiguous={n_amb} max rel-L2 {err.max():.3e}")
    assert np.all(err <= REL_L2_TOL), err
    return err, n_exact, n_amb


# --------------------------------------------------------------------------- small layer (bf16)

def test_small_bf16_layer_all_tokens():
    host, dl = _layer("c1_small_bf16", 1)
    x = gen.make_hidden(1, 4, 512)
    err, n_exact, _ = _run_layer_case(host, dl, x, "c1 bf16")
    assert err.max() <= FP32_PATH_TOL and n_exact == 4


def test_small_bf16_route_and_ffn_entry_points():
    host, dl = _layer("c1_small_bf16", 1)
    dims = host.dims
    x = gen.make_hidden(1, 4, 512, draw=1)
    xd = x.to(_dev())
    idx, w, logits = B.route_topk(dims, xd, dl.router, None)
    torch.cuda.synchronize()
    x64 = x.double().numpy()
    oi, ow, ol, oy = oracle.layer_forward(host, x64)
    lg = logits.cpu().numpy()
    band = router_band(x64, _router64(host))
    assert np.all(np.abs(lg - ol) <= band[:, None] / 2)
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), ol, oi, ow, band)
    # expert FFN on the oracle's routing
    oi_d = torch.from_numpy(oi).to(_dev())
    ow_d = torch.from_numpy(ow.astype(np.float32)).to(_dev())
    y = B.expert_ffn_q4(dims, xd, dl.experts, dl.tensor_scale, oi_d, ow_d)
    torch.cuda.synchronize()
    assert np.all(rel_l2(y.cpu().numpy(), oy) <= FP32_PATH_TOL)


def test_deterministic_repeat():
    host, dl = _layer("c1_small_bf16", 1)
    x = gen.make_hidden(1, 4, 512, draw=2).to(_dev())
    y1, i1, w1 = B.layer_forward(dl, x)
    y2, i2, w2 = B.layer_forward(dl, x)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(i1, i2) and torch.equal(w1, w2)


# --------------------------------------------------------------------------- ragged small shapes

@pytest.mark.parametrize("wfmt", ["bf16", "q4_1", "nvfp4"])
@pytest.mark.parametrize("T", [1, 3, 8])
def test_ragged_small_shapes(wfmt, T):
    # d_model 96 -> 3 units of 32 (lane groups of 4 with an idle lane);
    # d_ff 160 -> 5 units; 20 routed experts, top-3, two shared experts
    dims = gen.LayerDims(96, 160, n_routed=20, n_shared=2, top_k=3, wfmt=wfmt)
    host, dl = _layer(dims, 40)
    x = gen.make_hidden(40, T, 96, draw=T)
    err, _, _ = _run_layer_case(host, dl, x, f"ragged {wfmt}")
    assert err.max() <= FP32_PATH_TOL


@pytest.mark.parametrize("wfmt", ["q4_1", "nvfp4"])
def test_wide_rows_loop_over_units(wfmt):
    # d_model 4096 -> 128 units per row: each lane loops over two units
    dims = gen.LayerDims(4096, 96, n_routed=16, n_shared=1, top_k=6, wfmt=wfmt)
    host, dl = _layer(dims, 41)
    x = gen.make_hidden(41, 2, 4096)
    err, _, _ = _run_layer_case(host, dl, x, f"wide {wfmt}")
    assert err.max() <= FP32_PATH_TOL


def test_equal_logits_choose_lowest_indices():
    dims = gen.LayerDims(128, 64, n_routed=32, n_shared=1, top_k=6, wfmt="q4_1")
    host, dl = _layer(dims, 42, router_zero=True)
    x = gen.make_hidden(42, 2, 128).to(_dev())
    y, idx, w = B.layer_forward(dl, x)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(6, dtype=np.int32), (2, 1)))
    np.testing.assert_allclose(w.cpu().numpy(), np.full((2, 6), 1 / 6), rtol=1e-6)


# --------------------------------------------------------------------------- full-size layers

def test_full_q4_1_layer_batch1_many_tokens():
    """d_model 2048, d_ff 512, 256 + 1 experts, q4_1: 16 independent batch-1 decodes."""
    host, dl = _layer("c2_layer_q4_1", 2)
    errs = []
    for draw in range(16):
        x = gen.make_hidden(2, 1, 2048, draw=draw)
        err, _, _ = _run_layer_case(host, dl, x, f"c2 draw {draw}")
        errs.append(err.max())
    assert max(errs) <= FP32_PATH_TOL


def test_full_nvfp4_layer_batch1_and_batch8():
    host, dl = _layer("c4_layer_nvfp4", 4)
    for draw in range(4):
        err, _, _ = _run_layer_case(host, dl, gen.make_hidden(4, 1, 2048, draw=draw), f"c4 b1 draw {draw}")
        assert err.max() <= FP32_PATH_TOL
    err, _, _ = _run_layer_case(host, dl, gen.make_hidden(4, 8, 2048, draw=100), "c4 b8")
    assert err.max() <= FP32_PATH_TOL


def test_full_q4_1_expert_ffn_given_routing():
    host, dl = _layer("c2_layer_q4_1", 2)
    dims = host.dims
    x = gen.make_hidden(2, 2, 2048, draw=50)
    # a routing the router would not choose: fixed experts with uneven weights
    idx = np.array([[255, 0, 17, 128, 64, 3], [1, 2, 3, 4, 5, 6]], dtype=np.int32)
    w = np.array([[0.5, 0.1, 0.1, 0.1, 0.1, 0.1], [0.25, 0.25, 0.125, 0.125, 0.125, 0.125]])
    y = B.expert_ffn_q4(dims, x.to(_dev()), dl.experts, None, torch.from_numpy(idx).to(_dev()),
                        torch.from_numpy(w.astype(np.float32)).to(_dev()))
    torch.cuda.synchronize()
    oy = oracle.experts_given(host, x.double().numpy(), idx, w)
    assert np.all(rel_l2(y.cpu().numpy(), oy) <= FP32_PATH_TOL)


# --------------------------------------------------------------------------- stack

def test_stack_teacher_forced_and_end_to_end():
    """4 layers at full size (q4_1), RMS-normalised between layers."""
    dims = gen.WORKLOADS["c3_stack47_q4_1"]["dims"]
    L = 4
    hosts = [gen.make_layer(dims, cfg_id=3, layer=l) for l in range(L)]
    devs = [B.upload_layer(h, _dev()) for h in hosts]
    stack = B.StackHandle(devs)
    x0 = gen.make_hidden(3, 1, 2048)
    y, ytr, itr = B.stack_decode(stack, x0.to(_dev()), trace=True)
    torch.cuda.synchronize()
    y, ytr, itr = y.cpu().numpy(), ytr.cpu().numpy(), itr.cpu().numpy()
    assert np.array_equal(y, ytr[-1])
    x = x0.double().numpy()
    for l in range(L):
        oi, ow, ol, _ = oracle.layer_forward(hosts[l], x)
        band = router_band(x, _router64(hosts[l])) + 1e-5
        check_routing(itr[l], None, ol, oi, ow, band)
        _, _, _, oy = oracle.layer_forward(hosts[l], x, forced=itr[l])
        err = rel_l2(ytr[l], oy)
        print(f"[stack] layer {l} teacher-forced rel-L2 {err.max():.3e}")
        assert err.max() <= FP32_PATH_TOL
        x = oracle.rmsnorm(ytr[l][0])[None]
    # end to end: the oracle's own fp64 chain; equal selections in every layer
    # and the output within 2e-3, or a first difference that the drift between
    # the two chains' inputs explains
    oy_end, otr, oitr = oracle.stack_forward(hosts, x0.double().numpy())
    same = [np.array_equal(np.sort(oitr[l], axis=1), np.sort(itr[l], axis=1)) for l in range(L)]
    if all(same):
        err = rel_l2(y, oy_end)
        print(f"[stack] end-to-end rel-L2 {err.max():.3e}")
        assert err.max() <= REL_L2_TOL
    else:
        l = same.index(False)
        x_gpu = x0.double().numpy() if l == 0 else oracle.rmsnorm(ytr[l - 1][0])[None]
        x_orc = x0.double().numpy() if l == 0 else oracle.rmsnorm(otr[l - 1][0])[None]
        band = float(router_band(x_gpu, _router64(hosts[l]))[0]) + 1e-5
        check_chain_divergence(oracle, hosts[l], x_gpu, x_orc, band, dims.top_k)


# --------------------------------------------------------------------------- batch-1 path variants

@pytest.mark.parametrize("dims", [
    gen.LayerDims(512, 128, wfmt="bf16"),                                  # bf16 units, 16 lanes per down row
    gen.LayerDims(4096, 256, n_routed=64, n_shared=1, top_k=6, wfmt="q4_1"),  # two units per lane, 8 lanes per row
    gen.LayerDims(2048, 1024, n_routed=32, n_shared=0, top_k=4, wfmt="nvfp4"),  # no shared expert, 32 lanes per row
    gen.LayerDims(1024, 2048, n_routed=48, n_shared=2, top_k=6, wfmt="q4_1"),   # two shared experts, 64 lanes per row
], ids=["bf16", "q4_1-upl2", "nvfp4-noshared", "q4_1-2shared"])
def test_batch1_path_shapes(dims):
    host, dl = _layer(dims, 43)
    for draw in range(3):
        x = gen.make_hidden(43, 1, dims.d_model, draw=draw)
        err, _, _ = _run_layer_case(host, dl, x, f"b1 {dims}")
        assert err.max() <= FP32_PATH_TOL


def test_batch1_equal_logits_choose_lowest_indices():
    dims = gen.LayerDims(2048, 512, n_routed=64, n_shared=1, top_k=6, wfmt="q4_1")
    host, dl = _layer(dims, 44, router_zero=True)
    x = gen.make_hidden(44, 1, 2048)
    y, idx, w = B.layer_forward(dl, x.to(_dev()))
    torch.cuda.synchronize()
    assert idx.cpu().numpy().tolist() == [[0, 1, 2, 3, 4, 5]]
    np.testing.assert_allclose(w.cpu().numpy(), np.full((1, 6), 1 / 6), rtol=1e-6)
    _, _, _, oy = oracle.layer_forward(host, x.double().numpy())
    assert rel_l2(y.cpu().numpy(), oy).max() <= FP32_PATH_TOL


def test_stack_graph_replays_match_eager():
    """A captured stack step replayed several times equals the eager call each time."""
    dims = gen.LayerDims(1024, 256, n_routed=32, n_shared=1, top_k=6, wfmt="q4_1")
    devs = [_layer(dims, 45, layer=l)[1] for l in range(3)]
    stack = B.StackHandle(devs)
    xs = gen.make_hidden(45, 4, 1024, device=_dev())
    x_static = torch.empty((1, 1024), device=_dev())
    y_static = torch.empty((1, 1024), device=_dev())
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
        ref, _, _ = B.stack_decode(stack, xs[i:i + 1].contiguous(), ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), i


@pytest.mark.parametrize("T", [1, 3])
def test_stack_timed_matches_plain(T):
    """The timed stack entry (launches held behind a stream gate, then run back
    to back) computes exactly what the plain entry computes, and times every
    kernel of the path."""
    dims = gen.LayerDims(1024, 256, n_routed=32, n_shared=1, top_k=6, wfmt="q4_1")
    devs = [_layer(dims, 45, layer=l)[1] for l in range(3)]
    stack = B.StackHandle(devs)
    x = gen.make_hidden(45, T, 1024, draw=7, device=_dev())
    ws = B.workspace(dims, T)
    ref, _, ritr = B.stack_decode(stack, x, ws=ws, trace=True)
    torch.cuda.synchronize()
    ref, ritr = ref.clone(), ritr.clone()
    for _ in range(2):
        y, itr, us = B.stack_decode_timed(stack, x, ws=ws, trace=True)
        assert torch.equal(y, ref) and torch.equal(itr, ritr)
        assert len(us) in (3, 4) and all(v > 0 for v in us.values()), us  # 4 on the general path


# --------------------------------------------------------------------------- small-batch path (2-8 tokens)

@pytest.mark.parametrize("dims,T", [
    (gen.LayerDims(2048, 512, wfmt="q4_1"), 2),
    (gen.LayerDims(2048, 512, wfmt="q4_1"), 5),
    (gen.LayerDims(2048, 512, wfmt="q4_1"), 8),
    (gen.LayerDims(512, 128, wfmt="bf16"), 3),
    (gen.LayerDims(2048, 1024, n_routed=32, n_shared=0, top_k=4, wfmt="nvfp4"), 4),
    (gen.LayerDims(4096, 512, n_routed=64, n_shared=2, top_k=6, wfmt="q4_1"), 7),
    # 9-16 tokens: two token groups in the down projection, two tokens per
    # selection wave
    (gen.LayerDims(2048, 512, wfmt="q4_1"), 9),
    (gen.LayerDims(2048, 512, wfmt="q4_1"), 16),
    (gen.LayerDims(2048, 512, wfmt="nvfp4"), 12),
    (gen.LayerDims(512, 128, wfmt="bf16"), 16),
    (gen.LayerDims(4096, 512, n_routed=64, n_shared=2, top_k=6, wfmt="q4_1"), 13),
    # 17-32 tokens: two router blocks per expert, four selection tokens per wave
    (gen.LayerDims(2048, 512, wfmt="q4_1"), 32),
    (gen.LayerDims(2048, 512, wfmt="nvfp4"), 21),
    (gen.LayerDims(4096, 512, n_routed=64, n_shared=2, top_k=6, wfmt="q4_1"), 27),
], ids=["q4_1-t2", "q4_1-t5", "q4_1-t8", "bf16-t3", "nvfp4-noshared-t4", "q4_1-upl2-2shared-t7", "q4_1-t9",
        "q4_1-t16", "nvfp4-t12", "bf16-t16", "q4_1-upl2-2shared-t13", "q4_1-t32", "nvfp4-t21",
        "q4_1-upl2-2shared-t27"])
def test_small_batch_path_shapes(dims, T):
    host, dl = _layer(dims, 46)
    x = gen.make_hidden(46, T, dims.d_model, draw=T)
    err, _, _ = _run_layer_case(host, dl, x, f"bn {dims} T={T}")
    assert err.max() <= FP32_PATH_TOL


def test_small_batch_given_routing_with_invalid_indices():
    dims = gen.LayerDims(2048, 512, n_routed=64, n_shared=1, top_k=6, wfmt="q4_1")
    host, dl = _layer(dims, 47)
    T = 4
    x = gen.make_hidden(47, T, 2048, draw=3)
    rng = np.random.default_rng(11)
    idx = np.stack([rng.choice(64, 6, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, 6)).astype(np.float32)
    idx[1, 2] = -1
    idx[3, 5] = 64  # out of range: selects nothing
    y = B.expert_ffn_q4(dims, x.to(_dev()), dl.experts, None, torch.from_numpy(idx).to(_dev()),
                        torch.from_numpy(w).to(_dev()))
    torch.cuda.synchronize()
    valid = (idx >= 0) & (idx < 64)
    # "select nothing" = a zero-weight term (adds an exact +0.0 in the oracle)
    oy = oracle.experts_given(host, x.double().numpy(), np.where(valid, idx, 0),
                              np.where(valid, w, 0.0).astype(np.float64))
    assert np.all(rel_l2(y.cpu().numpy(), oy) <= FP32_PATH_TOL)


@pytest.mark.parametrize("dims,T", [
    (gen.LayerDims(2048, 512, n_routed=64, n_shared=1, top_k=6, wfmt="q4_1"), 1),   # small-batch kernels at T = 1
    (gen.LayerDims(2048, 512, n_routed=64, n_shared=1, top_k=6, wfmt="nvfp4"), 4),  # small-batch kernels
    (gen.LayerDims(96, 160, n_routed=20, n_shared=2, top_k=3, wfmt="q4_1"), 3),     # general decode kernels
], ids=["q4_1-t1", "nvfp4-t4", "ragged-t3"])
def test_given_routing_repeated_and_invalid_indices(dims, T):
    """A repeated index contributes once per slot (its weights add up) and an
    index outside [0, n_routed) contributes nothing, on every decode path."""
    host, dl = _layer(dims, 49)
    x = gen.make_hidden(49, T, dims.d_model, draw=5)
    rng = np.random.default_rng(17)
    K, E = dims.top_k, dims.n_routed
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    idx[0, K - 1] = idx[0, 0]          # a repeat in the first and last slots
    if T > 1:
        idx[T - 1, 1] = idx[T - 1, 2]  # adjacent slots
        idx[T - 1, 0] = E              # out of range
    if K > 2:
        idx[0, 1] = -3
    y = B.expert_ffn_q4(dims, x.to(_dev()), dl.experts, dl.tensor_scale, torch.from_numpy(idx).to(_dev()),
                        torch.from_numpy(w).to(_dev()))
    torch.cuda.synchronize()
    valid = (idx >= 0) & (idx < E)
    oy = oracle.experts_given(host, x.double().numpy(), np.where(valid, idx, 0),
                              np.where(valid, w, 0.0).astype(np.float64))
    err = rel_l2(y.cpu().numpy(), oy)
    print(f"[given repeated] {dims} T={T} max rel-L2 {err.max():.3e}")
    assert np.all(err <= FP32_PATH_TOL), err


@pytest.mark.parametrize("T", [8, 16, 32])
def test_small_batch_deterministic(T):
    host, dl = _layer(gen.LayerDims(2048, 512, wfmt="q4_1"), 46)
    x = gen.make_hidden(46, T, 2048, draw=77).to(_dev())
    y1, i1, w1 = B.layer_forward(dl, x)
    y2, i2, w2 = B.layer_forward(dl, x)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(i1, i2) and torch.equal(w1, w2)


def test_stack_small_batch_teacher_forced():
    """3 tokens through 3 full-size NVFP4 layers (RMSNorm between layers on the device)."""
    dims = gen.LayerDims(2048, 512, wfmt="nvfp4")
    L, T = 3, 3
    hosts = [gen.make_layer(dims, cfg_id=48, layer=l) for l in range(L)]
    devs = [B.upload_layer(h, _dev()) for h in hosts]
    stack = B.StackHandle(devs)
    x0 = gen.make_hidden(48, T, 2048)
    y, ytr, itr = B.stack_decode(stack, x0.to(_dev()), trace=True)
    torch.cuda.synchronize()
    ytr, itr = ytr.cpu().numpy(), itr.cpu().numpy()
    x = x0.double().numpy()
    for l in range(L):
        oi, ow, ol, _ = oracle.layer_forward(hosts[l], x)
        check_routing(itr[l], None, ol, oi, ow, decode_band(x, _router64(hosts[l])) + 1e-5)
        _, _, _, oy = oracle.layer_forward(hosts[l], x, forced=itr[l])
        err = rel_l2(ytr[l], oy)
        print(f"[stack T={T}] layer {l} teacher-forced rel-L2 {err.max():.3e}")
        assert err.max() <= FP32_PATH_TOL
        x = np.stack([oracle.rmsnorm(ytr[l][t]) for t in range(T)])
