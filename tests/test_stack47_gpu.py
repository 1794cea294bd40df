"""GPU parity of the benchmarked workload itself: one token through the stack
of 47 independent q4_1 layers at d_model 2048, d_ff 512, 256 routed + 1
shared experts, top-6 (cfg 3: the same 47 layers the benchmark generates,
and an N(0, 1) token drawn like its tokens), RMS-normalised between layers.

Every layer is checked teacher-forced: the oracle takes the GPU's own
normalised output of the previous layer as input, must select the same
experts outside the fp32 rounding band, and must give the GPU's layer output
within relative L2 2e-3 (and the fp32-path guard).  A free-running oracle
chain (fp64 from x_0) runs beside it: while its selections equal the GPU's,
the two chains' outputs are compared; at the first layer where a selection
differs, the difference must be explained by the drift between the chains'
inputs (helpers.check_chain_divergence), since 47 random layers amplify the
fp32/fp64 difference of every layer."""
import numpy as np
import pytest
import torch

import oracle
from sparse_moe_decode_route_amd import binding as B
from sparse_moe_decode_route_amd import inputs as gen
from tests.helpers import REL_L2_TOL, check_chain_divergence, check_routing, rel_l2, router_band

pytestmark = pytest.mark.gpu

FP32_PATH_TOL = 5e-5
N_LAYERS = 47
CFG = 3
TOKEN_DRAW = 777  # the draw of the benchmark's token stream


def _router64(host):
    return oracle.bf16_array(host.router.numpy().view(np.uint16))


def test_stack47_q4_1_every_layer_and_chain():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    dims = gen.WORKLOADS["c3_stack47_q4_1"]["dims"]
    canon, devs = [], []
    for l in range(N_LAYERS):
        lay = gen.make_layer(dims, cfg_id=CFG, layer=l, device="cuda")
        packed = torch.empty_like(lay.experts)
        B.repack_weights(dims, lay.experts, packed, dims.n_experts)
        devs.append(B.DeviceLayer(dims, lay.router, None, packed, lay.tensor_scale))
        canon.append(lay)  # canonical bytes stay on the device; one layer at a time goes to the host
    torch.cuda.synchronize()
    stack = B.StackHandle(devs)
    x0 = gen.make_hidden(CFG, 1, 2048, draw=TOKEN_DRAW, device="cuda")
    y, ytr, itr = B.stack_decode(stack, x0, trace=True)
    torch.cuda.synchronize()
    y, ytr, itr = y.cpu().numpy(), ytr.cpu().numpy(), itr.cpu().numpy()
    assert np.array_equal(y, ytr[-1])
    x_tf = x0.cpu().double().numpy()          # teacher-forced input: the GPU's own chain
    x_fr = x_tf.copy()                        # free-running oracle chain
    diverged = None
    worst = 0.0
    for l in range(N_LAYERS):
        lay = canon[l]
        host = gen.Layer(dims, lay.router.cpu(), None, lay.experts.cpu(), None)
        oi, ow, ol, _ = oracle.layer_forward(host, x_tf)
        band = router_band(x_tf, _router64(host)) + 1e-5
        check_routing(itr[l], None, ol, oi, ow, band)
        _, _, _, oy = oracle.layer_forward(host, x_tf, forced=itr[l])
        err = float(rel_l2(ytr[l], oy).max())
        worst = max(worst, err)
        assert err <= REL_L2_TOL and err <= FP32_PATH_TOL, (l, err)
        if diverged is None:
            fi, _, _, fy = oracle.layer_forward(host, x_fr)
            if not np.array_equal(np.sort(fi, axis=1), np.sort(itr[l], axis=1)):
                gap, drift = check_chain_divergence(oracle, host, x_tf, x_fr, float(band[0]), dims.top_k)
                diverged = l
                print(f"[stack47] chains select differently first at layer {l}: oracle gap {gap:.3e}, "
                      f"logit drift {drift:.3e}")
            else:
                x_fr = oracle.rmsnorm(fy[0])[None]
        x_tf = oracle.rmsnorm(ytr[l][0])[None]
        del host
    if diverged is None:
        e2e = float(rel_l2(y, fy).max())
        print(f"[stack47] same selections in all {N_LAYERS} layers, end-to-end rel-L2 {e2e:.3e}")
        assert e2e <= REL_L2_TOL
    print(f"[stack47] worst teacher-forced rel-L2 over {N_LAYERS} layers {worst:.3e}")
