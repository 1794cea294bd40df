"""Benchmark of the sparse MoE decode layer on one MI355X.

Default workload: batch-1 decode of one fresh token per step through a stack
of 47 independent seeded MoE layers (d_model 2048, d_ff 512, 256 routed + 1
shared experts, top-6, q4_1 weights), RMS-normalised between layers.  The
23.7 GB stack is far larger than the 256 MB Infinity Cache, so every step
streams its experts from HBM.  One step = the whole stack for one token
(47 MoE-layer decodes); the reported value is MoE-layer decode tokens/s.

The step is captured once in a HIP graph (torch.cuda.CUDAGraph) that first
stages the next pre-generated token into the graph's input buffer, then
enqueues libmoe's stack decode; timing is HIP events on the replay stream.

Prints one JSON line.  Other workloads (NVFP4 batch 1 / batch 8 stacks, the
4096-token prefill) via --workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="stack_q4_1_b1",
                    choices=["stack_q4_1_b1", "stack_nvfp4_b1", "stack_nvfp4_b8", "prefill_q4_1"])
    ap.add_argument("--layers", type=int, default=47)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-layers", type=int, default=47, help="layers in the CPU baseline sample")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_stack(dims, cfg_id, n_layers, keep_host: bool):
    """Generate n_layers on the device, keep canonical host copies if asked, repack."""
    from sparse_moe_decode_route_amd import binding as B
    from sparse_moe_decode_route_amd import inputs as gen
    devs, hosts = [], []
    for l in range(n_layers):
        lay = gen.make_layer(dims, cfg_id=cfg_id, layer=l, device="cuda")
        if keep_host:
            hosts.append(gen.Layer(dims, lay.router.cpu(), None, lay.experts.cpu(),
                                   None if lay.tensor_scale is None else lay.tensor_scale.cpu()))
        packed = torch.empty_like(lay.experts)
        B.repack_weights(dims, lay.experts, packed, dims.n_experts)
        torch.cuda.synchronize()
        devs.append(B.DeviceLayer(dims, lay.router, None, packed, lay.tensor_scale))
        del lay
        if (l + 1) % 8 == 0 or l + 1 == n_layers:
            log(f"generated {l + 1}/{n_layers} layers")
    return devs, hosts


def union_bytes(idx_trace: np.ndarray, dims, expert_bytes: int) -> float:
    """Mean over layers of distinct experts touched (routed union + shared) times expert bytes."""
    tot = 0
    for l in range(idx_trace.shape[0]):
        tot += len(set(idx_trace[l].reshape(-1).tolist())) + dims.n_shared
    return tot / idx_trace.shape[0] * expert_bytes


def bench_stack(args, wfmt: str, T: int):
    from sparse_moe_decode_route_amd import binding as B
    from sparse_moe_decode_route_amd import inputs as gen
    cfg_id = 3 if wfmt == "q4_1" else 4
    dims = gen.LayerDims(2048, 512, wfmt=wfmt)
    L = args.layers
    want_cpu = (not args.no_cpu) and T == 1
    t0 = time.time()
    devs, hosts = build_stack(dims, cfg_id, L, keep_host=want_cpu)
    log(f"stack of {L} layers ready in {time.time() - t0:.1f}s")
    stack = B.StackHandle(devs)
    eb = B.packed_expert_bytes(dims)
    n_tok = args.warmup + args.steps + 1
    xs = gen.make_hidden(cfg_id, n_tok * T, 2048, draw=777, device="cuda").reshape(n_tok, T, 2048)
    x_static = torch.empty((T, 2048), device="cuda")
    y_static = torch.empty((T, 2048), device="cuda")
    ctr = torch.zeros(1, dtype=torch.long, device="cuda")
    ws = B.workspace(dims, T)

    # routing statistics (expert union per layer) from an eager traced run of the first token
    y0, ytr, itr = B.stack_decode(stack, xs[0].contiguous(), ws=ws, trace=True)
    torch.cuda.synchronize()
    itr_np = itr.cpu().numpy()
    bytes_per_layer = union_bytes(itr_np, dims, eb)

    def step():
        x_static.copy_(torch.index_select(xs, 0, ctr).reshape(T, 2048))
        ctr.add_(1)
        B.stack_decode(stack, x_static, ws=ws, y=y_static)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm the allocator / code objects outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    ctr.zero_()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    layer_tok_s = L * T / (ms * 1e-3)
    # the graph replayed the same arithmetic as the eager call: check the last replay against eager
    last = int(ctr.item()) - 1
    y_eager, _, _ = B.stack_decode(stack, xs[last].contiguous(), ws=ws)
    torch.cuda.synchronize()
    graph_matches_eager = bool(torch.equal(y_eager, y_static))

    router_b = dims.n_routed * dims.d_model * 2
    algo_bytes_step = L * (bytes_per_layer + router_b)
    achieved = algo_bytes_step / (ms * 1e-3) / 1e9
    expert_gbs = L * bytes_per_layer / (ms * 1e-3) / 1e9
    out = dict(
        metric="MoE-layer decode tokens/s + achieved HBM GB/s (% of peak), 4-bit, batch 1",
        value=round(layer_tok_s, 1), unit="MoE-layer tok/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms, 5), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="f32", data="synthetic",
        config=dict(workload=f"moe_decode_{wfmt}_b{T}: d_model 2048, d_ff 512, 256 routed + 1 shared, top-6, "
                             f"{wfmt} experts, {L} independent layers chained with RMSNorm, batch {T}, one fresh "
                             f"N(0,1) token per step", global_batch=T, seq_len=1, parallelism="single-gpu",
                    layers=L, stack_tok_s=round(T / (ms * 1e-3), 2),
                    expert_bytes_per_layer=round(bytes_per_layer), router_bytes_per_layer=router_b,
                    expert_gbs=round(expert_gbs, 1), expert_frac_of_peak=round(expert_gbs / HBM_PEAK_GBS, 4),
                    graph_matches_eager=graph_matches_eager),
        roofline=dict(bound="hbm", kernel="moe_stack_decode (all kernels of one step)", achieved=round(achieved, 1),
                      peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4), traffic=None),
    )
    if want_cpu:
        out["cpu_baseline"] = cpu_baseline_stack(args, hosts, xs, dims, stack, ws)
    return out


def cpu_baseline_stack(args, hosts, xs, dims, stack, ws):
    """The oracle (fp64 plain C, one thread) on one token through the first cpu_layers layers."""
    import oracle
    from sparse_moe_decode_route_amd import binding as B
    n = min(args.cpu_layers, len(hosts))
    x0 = xs[0].cpu().double().numpy()
    oracle.lib()
    t0 = time.time()
    y, ytr, itr = oracle.stack_forward(hosts[:n], x0)
    dt = time.time() - t0
    # parity of this sample: GPU stack over the same layers and token
    sub = B.StackHandle(stack.layers[:n])
    yg, _, ig = B.stack_decode(sub, xs[0].contiguous(), ws=ws, trace=True)
    torch.cuda.synchronize()
    same_route = bool(np.array_equal(ig.cpu().numpy(), itr))
    yg = yg.cpu().double().numpy()
    err = float(np.linalg.norm(yg - y) / np.linalg.norm(y)) if same_route else None
    return dict(value=round(n / dt, 3), unit="MoE-layer tok/s", cores=1, kind="oracle",
                sample=f"1 token through {n} q4_1 layers (d_model 2048, d_ff 512, 256+1 experts), fp64 C, "
                       f"one thread, {dt:.1f}s",
                gpu_vs_oracle=dict(same_routing_all_layers=same_route, rel_l2_final=err))


def bench_prefill(args):
    raise SystemExit("prefill workload not built yet")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps(dict(error=f"this build runs on one GPU only; --gpus {args.gpus} is not supported")))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps(dict(error="no ROCm device visible")))
        sys.exit(2)
    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    from sparse_moe_decode_route_amd import binding as B
    B.lib()  # fails loudly if libmoe.so is missing
    if args.workload == "stack_q4_1_b1":
        out = bench_stack(args, "q4_1", 1)
    elif args.workload == "stack_nvfp4_b1":
        out = bench_stack(args, "nvfp4", 1)
    elif args.workload == "stack_nvfp4_b8":
        out = bench_stack(args, "nvfp4", 8)
    else:
        out = bench_prefill(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
