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
                    choices=["stack_q4_1_b1", "stack_nvfp4_b1", "stack_nvfp4_b8", "prefill_q4_1", "prefill_nvfp4", "sweep_q4_1",
                             "lm_head_q4_1", "lm_head_nvfp4", "lm_head_bf16", "attn_swa", "attn_full128k"])
    ap.add_argument("--layers", type=int, default=47)
    ap.add_argument("--decode-path", default="kernels", choices=["kernels", "persistent", "xcd"],
                    help="batch-1 decode path: three kernels per layer, the persistent kernel, or one kernel per "
                         "layer with one expert per XCD (the last two where built)")
    ap.add_argument("--lm-tokens", type=int, default=1, help="tokens per output-layer call (1..8)")
    ap.add_argument("--lm-cpu-rows", type=int, default=146_484, help="vocabulary rows in the CPU baseline sample")
    ap.add_argument("--lm-cpu-seconds", type=float, default=10.0, help="minimum CPU baseline time (whole passes)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-layers", type=int, default=47, help="layers in the CPU baseline sample")
    ap.add_argument("--cpu-tokens", type=int, default=4, help="tokens in the one-thread CPU baseline sample")
    ap.add_argument("--prefill-cpu-tokens", type=int, default=1024, help="tokens in the prefill CPU baseline sample")
    ap.add_argument("--timed-calls", type=int, default=20,
                    help="eager stack calls with per-kernel dispatch events (the roofline's kernel timing)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy five times (reference kernel for HBM counters)")
    ap.add_argument("--rocprof-summary", metavar="CSV",
                    help="summarise a rocprofv3 kernel_trace.csv or counter_collection.csv of this script per "
                         "kernel, split at the first timed call (needs no GPU), and exit")
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


def source_digest(files=("moe_decode_b1.hip", "moe_decode.hip", "moe_device.h", "moe_internal.h")) -> str:
    """Digest of kernel sources (default: the decode kernels'), comments and
    whitespace left out: stored counter readings apply only to the code they
    were taken on."""
    import hashlib
    import re
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_moe_decode_route_amd", "csrc")
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(root, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


BN_SOURCES = ("moe_decode_bn.hip", "moe_device.h", "moe_internal.h")
PREFILL_SOURCES = ("moe_prefill.hip", "moe_prefill.h", "moe_device.h", "moe_internal.h")
PERSIST_SOURCES = ("moe_stack_persist.hip", "moe_persist.h", "moe_device.h", "moe_internal.h")
XCD_SOURCES = ("moe_decode_xcd.hip", "moe_xcd.h", "moe_device.h", "moe_internal.h")
PS_LAYERS_PER_LAUNCH = 64  # layers per persistent-kernel launch (the library's limit)
LM_HEAD_SOURCES = ("moe_lm_head.hip", "moe_device.h", "moe_internal.h")
ATTN_SOURCES = ("moe_attn.hip", "moe_device.h", "moe_internal.h")


# HBM traffic per launch read from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this
# script (one run per counter), each scaled by the same counter's reading for a
# plain device copy of known size; keyed by (workload, kernel) and valid only for
# the kernel source digest it was taken on.
_FETCH_SCALE = 262144.0 / 131083.5  # 256 MiB device copy: true KiB read / FETCH_SIZE KiB
_WRITE_SCALE = 262144.0 / 262144.0  # same copy: true KiB written / WRITE_SIZE KiB
# Matrix-core counters of the fused prefill GEMM kernel (gate/up and down in
# one dispatch), per dispatch, from a rocprofv3 --pmc run of this script
# (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, SQ_INSTS_VALU_MFMA_MOPS_F16,
# SQ_BUSY_CYCLES); valid only for the source digest they were taken on.  The SQ
# counters sum over the chip's 1024 SIMDs (256 CUs x 4) and GRBM_GUI_ACTIVE over
# its 8 XCDs, so utilisation = (busy / 1024) / (active / 8); one MOP is 512 FLOPs
# of work issued to the matrix cores.
PREFILL_MFMA_COUNTERS = dict(
    source_digest="b18198ac95672289",
    # q4_1 layer: means per dispatch over the 4 timed dispatches of one run
    pf_ffn=dict(GRBM_GUI_ACTIVE=3441111.75, SQ_VALU_MFMA_BUSY_CYCLES=195428352.0,
                SQ_INSTS_VALU_MFMA_MOPS_F16=390856704.0, SQ_BUSY_CYCLES=12348378.25, duration_us=219.85),
)


def prefill_mfma_counters(flops: dict):
    """Counter-based MFMA utilisation of the prefill GEMM kernels ({kernel:
    algorithmic FLOPs per dispatch}), or None when the stored counters were
    taken on other kernel sources."""
    c = PREFILL_MFMA_COUNTERS
    if c is None or c["source_digest"] != source_digest(PREFILL_SOURCES):
        return None
    out = {}
    for k, fl in flops.items():
        v = c.get(k)
        if v is None:
            continue
        active = v["GRBM_GUI_ACTIVE"] / 8.0
        out[k] = dict(mfma_busy_frac=round(v["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024.0 / active, 4),
                      issued_flops=round(v["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512),
                      algorithmic_flops=fl, padding_overhead=round(v["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512 / fl - 1, 4),
                      clock_ghz=round(active / (v["duration_us"] * 1e3), 3), gui_active_cycles_per_xcd=round(active),
                      counters=v)
    return out or None


def _traffic(digest: str, fetch_kib: float, write_kib: float) -> dict:
    """A kernel's stored counter readings (KiB per dispatch, mean over the run) as bytes."""
    return dict(source_digest=digest, fetch_bytes=round(fetch_kib * _FETCH_SCALE * 1024),
                write_bytes=round(write_kib * _WRITE_SCALE * 1024))


COUNTER_TRAFFIC = {
    # batch-1 q4_1 stack
    ("stack_q4_1_b1", "b1_route"): _traffic("7d4ce39bbc3c9388", 563.0227, 16.0),
    ("stack_q4_1_b1", "b1_topk_gateup"): _traffic("7d4ce39bbc3c9388", 4595.5831, 14.6691),
    ("stack_q4_1_b1", "b1_down"): _traffic("7d4ce39bbc3c9388", 2325.5868, 8.0),
    # batch-8 NVFP4 stack
    ("stack_nvfp4_b8", "bn_router"): _traffic("57c1d2057ded3856", 788.51, 64.0),
    ("stack_nvfp4_b8", "bn_gateup"): _traffic("57c1d2057ded3856", 26673.5191, 112.4278),
    ("stack_nvfp4_b8", "bn_down"): _traffic("57c1d2057ded3856", 13520.6781, 64.0),
    # 4096-token prefill, q4_1 and NVFP4
    # (both GEMMs in one dispatch)
    ("prefill_q4_1", "pf_ffn"): _traffic("b18198ac95672289", 219437.6, 143400.2),
    ("prefill_nvfp4", "pf_ffn"): _traffic("b18198ac95672289", 207707.6, 143401.8),
    # q4_1 output layer, 1 token
    ("lm_head_q4_1_t1", "lm_head_kernel"): _traffic("c3b94d4e2367e0b5", 91654.112, 572.2188),
    # full-attention layer at 128k positions
    ("attn_full128k", "attn_chunk"): _traffic("70abf60267263961", 131362.8772, 2306.0),
}


def kernel_algo_bytes(dims, T: int, routed_union: float):
    """Algorithmic bytes one launch of each decode kernel must move.

    Weights: packed bytes of the matrices the kernel reads (router bf16 in the
    first kernel; gate and up of the routed union and the shared experts in
    the batch-1 gate/up kernel, of the shared experts in the general path's
    first kernel; down of every active expert in the last).  Activations:
    fp32 x in, logits, h and y as produced and consumed between kernels."""
    from sparse_moe_decode_route_amd import inputs as gen
    D, F, E, S = dims.d_model, dims.d_ff, dims.n_routed, dims.n_shared
    gu = gen.matrix_bytes(F, D, dims.wfmt)
    dn = gen.matrix_bytes(D, F, dims.wfmt)
    U = routed_union
    a = E * D * 2 + S * 2 * gu + T * D * 4 + T * E * 4 + S * T * F * 4
    b = T * E * 4 + U * 2 * gu + T * D * 4 + U * T * F * 4
    b1_a = E * D * 2 + T * D * 4 + T * E * 4
    b1_b = T * E * 4 + (U + S) * 2 * gu + T * D * 4 + (U + S) * T * F * 4
    c = (U + S) * dn + (U + S) * T * F * 4 + T * D * 4
    K = dims.top_k
    pairs = T * K + S * T  # (expert, token) rows of h
    bn = {"bn_router": E * D * 2 + T * D * 4 + T * E * 4,
          "bn_gateup": (U + S) * 2 * gu + T * D * 4 + T * E * 4 + pairs * F * 4,
          "bn_down": (U + S) * dn + pairs * F * 4 + T * D * 4 + T * E * 4}
    return {"b1_route": b1_a, "b1_topk_gateup": b1_b, "b1_down": c,
            "phase_a_kernel": a, "select_kernel": T * E * 4, "gateup_kernel": b, "down_kernel": c, **bn}


def time_kernels(args, stack, xs, ws, dims, T):
    """Per-kernel mean dispatch durations over --timed-calls eager stack calls (fresh token each)."""
    from sparse_moe_decode_route_amd import binding as B
    n = max(1, args.timed_calls)
    tot, unions = {}, []
    for i in range(2):  # untimed: the eager, event-bracketed path warms up first
        B.stack_decode_timed(stack, xs[i % xs.shape[0]].contiguous(), ws=ws)
    for i in range(n):
        _, itr, us = B.stack_decode_timed(stack, xs[i % xs.shape[0]].contiguous(), ws=ws, trace=True)
        for k, v in us.items():
            tot[k] = tot.get(k, 0.0) + v
        it = itr.cpu().numpy()
        unions.append(np.mean([len(set(it[l].reshape(-1).tolist())) for l in range(it.shape[0])]))
    return {k: v / n for k, v in tot.items()}, float(np.mean(unions))


def roofline(workload, dims, T, L, kernel_us, routed_union):
    if "ps_stack" in kernel_us:
        return roofline_persistent(workload, dims, L, kernel_us, routed_union)
    if "xl_layer" in kernel_us:
        return roofline_xcd(workload, dims, kernel_us, routed_union)
    algo = kernel_algo_bytes(dims, T, routed_union)
    dom = max(kernel_us, key=lambda k: kernel_us[k])
    us = kernel_us[dom]
    achieved = algo[dom] / (us * 1e-6) / 1e9
    def traffic_of(k):
        tr = COUNTER_TRAFFIC.get((workload, k))
        digest = source_digest(BN_SOURCES) if k.startswith("bn_") else source_digest()
        return tr["fetch_bytes"] + tr["write_bytes"] if tr is not None and tr["source_digest"] == digest else None

    traffic = traffic_of(dom)
    kernels = {k: dict(us_per_launch=round(v, 3), algo_bytes_per_launch=round(algo[k]),
                       gbs=round(algo[k] / (v * 1e-6) / 1e9, 1), traffic=traffic_of(k))
               for k, v in kernel_us.items()}
    return dict(bound="hbm", kernel=dom, achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                algo_bytes_per_launch=round(algo[dom]), us_per_launch=round(us, 3),
                timing="HIP dispatch events (hipExtLaunchKernelGGL) on the launch stream, "
                       "mean over every launch of the timed calls; each call's launches are "
                       "enqueued behind a stream hold and then run back to back, as in a graph replay",
                per_kernel=kernels)


def roofline_persistent(workload, dims, L, kernel_us, routed_union):
    """The persistent kernel runs the whole batch-1 step: its algorithmic bytes
    per launch are every layer's router, shared expert and routed union (the
    layer's packed weights the method must read), the input token and the
    output row; the launch time is its dispatch events' duration."""
    from sparse_moe_decode_route_amd import inputs as gen
    D, F, E, S = dims.d_model, dims.d_ff, dims.n_routed, dims.n_shared
    eb = 2 * gen.matrix_bytes(F, D, dims.wfmt) + gen.matrix_bytes(D, F, dims.wfmt)
    per_layer = E * D * 2 + (routed_union + S) * eb
    launches = -(-L // PS_LAYERS_PER_LAUNCH)
    algo = L * per_layer / launches + (D * 4 + D * 4) / launches
    us = kernel_us["ps_stack"] * L / launches
    achieved = algo / (us * 1e-6) / 1e9
    tr = COUNTER_TRAFFIC.get((workload, "ps_stack"))
    traffic = None
    if tr is not None and tr["source_digest"] == source_digest(PERSIST_SOURCES):
        traffic = tr["fetch_bytes"] + tr["write_bytes"]
    return dict(bound="hbm", kernel="ps_stack", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic, algo_bytes_per_launch=round(algo),
                us_per_launch=round(us, 3), layers_per_launch=L // launches, launches_per_step=launches,
                us_per_layer=round(kernel_us["ps_stack"], 4), clear_us_per_step=round(kernel_us["ps_clear"], 3),
                timing="HIP dispatch events (hipExtLaunchKernelGGL) on the launch stream, mean over the eager "
                       "timed calls",
                per_kernel={k: dict(us=round(v, 3)) for k, v in kernel_us.items()})


def roofline_xcd(workload, dims, kernel_us, routed_union):
    """One kernel per layer (one expert per XCD): its algorithmic bytes per
    launch are the layer's router, shared expert and routed union, the previous
    layer's 8 partial outputs it adds and its own 8 partial outputs."""
    from sparse_moe_decode_route_amd import inputs as gen
    D, F, E, S = dims.d_model, dims.d_ff, dims.n_routed, dims.n_shared
    eb = 2 * gen.matrix_bytes(F, D, dims.wfmt) + gen.matrix_bytes(D, F, dims.wfmt)
    algo = E * D * 2 + (routed_union + S) * eb + 2 * 8 * D * 4
    us = kernel_us["xl_layer"]
    achieved = algo / (us * 1e-6) / 1e9
    tr = COUNTER_TRAFFIC.get((workload, "xl_layer"))
    traffic = None
    if tr is not None and tr["source_digest"] == source_digest(XCD_SOURCES):
        traffic = tr["fetch_bytes"] + tr["write_bytes"]
    return dict(bound="hbm", kernel="xl_layer", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic, algo_bytes_per_launch=round(algo),
                us_per_launch=round(us, 3),
                timing="HIP dispatch events (hipExtLaunchKernelGGL) on the launch stream, mean over every launch "
                       "of the timed calls; each call's launches are enqueued behind a stream hold and then run "
                       "back to back, as in a graph replay",
                per_kernel={k: dict(us_per_launch=round(v, 3)) for k, v in kernel_us.items()})


def single_layer_times(args, dev, xs, ws, T, n_calls=47):
    """One layer (the stack's first) called n_calls times back to back in one HIP
    graph, each call on its own (not chained), per-call mean over the replays:
    with a fresh token per call (the routed experts mostly come from HBM: the
    layer's 506 MB exceed the 256 MB Infinity Cache), and warm, with the same
    token on every call (no flush: its 7 experts' 13.8 MB and the router stay
    on chip after the first call)."""
    from sparse_moe_decode_route_amd import binding as B
    one = B.StackHandle([dev])
    y_static = torch.empty((T, 2048), device="cuda")
    out = {}
    for name, fresh in (("fresh_token_us", True), ("warm_same_token_us", False)):
        xin = [xs[i % xs.shape[0] if fresh else 0].contiguous() for i in range(n_calls)]

        def calls():
            for x in xin:
                B.stack_decode(one, x, ws=ws, y=y_static)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            calls()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) * 1e3 / (reps * n_calls), 3)
    out["timing"] = (f"{n_calls} calls of one layer (not chained) in one HIP graph, per-call mean over 20 "
                     "replays")
    return out


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
    n_tok = max(args.warmup + args.steps + 1, 2 * cpu_workers() + 1)
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
    # one event between consecutive replays: the K step times, and their sum
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        g.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    step_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    layer_tok_s = L * T / (ms * 1e-3)
    # the graph replayed the same arithmetic as the eager call: check the last replay against eager
    last = int(ctr.item()) - 1
    y_eager, _, _ = B.stack_decode(stack, xs[last].contiguous(), ws=ws)
    torch.cuda.synchronize()
    graph_matches_eager = bool(torch.equal(y_eager, y_static))

    single = single_layer_times(args, devs[0], xs, ws, T) if T == 1 else None

    router_b = dims.n_routed * dims.d_model * 2
    algo_bytes_step = L * (bytes_per_layer + router_b)
    step_gbs = algo_bytes_step / (ms * 1e-3) / 1e9
    expert_gbs = L * bytes_per_layer / (ms * 1e-3) / 1e9
    workload = f"stack_{wfmt}_b{T}"
    kernel_us, routed_union = time_kernels(args, stack, xs, ws, dims, T)
    log(f"per-kernel us: {kernel_us}, routed union {routed_union:.2f}")
    pct = {f"p{q}": round(float(np.percentile(step_ms, q)), 5) for q in (10, 50, 90)}
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
                    step_gbs_incl_router=round(step_gbs, 1), graph_matches_eager=graph_matches_eager,
                    step_ms_percentiles=pct, single_layer=single,
                    decode_path=("persistent" if "ps_stack" in kernel_us else
                                 "xcd" if "xl_layer" in kernel_us else "kernels"),
                    kernel_source_digest=source_digest()),
        roofline=roofline(workload, dims, T, L, kernel_us, routed_union),
    )
    if want_cpu:
        out["cpu_baseline"] = cpu_baseline_stack(args, hosts, xs, dims, stack, ws)
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers() -> int:
    """Host threads for the all-core oracle timing: the host's cores, at most
    16 (a GPU's share of a shared host)."""
    return max(1, min(16, os.cpu_count() or 1))


def _oracle_chains(hosts, xa):
    """One fp64 oracle chain per token (rows of xa) through all hosts' layers."""
    import oracle
    return oracle.stack_forward(hosts, xa)


def cpu_baseline_stack(args, hosts, xs, dims, stack, ws):
    """The oracle (fp64 plain C) on tokens through the stack's layers, each token
    its own chain: one thread, then every worker thread running chains at once
    (the oracle is C called through ctypes, which releases the interpreter
    lock).  Also compares the GPU chain of the first token with the oracle's."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from sparse_moe_decode_route_amd import binding as B
    n = min(args.cpu_layers, len(hosts))
    nt = max(1, args.cpu_tokens)
    W = cpu_workers()
    xa_all = xs[:max(nt, 2 * W)].reshape(-1, dims.d_model).cpu().double().numpy()
    oracle.lib()
    # one thread
    xa = xa_all[:nt]
    t0 = time.time()
    y_all, ytr_all, itr_all = _oracle_chains(hosts[:n], xa)
    dt1 = time.time() - t0
    # all workers: two chains per worker, one chain per call
    xw = xa_all[:2 * W]
    t0 = time.time()
    with ThreadPoolExecutor(max_workers=W) as ex:
        list(ex.map(lambda i: _oracle_chains(hosts[:n], xw[i:i + 1]), range(len(xw))))
    dtw = time.time() - t0
    # parity of the first token's chain: GPU stack over the same layers and token, end to
    # end, and at the first layer whose selection differs, the oracle's fp64 logit gap
    # between the k-th and (k+1)-th expert on the GPU's own input to that layer
    x0 = xa[:1]
    y, ytr, itr = y_all[:1], ytr_all[:, :1], itr_all[:, :1]
    sub = B.StackHandle(stack.layers[:n])
    yg, ytr_g, ig = B.stack_decode(sub, xs[0].contiguous(), ws=ws, trace=True)
    torch.cuda.synchronize()
    ig = ig.cpu().numpy()
    same = [bool(np.array_equal(np.sort(ig[l], axis=-1), np.sort(itr[l], axis=-1))) for l in range(n)]
    first_diff = next((l for l in range(n) if not same[l]), None)
    yg = yg.cpu().double().numpy()
    err = float(np.linalg.norm(yg - y) / np.linalg.norm(y)) if first_diff is None else None
    gap, tf_match = None, None
    ytr_g = ytr_g.cpu().double().numpy()
    # relative difference of the two chains' layer outputs (fp32 GPU vs fp64 oracle): how far
    # the hidden states have drifted apart by the time a selection differs
    drift = [float(np.linalg.norm(ytr_g[l] - ytr[l]) / np.linalg.norm(ytr[l])) for l in range(n)]
    if first_diff is not None:
        xin = x0 if first_diff == 0 else oracle.rmsnorm(ytr_g[first_diff - 1])
        oi, _, lg, _ = oracle.layer_forward(hosts[first_diff], xin)
        srt = np.sort(lg[0])[::-1]
        gap = float(srt[dims.top_k - 1] - srt[dims.top_k])
        tf_match = bool(np.array_equal(np.sort(oi[0]), np.sort(ig[first_diff][0])))
    return dict(value=round(n * len(xw) / dtw, 3), unit="MoE-layer tok/s", cores=W, kind="oracle",
                sample=f"{len(xw)} tokens (independent chains, one per call) through {n} {dims.wfmt} layers "
                       f"(d_model 2048, d_ff 512, 256+1 experts), fp64 C, {W} threads, {dtw:.1f}s",
                cpu_model=cpu_model(), os_cpu_count=os.cpu_count(),
                single_thread=dict(value=round(n * nt / dt1, 3), cores=1,
                                   sample=f"{nt} tokens through {n} layers, one thread, {dt1:.1f}s"),
                gpu_vs_oracle=dict(layers_same_routing=int(sum(same)), layers=n, first_divergent_layer=first_diff,
                                   oracle_topk_gap_at_divergence=gap,
                                   teacher_forced_selection_matches_at_divergence=tf_match,
                                   hidden_drift_by_layer=[float(f"{v:.2e}") for v in drift[:(first_diff or n) + 1]],
                                   rel_l2_final=err))


def bench_prefill(args, wfmt="q4_1"):
    """4096 bf16 tokens through one 4-bit layer (q4_1, or the same layer in
    NVFP4) with a Zipf(1.1) router prior."""
    from sparse_moe_decode_route_amd import binding as B
    from sparse_moe_decode_route_amd import inputs as gen
    dims = gen.LayerDims(2048, 512, wfmt=wfmt)
    T = 4096
    lay = gen.make_layer(dims, cfg_id=5, layer=0, zipf_s=1.1, device="cuda")
    packed = torch.empty_like(lay.experts)
    B.repack_weights(dims, lay.experts, packed, dims.n_experts)
    torch.cuda.synchronize()
    ts = lay.tensor_scale if wfmt == "nvfp4" else None
    dev = B.DeviceLayer(dims, lay.router, lay.router_bias, packed, ts)
    host = None if args.no_cpu else gen.Layer(dims, lay.router.cpu(), lay.router_bias.cpu(), lay.experts.cpu(),
                                               None if ts is None else ts.cpu())
    del lay
    x = gen.to_bf16(gen.make_hidden(5, T, 2048, draw=0, device="cuda"))
    ws = B.workspace(dims, T)
    y = torch.empty((T, 2048), dtype=torch.float32, device="cuda")
    _, idx, _ = B.layer_forward(dev, x, ws=ws, y=y, prefill=True)
    torch.cuda.synchronize()
    loads = np.bincount(idx.cpu().numpy().reshape(-1), minlength=dims.n_routed)
    for _ in range(args.warmup):
        B.layer_forward(dev, x, ws=ws, y=y, want_routing=False, prefill=True)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # eager launches (host launch cost between the 7 kernels included), for context
    ev0.record()
    for _ in range(args.steps):
        B.layer_forward(dev, x, ws=ws, y=y, want_routing=False, prefill=True)
    ev1.record()
    torch.cuda.synchronize()
    ms_eager = ev0.elapsed_time(ev1) / args.steps
    y_eager = y.clone()
    # the timed step: one layer forward captured in a HIP graph and replayed
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.layer_forward(dev, x, ws=ws, y=y, want_routing=False, prefill=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.layer_forward(dev, x, ws=ws, y=y, want_routing=False, prefill=True)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    graph_matches_eager = bool(torch.equal(y, y_eager))
    # per-kernel dispatch timings
    n_timed = max(1, min(args.timed_calls, 20))
    tot = {}
    for _ in range(n_timed):
        _, us = B.layer_forward_prefill_timed(dev, x, ws=ws, y=y)
        for k, v in us.items():
            tot[k] = tot.get(k, 0.0) + v
    kus = {k: v / n_timed for k, v in tot.items()}
    log(f"prefill per-kernel us: {kus}")
    D, F, E, S, K = dims.d_model, dims.d_ff, dims.n_routed, dims.n_shared, dims.top_k
    rows = T * (K + S)
    fl_gu = rows * 2 * F * D * 2
    fl_dn = rows * D * F * 2
    fl_rt = 2 * T * E * D
    fl_all = fl_gu + fl_dn + fl_rt
    # kernels that did not run report -1 (the down GEMM when it runs fused
    # with the gate/up GEMM in one dispatch, pf_ffn)
    kus = {k: v for k, v in kus.items() if v > 0}
    fused = "pf_ffn" in kus
    dom = "pf_ffn" if fused else "pf_gemm_gateup"
    fl_dom = fl_gu + fl_dn if fused else fl_gu
    ach = fl_dom / (kus[dom] * 1e-6) / 1e12
    def pf_traffic_of(k):
        tr = COUNTER_TRAFFIC.get((f"prefill_{wfmt}", k))
        return (tr["fetch_bytes"] + tr["write_bytes"]
                if tr is not None and tr["source_digest"] == source_digest(PREFILL_SOURCES) else None)

    pf_traffic = pf_traffic_of(dom)
    per_kernel = {k: dict(us_per_launch=round(v, 2)) for k, v in kus.items()}
    per_kernel[dom]["tflops"] = round(ach, 1)
    if not fused:
        per_kernel["pf_gemm_down"]["traffic"] = pf_traffic_of("pf_gemm_down")
        per_kernel["pf_gemm_down"]["tflops"] = round(fl_dn / (kus["pf_gemm_down"] * 1e-6) / 1e12, 1)
    rname = "pf_router_gemm" if "pf_router_gemm" in kus else "pf_logits"
    per_kernel[rname]["tflops"] = round(fl_rt / (kus[rname] * 1e-6) / 1e12, 1)
    cpu = None if host is None else cpu_baseline_prefill(args, host, x)
    return dict(
        metric="MoE-layer prefill tokens/s (grouped GEMM on MFMA), 4-bit weights",
        value=round(T / (ms * 1e-3), 1), unit="tok/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f16",
        data="synthetic",
        config=dict(workload=f"moe_prefill_{wfmt}_t4096: 4096 bf16 tokens (N(0,1) rounded) through one layer, "
                             f"d_model 2048, d_ff 512, 256 routed + 1 shared, top-6, {wfmt} experts, Zipf(1.1) "
                             "router prior; MFMA operands fp16, fp32 accumulate",
                    global_batch=T, seq_len=T, parallelism="single-gpu",
                    flops_per_step=fl_all, layer_tflops=round(fl_all / (ms * 1e-3) / 1e12, 1),
                    layer_mfma_frac=round(fl_all / (ms * 1e-3) / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
                    experts_hit=int(np.count_nonzero(loads)), max_expert_load=int(loads.max()),
                    timing="HIP graph replay of one layer forward", eager_ms_per_step=round(ms_eager, 4),
                    graph_matches_eager=graph_matches_eager,
                    kernel_source_digest=source_digest(PREFILL_SOURCES)),
        roofline=dict(bound="mfma", kernel=dom, achieved=round(ach, 1), peak=MFMA_FP16_PEAK_TFLOPS,
                      unit="TFLOP/s", frac=round(ach / MFMA_FP16_PEAK_TFLOPS, 4), traffic=pf_traffic,
                      flops_per_launch=fl_dom, us_per_launch=round(kus[dom], 2),
                      timing="HIP dispatch events (hipExtLaunchKernelGGL) on the launch stream",
                      per_kernel=per_kernel,
                      mfma_counters=(prefill_mfma_counters({dom: fl_dom} if fused else
                                                           {"pf_gemm_gateup": fl_gu, "pf_gemm_down": fl_dn})
                                     if wfmt == "q4_1" else None)),
        cpu_baseline=cpu,
    )


def cpu_baseline_prefill(args, host, x):
    """The oracle (fp64 C) on the first --prefill-cpu-tokens tokens of the prefill
    batch (same layer, routing by the oracle's own top-k), split over the worker
    threads; reported as tokens/s."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    n = min(args.prefill_cpu_tokens, x.shape[0])
    xa = x[:n].float().cpu().double().numpy()
    W = cpu_workers()
    oracle.lib()
    chunks = np.array_split(np.arange(n), W)
    t0 = time.time()
    with ThreadPoolExecutor(max_workers=W) as ex:
        list(ex.map(lambda r: oracle.layer_forward(host, xa[r]), [c for c in chunks if len(c)]))
    dt = time.time() - t0
    return dict(value=round(n / dt, 2), unit="tok/s", cores=W, kind="oracle",
                sample=f"{n} of the 4096 bf16 tokens through the Zipf-skewed {host.dims.wfmt} layer, fp64 C, {W} threads, "
                       f"{dt:.1f}s", cpu_model=cpu_model(), os_cpu_count=os.cpu_count())


def bench_sweep(args):
    """Decode batch sweep: T tokens (fp32, N(0,1)) through 47 independent q4_1 layers, for
    T = 1 .. 64, on the decode path (T <= 32: batch-1 or small-batch kernels) and on the
    grouped-GEMM path (the prefill kernels, any T).  Each (T, path) is one HIP graph of
    47 layer calls, replayed; every layer has its own weights, so the active experts
    stream from HBM on every replay."""
    from sparse_moe_decode_route_amd import binding as B
    from sparse_moe_decode_route_amd import inputs as gen
    dims = gen.LayerDims(2048, 512, wfmt="q4_1")
    L = args.layers
    devs, _ = build_stack(dims, 3, L, keep_host=False)
    eb = B.packed_expert_bytes(dims)
    rows = []
    for T in (1, 2, 4, 8, 12, 16, 24, 32, 64):
        x = gen.make_hidden(3, T, 2048, draw=900 + T, device="cuda")
        for path in (("decode", "gemm") if T <= 32 else ("gemm",)):
            prefill = path == "gemm"
            ws = B.workspace(dims, T)
            y = torch.empty((T, 2048), device="cuda")
            # routing of every layer (for the distinct expert bytes)
            union = 0
            for d in devs:
                _, idx, _ = B.layer_forward(d, x, ws=ws, y=y, prefill=prefill)
                union += len(set(idx.cpu().numpy().reshape(-1).tolist())) + dims.n_shared

            def step():
                for d in devs:
                    B.layer_forward(d, x, ws=ws, y=y, want_routing=False, prefill=prefill)

            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                step()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            n = max(5, args.steps // 10)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            for _ in range(n):
                g.replay()
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / n
            del g
            rows.append(dict(T=T, path=path, ms_per_step=round(ms, 4), us_per_layer=round(ms * 1000 / L, 2),
                             layer_tok_s=round(L * T / (ms * 1e-3), 1),
                             experts_per_layer=round(union / L, 1),
                             expert_gbs=round(union * eb / (ms * 1e-3) / 1e9, 1)))
            log(f"sweep T={T} {path}: {rows[-1]}")
    best64 = max(r["layer_tok_s"] for r in rows if r["T"] == 64)
    crossover = [r["T"] for r in rows if r["path"] == "gemm" and r["T"] <= 32 and
                 r["layer_tok_s"] >= next(q["layer_tok_s"] for q in rows if q["T"] == r["T"] and q["path"] == "decode")]
    return dict(
        metric="MoE-layer decode tokens/s by batch size (q4_1, 47 independent layers)",
        value=best64, unit="MoE-layer tok/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=next(r["ms_per_step"] for r in rows if r["T"] == 64), higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload="moe_decode_sweep_q4_1: d_model 2048, d_ff 512, 256 routed + 1 shared, top-6, q4_1 "
                             "experts, 47 independent layers, T fp32 N(0,1) tokens per layer call, T = 1..64; "
                             "value and ms_per_step at T = 64",
                    global_batch=64, seq_len=1, parallelism="single-gpu", layers=L,
                    gemm_path_not_slower_at_T=crossover, sweep=rows))


def bench_lm_head(args, wfmt: str):
    """The output layer at decode: T tokens (fp32, N(0,1)) through W [146,484, 2048].

    One step is one moe_lm_head call.  The weights exist in n_copies copies
    (together larger than the chip's 256 MB last-level cache) and consecutive
    calls rotate through them, so every call streams its matrix from HBM."""
    from sparse_moe_decode_route_amd import binding as B
    from sparse_moe_decode_route_amd import inputs as gen
    import oracle
    V, D, T = gen.LM_HEAD_VOCAB, 2048, args.lm_tokens
    wbytes = B.lm_head_bytes(V, D, wfmt)
    n_copies = max(2, -(-1024 * 2 ** 20 // wbytes))
    t0 = time.time()
    blob, s_t = gen.make_lm_head(V, D, wfmt, cfg_id=gen.LM_HEAD_CFG, device="cuda")
    heads = [B.upload_lm_head(V, D, wfmt, blob, s_t, "cuda") for _ in range(n_copies)]
    torch.cuda.synchronize()
    log(f"output layer {wfmt}: {n_copies} copies of {wbytes / 1e6:.1f} MB ready in {time.time() - t0:.1f}s")
    x = gen.make_hidden(gen.LM_HEAD_CFG, T, D, draw=500, device="cuda")
    out = torch.empty((T, V), dtype=torch.float32, device="cuda")
    ref = B.lm_head(heads[0], x)
    torch.cuda.synchronize()

    per_graph = n_copies * max(1, -(-24 // n_copies))  # >= 24 calls per replay: launch cost amortised

    def step_all():
        for i in range(per_graph):
            B.lm_head(heads[i % n_copies], x, logits=out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step_all()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_all()
    reps = max(1, -(-args.steps // per_graph))
    wreps = max(1, -(-args.warmup // per_graph))
    for _ in range(wreps):
        g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    steps = reps * per_graph
    ms = ev0.elapsed_time(ev1) / steps
    graph_matches_eager = bool(torch.equal(out, ref))
    # per-launch dispatch durations (events on the launch stream), rotating copies
    n_timed = max(1, min(args.timed_calls, 40))
    kus = [B.lm_head_timed(heads[i % n_copies], x, logits=out)[1] for i in range(n_timed)]
    us = float(np.mean(kus))
    algo = wbytes + T * D * 4 + T * V * 4 + (4 if wfmt == "nvfp4" else 0)
    ach = algo / (us * 1e-6) / 1e9
    kname = "lm_head_kernel"
    tr = COUNTER_TRAFFIC.get((f"lm_head_{wfmt}_t{T}", kname))
    traffic = None
    if tr is not None and tr["source_digest"] == source_digest(LM_HEAD_SOURCES):
        traffic = tr["fetch_bytes"] + tr["write_bytes"]
    cpu = None
    if not args.no_cpu:
        hb = blob.cpu().numpy()
        xs = x.cpu().double().numpy()
        rows = min(V, max(1, args.lm_cpu_rows))
        st = 1.0 if s_t is None else float(s_t.reshape(-1)[0])
        passes, c0 = 0, time.time()
        while passes == 0 or time.time() - c0 < args.lm_cpu_seconds:
            oracle.lm_head(gen.WFMT_CODES[wfmt], hb, V, D, xs, s_t=st, rows=np.arange(rows))
            passes += 1
        dt = (time.time() - c0) / passes
        cpu = dict(value=round(T / (dt * V / rows), 3), unit="tok/s", cores=1, kind="oracle",
                   sample=f"{passes} pass(es) over {rows} of {V} vocabulary rows for {T} token(s), fp64 C "
                          f"oracle, one thread, {dt:.2f}s per pass; scaled to the full vocabulary")
    return dict(
        metric=f"output-layer (lm_head) decode tokens/s, {wfmt} weights",
        value=round(T / (ms * 1e-3), 1), unit="tok/s", n_gpus=1, steps=steps, warmup=wreps * per_graph,
        ms_per_step=round(ms, 5), higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
        data="synthetic",
        config=dict(workload=f"lm_head_{wfmt}: vocab {V} x d_model {D} {wfmt} output layer, {T} fp32 N(0,1) "
                             f"token(s) per call, weights N(0, 0.02)",
                    global_batch=T, seq_len=1, parallelism="single-gpu", weight_bytes=wbytes,
                    weight_copies=n_copies,
                    timing=f"HIP graph of {per_graph} calls rotating over the weight copies, replayed",
                    graph_matches_eager=graph_matches_eager),
        roofline=dict(bound="hbm", kernel=kname, achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic, algo_bytes_per_launch=algo,
                      us_per_launch=round(us, 3),
                      timing=f"HIP dispatch events (hipExtLaunchKernelGGL) on the launch stream, mean of "
                             f"{n_timed} calls over rotating weight copies"),
        cpu_baseline=cpu,
    )


def bench_attn(args, kind: str):
    """Decode attention for one token (batch 1).

    attn_swa: the 35 sliding-window layers of one token, each with its own
    cache (8192 positions, the token at 8000: a full window of 513); one step
    is 35 calls.  attn_full128k: one full-attention layer at position 131,071
    of a 131,072-position cache (268 MB of keys and values); two caches used
    in turn so that every call streams from HBM."""
    from sparse_moe_decode_route_amd import binding as B
    from sparse_moe_decode_route_amd import inputs as gen
    import oracle
    Hq, Hkv, D = gen.ATTN_HQ, gen.ATTN_HKV, gen.ATTN_D
    if kind == "swa":
        window, max_len, P, n_layers = gen.ATTN_WINDOW, 8192, 8000, 35
    else:
        window, max_len, P, n_layers = 0, 131072, 131071, 2
    dims = B.attn_dims(Hq, Hkv, window, gen.ATTN_ROPE_BASE, 1e-6)
    layers = [gen.make_attn(1, Hq, Hkv, D, max_len, cfg_id=gen.ATTN_CFG, draw=l, device="cuda") for l in range(n_layers)]
    pos = torch.tensor([P], dtype=torch.int32, device="cuda")
    ws = B.attn_workspace(dims, 1, max_len)
    out = torch.empty((1, Hq, D), device="cuda")
    ref = B.attn_decode(dims, layers[0], pos, ws=ws).clone()
    torch.cuda.synchronize()
    per_graph = n_layers * max(1, -(-8 // n_layers))

    def step_all():
        for i in range(per_graph):
            B.attn_decode(dims, layers[i % n_layers], pos, out=out, ws=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step_all()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_all()
    reps = max(1, -(-args.steps // per_graph))
    for _ in range(max(1, -(-args.warmup // per_graph))):
        g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    calls = reps * per_graph
    ms_call = ev0.elapsed_time(ev1) / calls
    # the last replay's last call used layer (per_graph - 1) % n_layers
    last = B.attn_decode(dims, layers[(per_graph - 1) % n_layers], pos, ws=ws)
    graph_matches_eager = bool(torch.equal(out, last))
    n_timed = max(1, min(args.timed_calls, 20))
    kus = {}
    for i in range(n_timed):
        _, us = B.attn_decode_timed(dims, layers[i % n_layers], pos, ws=ws)
        for k, v in us.items():
            kus[k] = kus.get(k, 0.0) + v / n_timed
    n_pos = min(P + 1, window) if window > 0 else P + 1
    kv_bytes = n_pos * Hkv * D * 2 * 2
    # chunk partials written: one per chunk that holds positions of the range
    chunk, _ = B.attn_chunk_plan(dims, 1, max_len)
    lo = P + 1 - n_pos
    nc = P // chunk - lo // chunk + 1
    part_bytes = Hq * nc * (D + 2) * 4
    algo = kv_bytes + Hq * D * 4 + part_bytes  # keys, values, queries in, chunk partials out
    ach = algo / (kus["attn_chunk"] * 1e-6) / 1e9
    tr = COUNTER_TRAFFIC.get((f"attn_{kind}", "attn_chunk"))
    traffic = None
    if tr is not None and tr["source_digest"] == source_digest(ATTN_SOURCES):
        traffic = tr["fetch_bytes"] + tr["write_bytes"]
    step_layers = n_layers if kind == "swa" else 1
    ms_step = ms_call * step_layers
    cpu = None
    if not args.no_cpu:
        l0 = layers[0]
        c0 = time.time()
        oracle.attn_decode(l0.q.cpu().numpy(), l0.k_new.cpu().numpy(), l0.v_new.cpu().numpy(),
                           l0.q_norm_w.cpu().numpy(), l0.k_norm_w.cpu().numpy(), l0.sinks.cpu().numpy(),
                           l0.k_cache.cpu().numpy().view(np.uint16), l0.v_cache.cpu().numpy().view(np.uint16),
                           np.array([P]), window, gen.ATTN_ROPE_BASE, 1e-6)
        dt = time.time() - c0
        cpu = dict(value=round(1.0 / (dt * step_layers), 4), unit="tok/s", cores=1, kind="oracle",
                   sample=f"one call of the fp64 C oracle ({dt:.2f}s, cache copy included), one thread; "
                          f"x{step_layers} for the step")
    name = "35 sliding-window layers" if kind == "swa" else "one full-attention layer at 128k context"
    return dict(
        metric=f"decode attention tokens/s ({name}, batch 1)",
        value=round(1.0 / (ms_step * 1e-3), 1), unit="tok/s", n_gpus=1, steps=calls, warmup=per_graph,
        ms_per_step=round(ms_step, 5), higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
        data="synthetic",
        config=dict(workload=f"attn_{kind}: 32 query / 4 key-value heads of 128, bf16 cache of {max_len} positions, "
                             f"new token at {P}, " + ("window 513 with rotary embeddings, 35 layers with their own "
                             "caches per step" if kind == "swa" else "full attention (no rotary embedding)"),
                    global_batch=1, seq_len=P + 1, parallelism="single-gpu", us_per_call=round(ms_call * 1e3, 3),
                    kernel_us={k: round(v, 3) for k, v in kus.items()},
                    timing=f"HIP graph of {per_graph} calls over {n_layers} caches, replayed",
                    graph_matches_eager=graph_matches_eager),
        roofline=dict(bound="hbm", kernel="attn_chunk", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic, algo_bytes_per_launch=algo,
                      us_per_launch=round(kus["attn_chunk"], 3),
                      timing=f"HIP dispatch events (hipExtLaunchKernelGGL) on the launch stream, mean of {n_timed} calls"),
        cpu_baseline=cpu,
    )


def _short_kernel_name(name: str) -> str:
    """Kernel name without return type, namespaces and argument list."""
    n = name.replace("void ", "").replace("moe::", "").replace("(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in n:
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            break
        out.append(ch)
    return "".join(out).strip()


def _stats(v):
    v = np.asarray(v, dtype=np.float64)
    if v.size == 0:
        return None
    return dict(n=int(v.size), mean=round(float(v.mean()), 4), p10=round(float(np.percentile(v, 10)), 4),
                p50=round(float(np.percentile(v, 50)), 4), p90=round(float(np.percentile(v, 90)), 4))


def rocprof_summary(path: str) -> dict:
    """Per-kernel summary of a rocprofv3 CSV written while this script ran.

    Dispatches are split at the first hold_stream dispatch: before it, the
    graph replays (and the untimed eager calls); from it on, the timed calls,
    whose launches were enqueued behind the hold and ran back to back.  A
    kernel_trace.csv gives durations in microseconds; a counter_collection.csv
    gives each counter's value per dispatch, and the dispatch's duration."""
    import csv
    with open(path) as f:
        rows = list(csv.DictReader(f))
    counters = "Counter_Name" in (rows[0] if rows else {})
    disp = {}
    for r in rows:
        d = disp.setdefault(int(r["Dispatch_Id"]), dict(k=_short_kernel_name(r["Kernel_Name"]),
                                                        s=int(r["Start_Timestamp"]), e=int(r["End_Timestamp"]),
                                                        c={}))
        if counters:
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ds = sorted(disp.values(), key=lambda d: d["s"])
    first_hold = next((d["s"] for d in ds if d["k"] == "hold_stream"), None)
    per = {}
    for d in ds:
        ph = "graph" if first_hold is None or d["s"] < first_hold else "timed"
        vals = dict(d["c"], duration_us=(d["e"] - d["s"]) / 1e3) if counters else {"duration_us": (d["e"] - d["s"]) / 1e3}
        for c, v in vals.items():
            per.setdefault(d["k"], {}).setdefault(c, {"graph": [], "timed": []})[ph].append(v)
    return {k: {c: dict(all=_stats(v["graph"] + v["timed"]), graph=_stats(v["graph"]), timed=_stats(v["timed"]))
                for c, v in cs.items()} for k, cs in per.items()}


def main():
    args = parse()
    if args.rocprof_summary:
        print(json.dumps(rocprof_summary(args.rocprof_summary), indent=1))
        return
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
    B.set_decode_path({"persistent": B.PATH_PERSISTENT, "xcd": B.PATH_XCD}.get(args.decode_path, B.PATH_KERNELS))
    if args.workload == "stack_q4_1_b1":
        out = bench_stack(args, "q4_1", 1)
    elif args.workload == "stack_nvfp4_b1":
        out = bench_stack(args, "nvfp4", 1)
    elif args.workload == "sweep_q4_1":
        out = bench_sweep(args)
    elif args.workload.startswith("attn_"):
        out = bench_attn(args, args.workload[len("attn_"):])
    elif args.workload.startswith("lm_head_"):
        out = bench_lm_head(args, args.workload[len("lm_head_"):])
    elif args.workload == "stack_nvfp4_b8":
        out = bench_stack(args, "nvfp4", 8)
    else:
        out = bench_prefill(args, args.workload[len("prefill_"):])
    if args.copy_calibration:
        copy_calibration()
    print(json.dumps(out), flush=True)


def copy_calibration():
    """A plain device copy of 256 MiB, five times: the reference kernel whose
    FETCH_SIZE / WRITE_SIZE readings scale the counters of the decode kernels."""
    n = 64 * 1024 * 1024
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 5 x {n * 4} bytes read and written")


if __name__ == "__main__":
    main()
