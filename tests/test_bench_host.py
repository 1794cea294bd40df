"""Host-side logic of bench.py (no GPU): algorithmic byte counts, the roofline
arithmetic, the rocprofv3 summary's phase split, the counter-based MFMA
utilisation, and the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from sparse_moe_decode_route_amd import inputs as gen  # noqa: E402


def test_batch1_algorithmic_bytes_per_launch():
    # one q4_1 matrix [512, 2048] (or [2048, 512]) is 655,360 B: 2048 * 512 / 32
    # blocks of 20 B; the router is 256 x 2048 bf16
    dims = gen.LayerDims(2048, 512, wfmt="q4_1")
    assert gen.matrix_bytes(512, 2048, "q4_1") == 655_360
    a = bench.kernel_algo_bytes(dims, 1, 6.0)
    # router + x + logits
    assert a["b1_route"] == 1_048_576 + 8_192 + 1_024
    # logits + 7 experts' gate/up (6 routed, 1 shared) + x + h
    assert a["b1_topk_gateup"] == 1_024 + 7 * 1_310_720 + 8_192 + 14_336
    # 7 experts' down + h + y
    assert a["b1_down"] == 7 * 655_360 + 14_336 + 8_192
    assert a["b1_topk_gateup"] == 9_198_592 and a["b1_down"] == 4_610_048


def test_small_batch_gateup_bytes_count_each_expert_once():
    dims = gen.LayerDims(2048, 512, wfmt="nvfp4")
    gu = gen.matrix_bytes(512, 2048, "nvfp4")
    assert gu == 589_824
    a = bench.kernel_algo_bytes(dims, 8, 45.0)
    pairs = 8 * 6 + 8
    assert a["bn_gateup"] == 46 * 2 * gu + 8 * 2048 * 4 + 8 * 256 * 4 + pairs * 512 * 4


def test_roofline_takes_the_longest_kernel():
    dims = gen.LayerDims(2048, 512, wfmt="q4_1")
    us = {"b1_route": 4.0, "b1_topk_gateup": 5.0, "b1_down": 4.5}
    r = bench.roofline("stack_q4_1_b1", dims, 1, 47, us, 6.0)
    assert r["kernel"] == "b1_topk_gateup" and r["bound"] == "hbm" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(9_198_592 / 5e-6 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, abs=1e-4)


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_rocprof_summary_splits_at_the_first_hold(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    k = "void moe::(anonymous namespace)::b1_down<1, 16>(moe::DecodeParams)"
    rows = [[1, k, 1000, 5000], [2, k, 6000, 9000],
            [3, "(anonymous namespace)::hold_stream(unsigned int*, unsigned int, unsigned long)", 10000, 20000],
            [4, k, 21000, 23000], [5, k, 24000, 26000]]
    p = tmp_path / "run_kernel_trace.csv"
    _write_csv(p, hdr, rows)
    s = bench.rocprof_summary(str(p))
    d = s["b1_down<1, 16>"]["duration_us"]
    assert d["graph"]["n"] == 2 and d["graph"]["mean"] == pytest.approx(3.5)
    assert d["timed"]["n"] == 2 and d["timed"]["mean"] == pytest.approx(2.0)
    assert d["all"]["n"] == 4
    assert s["hold_stream"]["duration_us"]["timed"]["n"] == 1


def test_rocprof_summary_counters(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    k = "void moe::(anonymous namespace)::pf_gemm_q4<0, 128>(moe::(anonymous namespace)::PfParams)"
    rows = [[7, k, "FETCH_SIZE", 10.0, 1, 2], [7, k, "FETCH_SIZE", 5.0, 1, 2], [8, k, "FETCH_SIZE", 21.0, 3, 4]]
    p = tmp_path / "run_counter_collection.csv"
    _write_csv(p, hdr, rows)
    s = bench.rocprof_summary(str(p))
    f = s["pf_gemm_q4<0, 128>"]["FETCH_SIZE"]["all"]
    # the rows of one dispatch are summed (one per hardware instance), then averaged over dispatches
    assert f["n"] == 2 and f["mean"] == pytest.approx(18.0)


def test_prefill_mfma_counter_arithmetic(monkeypatch):
    digest = bench.source_digest(bench.PREFILL_SOURCES)
    v = dict(GRBM_GUI_ACTIVE=8 * 300_000.0, SQ_VALU_MFMA_BUSY_CYCLES=1024 * 120_000.0,
             SQ_INSTS_VALU_MFMA_MOPS_F16=250e6, duration_us=160.0)
    monkeypatch.setattr(bench, "PREFILL_MFMA_COUNTERS", dict(source_digest=digest, pf_ffn=v))
    out = bench.prefill_mfma_counters({"pf_ffn": 180e9})
    g = out["pf_ffn"]
    assert g["mfma_busy_frac"] == pytest.approx(0.4)
    assert g["issued_flops"] == round(250e6 * 512)
    assert g["padding_overhead"] == pytest.approx(250e6 * 512 / 180e9 - 1, abs=1e-4)
    assert g["clock_ghz"] == pytest.approx(300_000 / 160e3, abs=1e-3)
    # kernels without stored counters are left out
    assert bench.prefill_mfma_counters({"pf_gemm_gateup": 120e9}) is None
    monkeypatch.setattr(bench, "PREFILL_MFMA_COUNTERS", dict(source_digest="stale", pf_ffn=v))
    assert bench.prefill_mfma_counters({"pf_ffn": 180e9}) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
