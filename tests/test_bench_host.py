"""Host-side logic of bench.py (no GPU): the work counts behind the
TFLOP/s figures, the traffic lookup, and the one-GPU contract."""

import os
import subprocess
import sys

import numpy as np

import bench
import rsa_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def brute_pairs(w, x, causal):
    """(query row, visible valid key) pairs of one head by enumeration."""
    L = w.L
    rows = np.arange(w.Lq) + (w.rank * w.Lc if w.rank is not None else 0)
    total = 0
    for b in range(w.B):
        valid = np.ones(L, bool) if x["mask"] is None else x["mask"][b].astype(bool)
        for i in rows:
            vis = valid.copy()
            if causal:
                vis[i + 1:] = False
            total += int(vis.sum())
    return float(total)


def test_pair_count_matches_enumeration():
    cases = [
        rsa_inputs.Workload("t1", B=2, H=3, L=64, d=64, N=4, dtype="bf16", seed=1, valid_range=(20, 60)),
        rsa_inputs.Workload("t2", B=1, H=2, L=96, d=64, N=8, dtype="bf16", seed=2, valid_range=(50, 90), rank=5),
        rsa_inputs.Workload("t3", B=2, H=1, L=40, d=64, N=5, dtype="bf16", seed=3),
    ]
    for w in cases:
        x = rsa_inputs.make_inputs(w.B, w.H, w.L, 8, w.seed, "bf16", 1.0, w.valid_range, Lq=w.Lq)
        for causal in (False, True):
            assert bench.pair_count(w, x, causal) == brute_pairs(w, x, causal), (w.name, causal)


def test_causal_pairs_closed_form():
    w = rsa_inputs.WORKLOADS["long_seq"]
    x = {"mask": None, "valid_len": None}
    assert bench.pair_count(w, x, True) == w.B * w.L * (w.L + 1) / 2
    assert bench.pair_count(w, x, False) == w.B * w.L * w.L


def test_recorded_traffic_needs_matching_sources():
    assert bench.recorded_traffic("long_seq", "no_such_kernel") is None
    assert bench.recorded_traffic("no_such_workload", "forward") is None
    for kernel in bench.KERNEL_SOURCES:
        for f in bench.KERNEL_SOURCES[kernel]:
            assert os.path.exists(os.path.join(ROOT, "sequence_transformer_attention_rsa_amd", "csrc", f)), f


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_reports_cores_model_and_work():
    """The CPU baseline times the oracle on one head per thread across batch
    rows and reports the threads used, the affinity and the CPU model."""
    w = rsa_inputs.Workload("tiny", B=2, H=2, L=64, d=64, N=4, dtype="bf16", seed=4, valid_range=(40, 64),
                            backward=True)
    x = rsa_inputs.workload_inputs(w)
    r = bench.cpu_baseline(w, x, threads=3)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert r["cores"] >= 1 and r["affinity_cores"] == len(os.sched_getaffinity(0))
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]
    assert "3 of the 4 heads" in r["sample"] and "forward+backward" in r["sample"]
    # the credited work: 12 d flops per visible pair, heads (0,0), (0,1) of row 0 and (1,0) of row 1
    vl = [int(v) for v in x["valid_len"]]
    flops = 12.0 * w.d * w.L * (2 * vl[0] + vl[1])
    assert abs(r["value"] * 1e12 * r["seconds"] - flops) <= 1e-6 * flops
