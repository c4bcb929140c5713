"""Benchmark of the Ring Self-Attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_seq]

One step is one pass of the whole path over one batch of seeded synthetic
input already resident in HBM: the forward over all N ranks (rsa_forward,
writing O and lse) and the backward (rsa_backward, whose dQ kernel also forms
the row statistics). The timed region runs K such steps with nothing between
the calls. A second pass of K steps makes the backward as its three stage
calls (rsa_backward_preprocess, rsa_backward_dq, rsa_backward_dkdv), each of
which launches exactly one kernel, so HIP events recorded between the calls on
the library's stream (torch's current stream) time every kernel separately;
the causal and dropout backwards have no stage calls and are timed whole. Rank-share workloads (--workload rank_share)
time rsa_forward_rank (split kernel + merge) and have no backward.
`--forward-variant twopass` times rsa_forward_twopass instead (score rows
materialised in HBM, row softmax, then P V; forward only): its roofline is
HBM bandwidth, 12 bytes per (query, key) pair -- fp32 scores written and read
back, bf16 weights written and read back -- plus Q, K, V and O once.

Algorithmic work (only what the method must compute, recomputation not
credited): forward 4*B*H*Lq*Lk*d flops, backward 8*B*H*Lq*Lk*d (the dV, dP,
dQ and dK contractions), so a step counts 12*B*H*Lq*Lk*d; with a key mask the
valid-key count replaces Lk. Per kernel: forward 4 (S and PV), dQ kernel 4
(dP and dQ), dK/dV kernel 4 (dV and dK) times B*H*Lq*Lk*d.

Prints one JSON line. `value` is whole-step TFLOP/s; `roofline` describes
the kernel with the longest average duration against MI355X's dense bf16
MFMA peak (2516.6 TFLOP/s); `cpu_baseline` times the fp64 CPU oracle on a
bounded sample of the same workload (rank 0 only, N=1 only).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import rsa_inputs  # noqa: E402

METRIC = "RSA attention TFLOP/s (fwd, fwd+bwd) and % of MI355X bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6     # 256 CUs x 4096 flop/clk/CU x 2.4 GHz, dense
PEAK_F32_MATRIX_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="long_seq", choices=sorted(rsa_inputs.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads for the CPU baseline (default: OMP_NUM_THREADS if set, else every "
                         "core of the process's affinity)")
    ap.add_argument("--forward-only", action="store_true", help="time the forward alone")
    ap.add_argument("--forward-variant", default="fused", choices=("fused", "twopass"),
                    help="fused online-softmax kernel, or the two-stage form with score rows in HBM "
                         "(implies --forward-only)")
    ap.add_argument("--causal", action="store_true",
                    help="the causal variant (row i sees keys j <= i); the backward is timed as one call")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability of the softmax weights (Philox-4x32-10 keep decisions, seed 1234); "
                         "the backward is timed as one call")
    ap.add_argument("--capacity", action="store_true",
                    help="single-GPU sequence-length capacity of the fused and the two-stage forward "
                         "(B=H=1, d=64) instead of the step benchmark")
    ap.add_argument("--layer", action="store_true",
                    help="time the encoder layer around RSA (QKV projection, attention, output projection, "
                         "layer norms, GeLU MLP) instead of the attention step")
    ap.add_argument("--layer-workload", default="layer_long_seq", choices=sorted(rsa_inputs.LAYERS))
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


KERNEL_SOURCES = {
    "forward": ("rsa_fwd.hip", "rsa_tiles.h", "rsa_device.h"),
    "bwd_dq": ("rsa_bwd.hip", "rsa_tiles.h", "rsa_device.h"),
    "bwd_dkdv": ("rsa_bwd.hip", "rsa_tiles.h", "rsa_device.h"),
    "forward_twopass": ("rsa_twopass.hip", "rsa_tiles.h", "rsa_device.h"),
    "ff1_gelu": ("rsa_layer.hip", "rsa_tiles.h", "rsa_device.h"),
}


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the calibrated FETCH_SIZE/WRITE_SIZE counters
    summarised in profiles/<workload>_<kernel>_traffic.md, or None when there
    is no such summary or the kernel's sources changed since it was taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{workload}_{kernel}_traffic.md")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ")):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sequence_transformer_attention_rsa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source-sha256") != h.hexdigest() or "traffic_bytes" not in fields:
        return None
    return float(fields["traffic_bytes"])


def valid_key_count(w, x):
    """Sum over (b) of valid keys, times H: the Lk actually attended."""
    if x["mask"] is None:
        return w.B * w.L
    return int(x["valid_len"].sum())


def pair_count(w, x, causal):
    """(query row, visible valid key) pairs of one head, summed over batch
    rows: Lq * valid keys, or with the causal mask sum_i min(i + 1, valid)
    over the query positions i (keys are valid up to a prefix length)."""
    vls = [w.L] * w.B if x["mask"] is None else [int(v) for v in x["valid_len"]]
    if not causal:
        return float(w.Lq * sum(vls))
    pos = np.arange(w.Lq, dtype=np.int64) + (w.rank * w.Lc if w.rank is not None else 0)
    return float(sum(np.minimum(pos + 1, vl).sum() for vl in vls))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, threads, causal=False, dropout=None):
    """fp64 oracle, forward (+ backward) on the first `threads` heads of the
    workload (batch row 0 first, then row 1, ...; full sequence length),
    timed once. One head per thread keeps every thread busy in the backward,
    which the oracle parallelises over heads (the forward over rows)."""
    import oracle

    heads = max(1, min(threads, w.B * w.H))
    picks = [(b, h) for b in range(w.B) for h in range(w.H)][:heads]
    rows = np.arange(w.Lq) + (w.rank * w.Lc if w.rank is not None else 0)
    # the sampled heads as a batch of single-head rows, each with its own
    # batch row's key mask, so that one oracle call spreads them over threads
    bs = [b for b, _ in picks]
    q, k, v = (np.ascontiguousarray(np.stack([x[n][b, h] for b, h in picks])[:, None]) for n in ("q", "k", "v"))
    m = None if x["mask"] is None else np.ascontiguousarray(x["mask"][bs])
    vls = [w.L] * heads if x["mask"] is None else [int(x["valid_len"][b]) for b in bs]
    pairs = sum(float(np.minimum(rows + 1, vl).sum()) if causal else float(w.Lq * vl) for vl in vls)
    what = "forward"
    t0 = time.perf_counter()
    if w.rank is not None:
        oracle.forward(q, k, v, m, N=w.N, qpos=rows, causal=causal, dropout=dropout)
    else:
        oracle.forward(q, k, v, m, N=w.N, causal=causal, dropout=dropout)
    flops = 4.0 * pairs * w.d
    if w.rank is None and x.get("dout") is not None:
        g = np.ascontiguousarray(np.stack([x["dout"][b, h] for b, h in picks])[:, None])
        oracle.backward(q, k, v, g, m, N=w.N, causal=causal, dropout=dropout)
        flops += 8.0 * pairs * w.d
        what = "forward+backward"
    if causal:
        what = "causal " + what
    if dropout is not None:
        what += f" with dropout {dropout[0]}"
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"fp64 oracle {what} of {heads} of the {w.B * w.H} heads at full length "
                  f"({w.name}: L={w.L}, d={w.d}, N={w.N}); {dt:.1f} s wall",
        "seconds": dt,
        "cpu_model": cpu_model(),
        "affinity_cores": len(os.sched_getaffinity(0)),
    }


def capacity(args):
    """Longest sequence one GPU runs in each form, B = H = 1, d = 64, bf16.
    The fused forward needs O(L d) memory and is bounded by the key range one
    launch covers (1048576); the two-stage form holds 4 L^2 bytes of score rows,
    so its bound is the device memory. Each form is run once at its bound
    (after one warm-up call) and timed with events."""
    import torch

    import sequence_transformer_attention_rsa_amd as rsa

    dev = torch.device("cuda:0")
    d = 64
    res = {}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def tensors(L):
        g = torch.Generator(device=dev).manual_seed(7)
        return [torch.randn((1, 1, L, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(3)]

    # fused: the longest key range of one launch
    L = 64 * 16384
    q, k, v = tensors(L)
    out = torch.empty_like(q)
    ms = timed(lambda: rsa.forward(q, k, v, None, N=64, out=out))
    res["fused"] = {"L": L, "bound": "key range of one launch (tile table)", "ms": ms,
                    "device_bytes": 4 * L * d * 2, "tflops": 4.0 * L * L * d / ms / 1e9}
    del q, k, v, out
    torch.cuda.empty_cache()

    # two-stage: the longest L (multiple of 1024) whose score rows fit the free memory
    free, total = torch.cuda.mem_get_info(dev)
    L = 1024
    while True:
        nxt = L + 1024
        need = rsa.forward_twopass_workspace_bytes(1, 1, nxt, d, 1) + 4 * nxt * d * 2 + nxt * 4
        if need > 0.85 * free:
            break
        L = nxt
    q, k, v = tensors(L)
    out = torch.empty_like(q)
    ws = torch.empty(rsa.forward_twopass_workspace_bytes(1, 1, L, d, 1), dtype=torch.uint8, device=dev)
    ms = timed(lambda: rsa.forward_twopass(q, k, v, None, N=1, out=out, workspace=ws))
    res["twopass"] = {"L": L, "bound": "device memory (4 L^2 bytes of score rows)", "ms": ms,
                      "device_bytes": ws.numel() + 4 * L * d * 2, "tflops": 4.0 * L * L * d / ms / 1e9}
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    line = {"metric": "single-GPU sequence-length capacity, B=H=1, d=64, bf16", "unit": "tokens",
            "device_memory_bytes": total, "fused": res["fused"], "twopass": res["twopass"],
            "ratio": res["fused"]["L"] / res["twopass"]["L"], "gpu": torch.cuda.get_device_name(dev)}
    print(json.dumps(line), flush=True)
    return 0


def layer_bench(args):
    """The encoder layer around RSA, step by step: QKV projection (head split
    fused), RSA forward, output projection (head merge, bias and residual
    fused), layer norm, first MLP product (bias and GeLU fused), second MLP
    product (bias and residual fused), layer norm. One launch per step, timed
    with events between the calls; the chain equals rsa_layer_forward bit for
    bit (checked once here). Work: products 2*M*E*(3E + E + F + F) flops with
    M = B*L, attention 4*B*H*L*Lk*d; layer norms read and write M*E bf16."""
    import torch

    import sequence_transformer_attention_rsa_amd as rsa

    shp = rsa_inputs.LAYERS[args.layer_workload]
    dev = torch.device("cuda:0")
    x = rsa_inputs.layer_inputs(shp)
    B, L, E, H, F, N = shp.B, shp.L, shp.E, shp.H, shp.F, shp.N
    M = B * L

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(dev)

    w = {n: (bf(x[n]) if n.startswith("w_") else torch.from_numpy(x[n]).to(dev)) for n in rsa.LAYER_WEIGHTS}
    xin = bf(x["x"])
    mask = None if x["mask"] is None else torch.from_numpy(x["mask"]).to(dev)
    names = ["qkv_projection", "attention", "output_projection", "layernorm1", "ff1_gelu", "ff2_residual",
             "layernorm2"]
    keep = {}

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        q, k, v = rsa.qkv_projection(xin, w["w_qkv"], w["b_qkv"], H)
        mark(1)
        o = rsa.forward(q, k, v, mask, N=N)
        mark(2)
        a1 = rsa.output_projection(o, w["w_o"], w["b_o"], xin)
        mark(3)
        h1 = rsa.layernorm(a1, w["ln1_gamma"], w["ln1_beta"]).view(M, E)
        mark(4)
        f1 = rsa.linear(h1, w["w_ff1"], w["b_ff1"], activation="gelu")
        mark(5)
        a2 = rsa.linear(f1, w["w_ff2"], w["b_ff2"], residual=h1)
        mark(6)
        keep["y"] = rsa.layernorm(a2, w["ln2_gamma"], w["ln2_beta"])
        mark(7)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ref = rsa.layer_forward(xin, w, H=H, N=N, key_mask=mask)
    torch.cuda.synchronize()
    same = bool(torch.equal(ref.view(M, E), keep["y"]))
    # timed region without events between the calls, then a pass with them
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    lk = float(x["valid_len"].sum()) if x["valid_len"] is not None else float(B * L)
    d = E // H
    flops = {"qkv_projection": 2.0 * M * E * 3 * E, "attention": 4.0 * H * L * d * lk,
             "output_projection": 2.0 * M * E * E, "ff1_gelu": 2.0 * M * E * F, "ff2_residual": 2.0 * M * F * E}
    ln_bytes = 2.0 * M * E * 2 + 2 * E * 4
    per = {}
    for i, n in enumerate(names):
        durs = [events[s][i].elapsed_time(events[s][i + 1]) for s in range(args.steps)]
        per[n] = {"avg_ms": float(np.mean(durs)), "median_ms": float(np.median(durs))}
        if n in flops:
            per[n]["tflops"] = flops[n] / (per[n]["avg_ms"] * 1e-3) / 1e12
            per[n]["frac_peak"] = per[n]["tflops"] / PEAK_BF16_TFLOPS
        else:
            per[n]["gbs"] = ln_bytes / (per[n]["avg_ms"] * 1e-3) / 1e9
            per[n]["frac_hbm_peak"] = per[n]["gbs"] / PEAK_HBM_GBS
    total = sum(flops.values())
    value = total / (ms_per_step * 1e-3) / 1e12
    gemm = [n for n in names if n in flops and n != "attention"]
    gemm_ms = sum(per[n]["avg_ms"] for n in gemm)
    dom = max(gemm, key=lambda n: per[n]["avg_ms"])
    line = {
        "metric": "SP encoder layer forward TFLOP/s (QKV proj + RSA + out proj + LN + GeLU MLP + LN), "
                  "% of MI355X bf16 MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": shp.name, "B": B, "L": L, "E": E, "H": H, "F": F, "N": N,
                   "key_mask": shp.valid_range is not None, "description": shp.description},
        "frac_peak": value / PEAK_BF16_TFLOPS,
        "products_tflops": sum(flops[n] for n in gemm) / (gemm_ms * 1e-3) / 1e12,
        "products_share_of_step": gemm_ms / ms_per_step,
        "chain_equals_rsa_layer_forward": same,
        "kernels": per,
        "roofline": {"kernel": f"rsa_gemm_bf16_256 ({dom})", "bound": "mfma",
                     "achieved": per[dom]["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": per[dom]["tflops"] / PEAK_BF16_TFLOPS,
                     "traffic": recorded_traffic(shp.name, dom),
                     "traffic_unit": "bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)",
                     "avg_ms": per[dom]["avg_ms"], "flops_per_launch": flops[dom]},
        "gpu": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line), flush=True)
    return 0 if same else 1


def main():
    args = parse()
    if args.layer:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            return 2
        return layer_bench(args)
    if args.capacity:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            return 2
        return capacity(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        return 2

    import torch

    import sequence_transformer_attention_rsa_amd as rsa

    w = rsa_inputs.WORKLOADS[args.workload]
    if w.dtype not in ("bf16", "f32"):
        print(f"workload {w.name} is CPU-only", file=sys.stderr)
        return 2
    twopass = args.forward_variant == "twopass"
    causal = args.causal
    dropout = (args.dropout, 1234, 0) if args.dropout > 0 else None
    if twopass and (w.rank is not None or w.dtype != "bf16" or causal or dropout):
        print("the two-stage forward covers full-sequence, non-causal bf16 workloads without dropout",
              file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    with_dout = w.rank is None
    x = rsa_inputs.make_inputs(w.B, w.H, w.L, w.d, w.seed, w.dtype, w.scale, w.valid_range,
                               Lq=w.Lq, with_dout=with_dout)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a):
        return torch.from_numpy(a).to(tdt).to(dev).contiguous()

    q, k, v = up(x["q"]), up(x["k"]), up(x["v"])
    g = up(x["dout"]) if with_dout else None
    mask = None if x["mask"] is None else torch.from_numpy(x["mask"]).to(dev)
    do_bwd = with_dout and w.dtype == "bf16" and not args.forward_only and not twopass

    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stats = torch.empty((2,) + tuple(lse.shape), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = None
    if w.rank is not None:
        ws = torch.empty(rsa.forward_rank_workspace_bytes(w.B, w.H, w.L, w.d, w.N), dtype=torch.uint8, device=dev)
    if twopass:
        ws = torch.empty(rsa.forward_twopass_workspace_bytes(w.B, w.H, w.L, w.d, w.N), dtype=torch.uint8,
                         device=dev)
    bws = None
    has_stages = not (causal or dropout is not None)   # the stage entry points have no causal or dropout form
    if do_bwd:
        bws = torch.empty(rsa.backward_workspace_bytes(w.B, w.H, w.L, w.d, w.N), dtype=torch.uint8, device=dev)

    if not has_stages:
        names = ["forward"] + (["backward"] if do_bwd else [])
    else:
        names = ["forward"] + (["bwd_preprocess", "bwd_dq", "bwd_dkdv"] if do_bwd else [])

    def step(ev=None, stages=True):
        # stages: the backward as its three stage calls, one kernel each, so
        # that events between them time each kernel; else one rsa_backward
        # call, which forms the row statistics inside the dQ kernel
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        if twopass:
            rsa.forward_twopass(q, k, v, mask, N=w.N, out=out, lse=lse, workspace=ws)
        elif w.rank is not None:
            rsa.forward_rank(q, k, v, mask, N=w.N, rank=w.rank, out=out, lse=lse, workspace=ws, causal=causal,
                             dropout=dropout)
        else:
            rsa.forward(q, k, v, mask, N=w.N, out=out, lse=lse, causal=causal, dropout=dropout)
        mark(1)
        if do_bwd and (not has_stages or not stages):
            rsa.backward(q, k, v, out, g, lse, mask, N=w.N, dq=dq, dk=dk, dv=dv, workspace=bws, causal=causal,
                         dropout=dropout)
            mark(2)
        elif do_bwd:
            rsa.backward_preprocess(out, g, lse, rowstats=stats)
            mark(2)
            rsa.backward_dq(q, k, v, g, stats, mask, N=w.N, dq=dq)
            mark(3)
            rsa.backward_dkdv(q, k, v, g, stats, mask, N=w.N, dk=dk, dv=dv)
            mark(4)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step(stages=False)
    torch.cuda.synchronize()

    # The timed region: K steps of the one-call API with nothing recorded
    # between the calls (an event between two kernels costs a few
    # microseconds of its own).
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for s in range(args.steps):
        step(stages=False)
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(stop)
    ms_per_step = ms_total / args.steps
    # Per-call times: a second pass of K steps with HIP events between the
    # calls, the backward as its stages where it has them.
    nev = len(names) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for _ in range(2):
        step()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    per_kernel = {}
    for i, name in enumerate(names):
        durs = [events[s][i].elapsed_time(events[s][i + 1]) for s in range(args.steps)]
        per_kernel[name] = {"avg_ms": float(np.mean(durs)), "median_ms": float(np.median(durs)),
                            "p10_ms": float(np.percentile(durs, 10)), "p90_ms": float(np.percentile(durs, 90))}

    # algorithmic work: 4 d flops per visible (query, key) pair forward, 8 d backward
    pairs = w.H * pair_count(w, x, causal)
    fwd_flops = 4.0 * w.d * pairs
    fwd_flops_nominal = 4.0 * w.B * w.H * w.Lq * w.L * w.d
    bwd_flops = 8.0 * w.d * pairs if do_bwd else 0.0
    step_flops = fwd_flops + bwd_flops
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MATRIX_TFLOPS

    credited = {"forward": fwd_flops, "bwd_dq": 4.0 * w.d * pairs, "bwd_dkdv": 4.0 * w.d * pairs,
                "backward": 8.0 * w.d * pairs}
    executed = {"forward": fwd_flops, "bwd_dq": 6.0 * w.d * pairs, "bwd_dkdv": 8.0 * w.d * pairs,
                "backward": 14.0 * w.d * pairs}
    for name in names:
        avg_s = per_kernel[name]["avg_ms"] * 1e-3
        if name in credited:
            per_kernel[name]["tflops_algorithmic"] = credited[name] / avg_s / 1e12
            per_kernel[name]["tflops_mfma_executed"] = executed[name] / avg_s / 1e12
        else:  # preprocess: reads O, dO and lse, writes the row statistics
            nbytes = 2 * q.numel() * q.element_size() + lse.numel() * 4 + stats.numel() * 4
            per_kernel[name]["gbs"] = nbytes / avg_s / 1e9
    dominant = max((n for n in names if n in credited), key=lambda n: per_kernel[n]["avg_ms"])
    dom_s = per_kernel[dominant]["avg_ms"] * 1e-3
    if twopass:
        # 12 bytes per (query, key) pair, plus q, k, v read and out, lse written once
        pairs = w.B * w.H * w.L * w.L
        nbytes = 12.0 * pairs + 4 * q.numel() * q.element_size() + lse.numel() * 4
        achieved = nbytes / dom_s / 1e9
        roofline = {
            "kernel": "rsa_2p_scores + rsa_2p_softmax + rsa_2p_pv",
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": recorded_traffic(w.name, "forward_twopass"),
            "traffic_unit": "bytes per call (calibrated FETCH_SIZE + WRITE_SIZE, three kernels)",
            "avg_ms": per_kernel[dominant]["avg_ms"],
            "bytes_per_launch": nbytes,
        }
    else:
        achieved = credited[dominant] / dom_s / 1e12
        roofline = {
            "kernel": {"forward": "rsa_fwd_kernel" if w.rank is None else "rsa_fwd_kernel + rsa_merge_kernel",
                       "bwd_dq": "rsa_bwd_dq", "bwd_dkdv": "rsa_bwd_dkdv",
                       "backward": "rsa_bwd_pre + rsa_bwd_dq + rsa_bwd_dkdv"}[dominant],
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": None if not has_stages else recorded_traffic(w.name, dominant),
            "traffic_unit": "bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)",
            "avg_ms": per_kernel[dominant]["avg_ms"],
            "flops_per_launch": credited[dominant],
        }

    fwd_s = per_kernel["forward"]["avg_ms"] * 1e-3
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "N": w.N,
                   "rank": w.rank, "key_mask": w.valid_range is not None,
                   "pass": "fwd+bwd" if do_bwd else "fwd", "forward": args.forward_variant, "causal": causal,
                   "dropout": args.dropout,
                   "description": w.description},
        "fwd_tflops": fwd_flops / fwd_s / 1e12,
        "fwd_tflops_nominal_keys": fwd_flops_nominal / fwd_s / 1e12,
        "fwd_frac_peak": fwd_flops / fwd_s / 1e12 / peak,
        "bwd_tflops": (bwd_flops / (sum(per_kernel[n]["avg_ms"] for n in names[1:]) * 1e-3) / 1e12
                       if do_bwd else None),
        "step_frac_peak": value / peak,
        "kernels": per_kernel,
        "backward_calls": None if not do_bwd else {
            "timed_region": "rsa_backward",
            "kernels_pass": "rsa_backward" if not has_stages else
            "rsa_backward_preprocess + rsa_backward_dq + rsa_backward_dkdv"},
        "roofline": roofline,
        "wall_s_timed_region": t_wall,
        "gpu": torch.cuda.get_device_name(dev),
    }
    if not args.no_cpu_baseline:
        # every core of the process's affinity, unless the environment
        # (OMP_NUM_THREADS, which the GPU hosts set to their CPU share) or
        # --cpu-threads says fewer
        threads = args.cpu_threads or int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
        os.environ["OMP_NUM_THREADS"] = str(threads)
        line["cpu_baseline"] = cpu_baseline(w, x, threads, causal, dropout)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
