"""GPU parity of the RSA backward (dQ, dK, dV) against the fp64 oracle,
through the C ABI. The GPU backward receives the GPU forward's output and
lse, as a training step would."""

import numpy as np
import pytest
import torch

import rsa_inputs
import sequence_transformer_attention_rsa_amd as rsa
from gates import LSE_TOL, MAX_ABS, REL_FRO_GRAD, assert_parity, errors
from gpu_util import device, report, from_dev, inputs, mask_dev, say, to_dev

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(x, N, dev):
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    out, lse = rsa.forward(q, k, v, m, N=N, return_lse=True)
    dq, dk, dv = rsa.backward(q, k, v, out, g, lse, m, N=N)
    torch.cuda.synchronize()
    return from_dev(dq), from_dev(dk), from_dev(dv)


def check_grads(got, want, what):
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_parity(a, b, "bf16", f"{what} {name}", grad=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,N,valid", [
    (256, 4, None),
    (256, 4, (150, 256)),
    (200, 5, (120, 200)),    # chunks of 40: tiles straddle chunks, ragged tails
    (130, 13, (60, 130)),    # chunks of 10, 130 = one 128-row tile + 2 rows
    (64, 64, None),          # one token per chunk
    (128, 2, (70, 128)),     # two query tiles: the copy two tiles ahead never issued
    (192, 3, None),          # three query tiles
    (32, 8, (24, 32)),       # the finite-difference slice's shape
])
def test_backward_small_parity(oracle_lib, d, L, N, valid):
    dev = device()
    x = inputs(2, 2, L, d, seed=L * 7 + N + d, dtype="bf16", valid_range=valid, with_dout=True)
    say("backward", d, L, N, valid)
    got = gpu_fwd_bwd(x, N, dev)
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=N)
    check_grads(got, want, f"d={d} L={L} N={N}")
    if x["mask"] is not None:
        for b, vl in enumerate(x["valid_len"]):
            assert np.all(got[1][b, :, vl:] == 0) and np.all(got[2][b, :, vl:] == 0)


@pytest.mark.parametrize("jump", [25.0, 60.0])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_late_score_jumps(oracle_lib, jump, d):
    """Gradients when three late keys outscore every other key by jump,
    jump + 1 and jump + 2 natural units (the forward's lazy rescale under
    stress, and large lse). dK and dV of the planted keys reach 10-30, where
    the bf16 rounding of the stored gradient alone exceeds the unit-scale
    max-abs bound, so that bound is taken relative to max(1, max |want|);
    the relative Frobenius bound is the usual one."""
    dev = device()
    L, N = 1024, 4
    x = inputs(1, 2, L, d, seed=int(jump) * 3 + d, dtype="bf16", scale=0.5, with_dout=True)
    rsa_inputs.plant_score_jumps(x, jump, [L - 400, L - 200, L - 30])
    say("backward late score jumps", jump, d)
    got = gpu_fwd_bwd(x, N, dev)
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], None, N=N)
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        e = errors(a, b)
        bound = MAX_ABS["bf16"] * max(1.0, float(np.abs(b).max()))
        report(f"backward late score jumps {jump} d={d} {name}", e)
        assert e["finite"], f"{name}: non-finite values"
        assert e["max_abs"] <= bound, f"{name}: max-abs {e['max_abs']:.3e} > {bound:.3e}"
        assert e["rel_fro"] <= REL_FRO_GRAD["bf16"], f"{name}: rel-fro {e['rel_fro']:.3e}"


@pytest.mark.parametrize("variant", ["plain", "causal", "dropout"])
def test_backward_d128_all_heads(oracle_lib, variant):
    """d = 128 at a grid that fills the GPU's XCDs (B=2, H=4: eight heads, so
    each XCD takes one; L = 2048, N = 8, key padding): forward and backward
    through the C ABI, every element of out, lse, dQ, dK and dV of every
    head against the oracle, plain, causal and with dropout 0.1."""
    dev = device()
    B, H, L, d, N = 2, 4, 2048, 128, 8
    x = inputs(B, H, L, d, seed=128 + len(variant), dtype="bf16", valid_range=(1500, 2048), with_dout=True)
    causal = variant == "causal"
    drop = (0.1, 77, 3) if variant == "dropout" else None
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    say("backward d=128 all heads", variant)
    out, lse = rsa.forward(q, k, v, m, N=N, return_lse=True, causal=causal, dropout=drop)
    dq, dk, dv = rsa.backward(q, k, v, out, g, lse, m, N=N, causal=causal, dropout=drop)
    torch.cuda.synchronize()
    want_o, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=N, causal=causal, dropout=drop)
    report(f"backward d=128 {variant} out", assert_parity(from_dev(out), want_o, "bf16", f"d=128 {variant} out"))
    got_lse = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(want_lse)
    assert np.array_equal(np.isfinite(got_lse), fin)
    assert np.abs(got_lse[fin] - want_lse[fin]).max() <= LSE_TOL["bf16"]
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=N, causal=causal, dropout=drop)
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        report(f"backward d=128 {variant} {name}",
               assert_parity(from_dev(a), b, "bf16", f"d=128 {variant} {name}", grad=True))


def test_backward_every_ring_size(oracle_lib):
    dev = device()
    L, d = 256, 64
    x = inputs(1, 2, L, d, seed=21, dtype="bf16", valid_range=(180, 180), with_dout=True)
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=1)
    for N in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        say("backward ring size", N)
        check_grads(gpu_fwd_bwd(x, N, dev), want, f"N={N}")


def test_backward_fully_masked_row():
    dev = device()
    L, d = 192, 64
    x = inputs(2, 2, L, d, seed=22, dtype="bf16", with_dout=True)
    mask = np.ones((2, L), np.uint8)
    mask[0] = 0
    x["mask"] = mask
    say("backward fully masked row")
    dq, dk, dv = gpu_fwd_bwd(x, 3, dev)
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0) and np.all(dv[0] == 0)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))


def test_backward_stages_match_and_are_deterministic():
    dev = device()
    L, d, N = 512, 64, 8
    x = inputs(2, 3, L, d, seed=23, dtype="bf16", valid_range=(300, 512), with_dout=True)
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    say("backward stages")
    out, lse = rsa.forward(q, k, v, m, N=N, return_lse=True)
    full = rsa.backward(q, k, v, out, g, lse, m, N=N)
    again = rsa.backward(q, k, v, out, g, lse, m, N=N)
    stats = rsa.backward_preprocess(out, g, lse)
    dq = rsa.backward_dq(q, k, v, g, stats, m, N=N)
    dk, dv = rsa.backward_dkdv(q, k, v, g, stats, m, N=N)
    torch.cuda.synchronize()
    for a, b in zip(full, again):
        assert torch.equal(a, b)
    for a, b in zip(full, (dq, dk, dv)):
        assert torch.equal(a, b)
    want_delta = (out.float() * g.float()).sum(-1)
    assert torch.allclose(-stats[0], want_delta, rtol=1e-5, atol=1e-5)
    assert torch.allclose(-stats[1], lse * 1.4426950408889634, rtol=1e-6, atol=1e-6)


def test_backward_invariants():
    """Key gradients sum to zero over keys; value gradients sum to the sum of dO."""
    dev = device()
    L, d = 512, 64
    x = inputs(1, 2, L, d, seed=24, dtype="bf16", with_dout=True)
    say("backward invariants")
    dq, dk, dv = gpu_fwd_bwd(x, 4, dev)
    scale_k = np.abs(dk).sum(axis=2)
    assert np.all(np.abs(dk.sum(axis=2)) <= 2e-2 * scale_k + 1e-3)
    gsum = x["dout"].astype(np.float64).sum(axis=2)
    assert np.abs(dv.sum(axis=2) - gsum).max() <= 2e-2 * np.abs(gsum).max() + 0.05


def test_backward_workload_full_parity(oracle_lib):
    """B=4, H=12, L=4096, d=64, N=8, key padding: dQ, dK and dV of all 48
    heads element by element, each head also on its own."""
    w = rsa_inputs.WORKLOADS["backward"]
    dev = device()
    x = rsa_inputs.workload_inputs(w)
    say("workload backward, all heads")
    got = gpu_fwd_bwd(x, w.N, dev)
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=w.N)
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        report(f"backward {name} (48 heads)", assert_parity(a, b, "bf16", f"backward {name}", grad=True))
    for bb in range(w.B):
        for h in range(w.H):
            sl = (bb, h)
            check_grads([g[sl] for g in got], [g[sl] for g in want], f"backward b={bb} h={h}")


@pytest.mark.parametrize("H,L,N", [
    (20, 4096, 8),   # 640 workgroups of 128 rows: the standard forward and dQ instances
    (4, 1024, 4),    # 32 workgroups: the key-split forward and dQ (each wave pair one key half)
])
def test_mask_with_holes(oracle_lib, H, L, N):
    """A key mask with holes inside the sequence -- the first key, one whole
    64-key tile, scattered keys across several partly valid tiles (both
    32-key halves), padding at the end -- at B=1, d=64, on a grid that takes
    the standard instances and on one that takes the key-split ones. Output,
    lse, dQ, dK and dV of all heads against the oracle."""
    B, d = 1, 64
    dev = device()
    x = inputs(B, H, L, d, seed=4242 + L, dtype="bf16", with_dout=True)
    rng = np.random.default_rng(4243 + L)
    m = np.ones((B, L), dtype=np.uint8)
    m[0, 0] = 0
    m[0, 320:384] = 0                                 # tile 5, all of it
    span = slice(640, 640 + L // 4)
    m[0, span][rng.random(L // 4) < 0.15] = 0         # partly valid tiles
    m[0, L - 96:] = 0                                 # padding
    x["mask"] = m
    say("mask with holes", B, H, L, N)
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    md = mask_dev(m, dev)
    out, lse = rsa.forward(q, k, v, md, N=N, return_lse=True)
    dq, dk, dv = rsa.backward(q, k, v, out, g, lse, md, N=N)
    torch.cuda.synchronize()
    want_out, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], m, N=N)
    report(f"holes forward out (L={L}, {H} heads)", assert_parity(from_dev(out), want_out, "bf16", "holes out"))
    got_lse = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got_lse)) and np.all(np.isfinite(want_lse))
    assert np.abs(got_lse - want_lse).max() <= LSE_TOL["bf16"]
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], m, N=N)
    got = [from_dev(t) for t in (dq, dk, dv)]
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        report(f"holes backward {name} (L={L}, {H} heads)", assert_parity(a, b, "bf16", f"holes {name}", grad=True))
    masked = m[0] == 0
    for name, a in (("dk", got[1]), ("dv", got[2])):
        assert np.all(a[:, :, masked] == 0.0), f"holes {name}: a masked key's gradient is not zero"


def test_backward_long_sequence_four_heads(oracle_lib):
    """The bench's own step at B=2, H=12, L=8192, d=64, N=16, no mask: the
    forward and the backward as the bench launches it (one rsa_backward
    call, bitwise equal to the three stage calls its per-kernel pass times),
    and the gradients of the first and last head of both batch rows against
    the oracle, element by element."""
    w = rsa_inputs.WORKLOADS["long_seq"]
    dev = device()
    x = rsa_inputs.make_inputs(w.B, w.H, w.L, w.d, w.seed, w.dtype, w.scale, w.valid_range, with_dout=True)
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    say("long_seq backward stages")
    out, lse = rsa.forward(q, k, v, None, N=w.N, return_lse=True)
    stats = rsa.backward_preprocess(out, g, lse)
    dq = rsa.backward_dq(q, k, v, g, stats, None, N=w.N)
    dk, dv = rsa.backward_dkdv(q, k, v, g, stats, None, N=w.N)
    # the one call the bench times (its dQ kernel forms the row statistics)
    dq1, dk1, dv1 = rsa.backward(q, k, v, out, g, lse, None, N=w.N)
    torch.cuda.synchronize()
    for name, a, b in (("dq", dq, dq1), ("dk", dk, dk1), ("dv", dv, dv1)):
        assert torch.equal(a, b), f"long_seq {name}: one call differs from the stage calls"
    got = [from_dev(t) for t in (dq, dk, dv)]
    heads = ((0, 0), (0, w.H - 1), (1, 0), (1, w.H - 1))
    sel = lambda a: np.stack([a[b, h] for b, h in heads])[None]
    want = oracle_lib.backward(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["dout"]), None, N=w.N)
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        report(f"long_seq backward {name} (4 heads)",
               assert_parity(sel(a), b, "bf16", f"long_seq {name}", grad=True))
        for i, (bb, h) in enumerate(heads):
            assert_parity(a[bb, h], b[0, i], "bf16", f"long_seq {name} b={bb} h={h}", grad=True)


def test_backward_longest_key_range():
    """L = 1048576, the longest sequence one launch covers, with key padding.
    The oracle cannot evaluate a head this long, so the gradients are checked
    through identities that hold at any size: the key gradients sum to zero
    over the keys, the value gradients sum to the sum of dO over the queries,
    and padded keys get exactly zero."""
    dev = device()
    L, d, N = 64 * 16384, 64, 64
    x = inputs(1, 1, L, d, seed=45, dtype="bf16", valid_range=(L - 7000, L - 3000), with_dout=True)
    vl = int(x["valid_len"][0])
    say("backward longest key range, valid", vl)
    dq, dk, dv = gpu_fwd_bwd(x, N, dev)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.all(np.isfinite(g)), name
    assert np.all(dk[0, :, vl:] == 0) and np.all(dv[0, :, vl:] == 0)
    scale_k = np.abs(dk).sum(axis=2)
    assert np.all(np.abs(dk.sum(axis=2)) <= 2e-2 * scale_k + 1e-3)
    gsum = x["dout"].astype(np.float64).sum(axis=2)
    assert np.abs(dv.sum(axis=2) - gsum).max() <= 2e-2 * np.abs(gsum).max() + 0.05
    assert np.abs(dq).max() > 0


# ------------------------------------------------------------- fp32 ---

def gpu_fwd_bwd_f32(x, N, dev, causal=False):
    q, k, v, g = (to_dev(x[n], "f32", dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    out, lse = rsa.forward(q, k, v, m, N=N, return_lse=True, causal=causal)
    dq, dk, dv = rsa.backward(q, k, v, out, g, lse, m, N=N, causal=causal)
    torch.cuda.synchronize()
    return from_dev(dq), from_dev(dk), from_dev(dv)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,N,valid,causal", [
    (256, 4, None, False),          # the fp32 workload's shape
    (256, 4, (150, 256), True),
    (200, 5, (120, 200), False),    # chunks of 40: tiles straddle chunks, ragged tails
    (130, 13, (60, 130), True),     # chunks of 10, one 128-row tile + 2 rows
    (64, 64, None, False),          # one token per chunk
    (32, 8, (24, 32), False),       # the finite-difference slice's shape
])
def test_backward_f32_parity(oracle_lib, d, L, N, valid, causal):
    """fp32 in, fp32 out: dQ, dK, dV against the fp64 oracle at the fp32
    gates (max-abs 1e-4, relative Frobenius 1e-5)."""
    dev = device()
    x = inputs(2, 2, L, d, seed=L * 3 + N + d + causal, dtype="f32", valid_range=valid, with_dout=True)
    say("backward f32", d, L, N, valid, causal)
    got = gpu_fwd_bwd_f32(x, N, dev, causal)
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=N, causal=causal)
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_parity(a, b, "f32", f"f32 {name} d={d} L={L} N={N}", grad=True)
    if x["mask"] is not None:
        for b, vl in enumerate(x["valid_len"]):
            assert np.all(got[1][b, :, vl:] == 0) and np.all(got[2][b, :, vl:] == 0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_f32_eight_heads(oracle_lib, d, causal):
    """fp32 at eight heads (B=2 H=4, L=1024, N=8, key padding): several
    query and key tiles per head on every XCD, forward and backward against
    the oracle at the fp32 gates."""
    dev = device()
    x = inputs(2, 4, 1024, d, seed=1024 + d + causal, dtype="f32", valid_range=(700, 1024), with_dout=True)
    say("backward f32 eight heads", d, causal)
    q, k, v, g = (to_dev(x[n], "f32", dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    out, lse = rsa.forward(q, k, v, m, N=8, return_lse=True, causal=causal)
    dq, dk, dv = rsa.backward(q, k, v, out, g, lse, m, N=8, causal=causal)
    torch.cuda.synchronize()
    want_o, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=8, causal=causal)
    assert_parity(from_dev(out), want_o, "f32", f"f32 eight heads out d={d}")
    got_lse = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(want_lse)
    assert np.array_equal(np.isfinite(got_lse), fin)
    assert np.abs(got_lse[fin] - want_lse[fin]).max() <= LSE_TOL["f32"]
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=8, causal=causal)
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        report(f"f32 eight heads d={d} causal={causal} {name}",
               assert_parity(from_dev(a), b, "f32", f"f32 eight heads {name}", grad=True))


def test_backward_f32_workload_and_stages(oracle_lib):
    """The fp32 workload's shape (B=1 H=2 L=256 d=64 N=4) with an upstream
    gradient: the one-call backward equals its three stages bit for bit,
    does not depend on N, and meets the fp32 gates."""
    w = rsa_inputs.WORKLOADS["fp32_small"]
    dev = device()
    x = rsa_inputs.make_inputs(w.B, w.H, w.L, w.d, w.seed, "f32", with_dout=True)
    q, k, v, g = (to_dev(x[n], "f32", dev) for n in ("q", "k", "v", "dout"))
    say("backward f32 workload")
    out, lse = rsa.forward(q, k, v, None, N=w.N, return_lse=True)
    full = rsa.backward(q, k, v, out, g, lse, None, N=w.N)
    stats = rsa.backward_preprocess(out, g, lse)
    dq = rsa.backward_dq(q, k, v, g, stats, None, N=w.N)
    dk, dv = rsa.backward_dkdv(q, k, v, g, stats, None, N=w.N)
    torch.cuda.synchronize()
    for a, b in zip(full, (dq, dk, dv)):
        assert torch.equal(a, b)
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], None, N=w.N)
    for name, a, b in zip(("dq", "dk", "dv"), full, want):
        report(f"fp32_small backward {name}", assert_parity(from_dev(a), b, "f32", f"f32 {name}", grad=True))
    for N in (1, 2, 16, 256):
        for name, a, b in zip(("dq", "dk", "dv"), gpu_fwd_bwd_f32(x, N, dev), want):
            assert_parity(a, b, "f32", f"f32 N={N} {name}", grad=True)
