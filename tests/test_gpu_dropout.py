"""GPU parity of the dropout variant against the fp64 oracle, through the C
ABI: the keep decisions bit for bit, and the outputs and gradients at the
usual gates.

The keep decisions are read out exactly: with the values one-hot over a
window of keys (v_{j0+x} = e_x, every other value row zero), output column x
of row i is P_{i,j0+x} Z_{i,j0+x}, exactly zero where the weight was dropped
and nonzero where it was kept (the weights are far from underflow). The same
with dO one-hot over a window of query rows reads them out of dV, which the
key-stationary backward kernel forms from its own copy of the decisions.
"""

import numpy as np
import pytest
import torch

import rsa_inputs
import sequence_transformer_attention_rsa_amd as rsa
from gates import LSE_TOL, assert_parity
from gpu_util import device, from_dev, inputs, mask_dev, report, say, to_dev

pytestmark = pytest.mark.gpu


def keep_block(oracle_lib, drop, bh, i0, ni, j0, nj):
    return oracle_lib.dropout_keep(drop, bh, i0, ni, j0, nj).astype(bool)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,L,N,j0s", [
    (64, 1024, 16, [0, 64, 448, 960]),       # chunk-aligned tiles
    (128, 1024, 8, [0, 384, 896]),
    (64, 640, 5, [0, 100, 576]),             # chunks of 128: tiles aligned
    (64, 600, 6, [40, 300, 536]),            # chunks of 100: tiles straddle chunks
])
def test_forward_keep_decisions_bit_exact(oracle_lib, dtype, d, L, N, j0s):
    dev = device()
    B, H = 2, 2
    x = inputs(B, H, L, d, seed=L + N + d, dtype=dtype)
    drop = (0.3, 0x5EED0000 + L, 7)
    q, k = to_dev(x["q"], dtype, dev), to_dev(x["k"], dtype, dev)
    for j0 in j0s:
        v = np.zeros((B, H, L, d), np.float32)
        w = min(d, L - j0)
        v[:, :, j0:j0 + w, :w] = np.eye(w, dtype=np.float32)
        say("dropout keep bits forward", dtype, d, L, N, j0)
        out = rsa.forward(q, k, to_dev(v, dtype, dev), None, N=N, dropout=drop)
        torch.cuda.synchronize()
        got = from_dev(out)[..., :w] != 0
        for b in range(B):
            for h in range(H):
                want = keep_block(oracle_lib, drop, b * H + h, 0, L, j0, w)
                bad = np.argwhere(got[b, h] != want)
                assert bad.size == 0, f"b={b} h={h} j0={j0}: {len(bad)} decisions differ, first {bad[:3]}"


@pytest.mark.parametrize("d,L,N", [(64, 1024, 16), (128, 512, 4), (64, 600, 6)])
def test_rank_share_keep_decisions_bit_exact(oracle_lib, d, L, N):
    """One rank's rows see the decisions of their sequence positions."""
    dev = device()
    x = inputs(1, 2, L, d, seed=L + 2 * N, dtype="bf16")
    drop = (0.5, 99, 1)
    Lc = L // N
    k = to_dev(x["k"], "bf16", dev)
    w = min(d, L)
    v = np.zeros((1, 2, L, d), np.float32)
    v[:, :, L - w:, :w] = np.eye(w, dtype=np.float32)
    vd = to_dev(v, "bf16", dev)
    for rank in (0, N - 1):
        rows = np.arange(rank * Lc, (rank + 1) * Lc)
        say("dropout keep bits rank share", d, L, N, rank)
        out = rsa.forward_rank(to_dev(x["q"][:, :, rows], "bf16", dev), k, vd, None, N=N, rank=rank,
                               dropout=drop)
        torch.cuda.synchronize()
        got = from_dev(out)[..., :w] != 0
        for h in range(2):
            want = keep_block(oracle_lib, drop, h, rank * Lc, Lc, L - w, w)
            assert np.array_equal(got[0, h], want), (rank, h)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,L,N,i0s", [
    (64, 1024, 16, [0, 512, 960]),
    (128, 512, 4, [0, 384]),
    (64, 600, 6, [30, 536]),                 # query tiles straddle chunks
])
def test_backward_keep_decisions_bit_exact(oracle_lib, dtype, d, L, N, i0s):
    """dV_j[x] = P_{i0+x,j} Z_{i0+x,j} with dO one-hot over rows i0 ..
    i0 + d - 1: the key-stationary kernel's decisions, bit for bit."""
    dev = device()
    B, H = 1, 2
    x = inputs(B, H, L, d, seed=L * 3 + N + d, dtype=dtype)
    drop = (0.25, 0xABCDEF0123456789, 3)
    q, k, v = (to_dev(x[n], dtype, dev) for n in ("q", "k", "v"))
    out, lse = rsa.forward(q, k, v, None, N=N, return_lse=True, dropout=drop)
    for i0 in i0s:
        w = min(d, L - i0)
        g = np.zeros((B, H, L, d), np.float32)
        g[:, :, i0:i0 + w, :w] = np.eye(w, dtype=np.float32)
        say("dropout keep bits backward", dtype, d, L, N, i0)
        dq, dk, dv = rsa.backward(q, k, v, out, to_dev(g, dtype, dev), lse, None, N=N, dropout=drop)
        torch.cuda.synchronize()
        got = (from_dev(dv)[..., :w] != 0).transpose(0, 1, 3, 2)   # [B, H, row x, key j]
        for h in range(H):
            want = keep_block(oracle_lib, drop, h, i0, w, 0, L)
            bad = np.argwhere(got[0, h] != want)
            assert bad.size == 0, f"h={h} i0={i0}: {len(bad)} decisions differ, first {bad[:3]}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,N,valid,causal", [
    (256, 4, None, False),
    (512, 8, (300, 512), False),
    (200, 5, (120, 200), False),      # chunks of 40: tiles straddle chunks, ragged tail
    (384, 3, (250, 384), True),
    (130, 13, None, True),            # chunks of 10
])
def test_dropout_forward_backward_parity(oracle_lib, dtype, d, L, N, valid, causal):
    dev = device()
    x = inputs(2, 2, L, d, seed=L + 5 * N + d + causal, dtype=dtype, valid_range=valid, with_dout=True)
    drop = (0.2, 1234567 + L, 11)
    q, k, v, g = (to_dev(x[n], dtype, dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    say("dropout parity", dtype, d, L, N, valid, causal)
    out, lse = rsa.forward(q, k, v, m, N=N, return_lse=True, causal=causal, dropout=drop)
    dq, dk, dv = rsa.backward(q, k, v, out, g, lse, m, N=N, causal=causal, dropout=drop)
    torch.cuda.synchronize()
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=N, causal=causal, dropout=drop)
    assert_parity(from_dev(out), want, dtype, f"dropout out {dtype} d={d} L={L} N={N}")
    lse_g = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(want_lse)
    assert np.array_equal(np.isfinite(lse_g), fin)
    assert np.abs(lse_g[fin] - want_lse[fin]).max() <= LSE_TOL[dtype]
    wg = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=N, causal=causal, dropout=drop)
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), wg):
        assert_parity(from_dev(a), b, dtype, f"dropout {name} {dtype} d={d} L={L} N={N}", grad=True)


def test_dropout_every_ring_size_and_zero_probability(oracle_lib):
    """The result does not depend on N (every divisor of L = 256); p = 0
    runs the plain kernels (bit for bit equal)."""
    dev = device()
    L, d = 256, 64
    x = inputs(1, 2, L, d, seed=31, dtype="bf16", valid_range=(200, 200), with_dout=True)
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    drop = (0.4, 2026, 0)
    want, _ = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=1, dropout=drop)
    wg = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=1, dropout=drop)
    for N in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        say("dropout ring size", N)
        out, lse = rsa.forward(q, k, v, m, N=N, return_lse=True, dropout=drop)
        grads = rsa.backward(q, k, v, out, g, lse, m, N=N, dropout=drop)
        torch.cuda.synchronize()
        assert_parity(from_dev(out), want, "bf16", f"dropout N={N}")
        for name, a, b in zip(("dq", "dk", "dv"), grads, wg):
            assert_parity(from_dev(a), b, "bf16", f"dropout N={N} {name}", grad=True)
    a, la = rsa.forward(q, k, v, m, N=4, return_lse=True)
    b, lb = rsa.forward(q, k, v, m, N=4, return_lse=True, dropout=(0.0, 5))
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_dropout_long_sequence_sampled(oracle_lib):
    """The long-sequence shape (B=2 H=12 L=8192 d=64 N=16) with dropout 0.1:
    the full forward and backward launches; 64 rows of every rank of two
    heads against the oracle's forward, and the gradients of one head."""
    w = rsa_inputs.WORKLOADS["long_seq"]
    dev = device()
    x = rsa_inputs.make_inputs(w.B, w.H, w.L, w.d, w.seed, w.dtype, with_dout=True)
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    drop = (0.1, 0xC0FFEE, 2)
    say("dropout long_seq")
    out, lse = rsa.forward(q, k, v, None, N=w.N, return_lse=True, dropout=drop)
    dq, dk, dv = rsa.backward(q, k, v, out, g, lse, None, N=w.N, dropout=drop)
    torch.cuda.synchronize()
    out = from_dev(out)
    rng = np.random.default_rng(8)
    rows = np.sort(np.concatenate([n * w.Lc + rng.choice(w.Lc, 64, replace=False) for n in range(w.N)]))
    for b, h in ((0, 0), (1, w.H - 1)):
        # the oracle sees the head at its own index b*H + h: pass the whole [B, H] layout's slice by position
        qb = np.zeros((w.B, w.H, len(rows), w.d), np.float32)
        qb[b, h] = x["q"][b, h, rows]
        want, _ = oracle_lib.forward(qb, x["k"], x["v"], None, N=w.N, qpos=rows, dropout=drop)
        report(f"long_seq dropout out b={b} h={h}", assert_parity(out[b, h, rows], want[b, h], "bf16",
                                                                 f"dropout long_seq b={b} h={h}"))
    # gradients of head (0, 0): the oracle's backward on a [1, 1] slice sees head index 0
    sl = (slice(0, 1), slice(0, 1))
    wg = oracle_lib.backward(x["q"][sl], x["k"][sl], x["v"][sl], x["dout"][sl], None, N=w.N, dropout=drop)
    for name, a, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), wg):
        report(f"long_seq dropout {name} b=0 h=0",
               assert_parity(from_dev(a)[sl], ref, "bf16", f"dropout long_seq {name}", grad=True))
