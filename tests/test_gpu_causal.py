"""GPU parity of the causal variant (the row at position i sees keys j <= i)
against the fp64 oracle, through the C ABI: the fused forward (bf16 and
fp32), one rank's share, and the backward. Gates as for the non-causal path
(tests/gates.py)."""

import numpy as np
import pytest
import torch

import rsa_inputs
import sequence_transformer_attention_rsa_amd as rsa
from gates import LSE_TOL, assert_parity
from gpu_util import device, from_dev, inputs, mask_dev, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu



def check_lse(got, want, dtype, what):
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: lse finiteness differs"
    if fin.any():
        err = np.abs(got[fin] - want[fin]).max()
        assert err <= LSE_TOL[dtype], f"{what}: lse max-abs {err:.3e}"


def gpu_forward(x, dtype, N, dev):
    q, k, v = (to_dev(x[n], dtype, dev) for n in ("q", "k", "v"))
    out, lse = rsa.forward(q, k, v, mask_dev(x["mask"], dev), N=N, return_lse=True, causal=True)
    torch.cuda.synchronize()
    return from_dev(out), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,N,valid", [
    (256, 4, None),          # chunks of one 64-key tile: the diagonal tile of each 128-row block
    (512, 4, (300, 512)),    # chunks of 128, key padding
    (200, 5, (120, 200)),    # chunks of 40: tiles straddle chunks
    (130, 13, None),         # chunks of 10
    (1, 1, None),
    (384, 2, None),          # three query blocks in a chunk of 192
    (1024, 4, None),         # chunks of 256, no key mask: the table-free walk, diagonal tiles at two offsets
    (1536, 4, None),         # chunks of 384: diagonal tiles at three offsets
    (512, 1, None),          # one chunk
])
def test_causal_forward_small_parity(oracle_lib, dtype, d, L, N, valid):
    dev = device()
    x = inputs(2, 2, L, d, seed=L + 11 * N + d, dtype=dtype, valid_range=valid)
    say("causal forward", dtype, d, L, N, valid)
    out, lse = gpu_forward(x, dtype, N, dev)
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=N, causal=True)
    assert_parity(out, want, dtype, f"causal {dtype} d={d} L={L} N={N}")
    check_lse(lse, want_lse, dtype, "causal lse")


def test_causal_first_row_copies_first_value_and_n_independence(oracle_lib):
    dev = device()
    L, d = 512, 64
    x = inputs(1, 3, L, d, seed=5, dtype="bf16")
    say("causal first row")
    want, _ = oracle_lib.forward(x["q"], x["k"], x["v"], None, N=1, causal=True)
    for N in (1, 2, 4, 8, 64, 512):
        out, _ = gpu_forward(x, "bf16", N, dev)
        assert np.array_equal(out[:, :, 0], x["v"][:, :, 0]), N   # weight exactly 1
        assert_parity(out, want, "bf16", f"causal N={N}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L,N,d", [(1024, 8, 64), (600, 6, 128), (96, 96, 64),
                                   (1536, 12, 128)])   # 8 ring-step groups of two or one steps
def test_causal_rank_share(oracle_lib, dtype, L, N, d):
    """One rank's share: ranks after the first meet chunks that hide nothing
    (before their own), their own chunk (the diagonal) and chunks that hide
    everything (after their own), possibly whole ring-step groups of them."""
    dev = device()
    x = inputs(2, 2, L, d, seed=L + N + 1, dtype=dtype, valid_range=(L // 2, L))
    Lc = L // N
    k, v = to_dev(x["k"], dtype, dev), to_dev(x["v"], dtype, dev)
    m = mask_dev(x["mask"], dev)
    for rank in sorted({0, 1, N // 2, N - 1}):
        rows = np.arange(rank * Lc, (rank + 1) * Lc)
        ql = to_dev(x["q"][:, :, rows], dtype, dev)
        say("causal rank share", dtype, L, N, d, rank)
        out, lse = rsa.forward_rank(ql, k, v, m, N=N, rank=rank, return_lse=True, causal=True)
        torch.cuda.synchronize()
        want, want_lse = oracle_lib.forward(x["q"][:, :, rows], x["k"], x["v"], x["mask"], N=N, qpos=rows,
                                            causal=True)
        assert_parity(from_dev(out), want, dtype, f"causal rank {rank}")
        check_lse(lse.cpu().numpy().astype(np.float64), want_lse, dtype, f"causal rank {rank}")


@pytest.mark.parametrize("B,H,L,N,rank", [
    (1, 2, 1024, 1, 0),        # one chunk: the share is the whole sequence
    (1, 8, 16384, 2, 1),       # 512 query tiles: one ring-step group, rows from position 8192
])
def test_causal_rank_share_unmasked_one_group(oracle_lib, B, H, L, N, rank):
    """A rank's share without a key mask launched as one ring-step group
    takes the forward's table-free causal walk; the oracle checks 96 sampled
    rows of every head."""
    dev = device()
    d = 64
    x = inputs(B, H, L, d, seed=L + N + rank, dtype="bf16")
    Lc = L // N
    rows = np.arange(rank * Lc, (rank + 1) * Lc)
    k, v = to_dev(x["k"], "bf16", dev), to_dev(x["v"], "bf16", dev)
    say("causal rank share unmasked", B, H, L, N, rank)
    out, lse = rsa.forward_rank(to_dev(x["q"][:, :, rows], "bf16", dev), k, v, None, N=N, rank=rank,
                                return_lse=True, causal=True)
    torch.cuda.synchronize()
    pick = np.sort(np.random.default_rng(L + rank).choice(Lc, 96, replace=False))
    want, want_lse = oracle_lib.forward(x["q"][:, :, rows[pick]], x["k"], x["v"], None, N=N, qpos=rows[pick],
                                        causal=True)
    assert_parity(from_dev(out)[:, :, pick], want, "bf16", f"causal unmasked rank {rank}")
    check_lse(lse.cpu().numpy().astype(np.float64)[:, :, pick], want_lse, "bf16", f"causal unmasked rank {rank}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,N,valid", [
    (256, 4, None),          # chunks of 64: 128-key workgroups span two chunks
    (512, 2, (400, 512)),    # chunks of 256, key padding
    (200, 5, (120, 200)),    # chunks of 40: every tile masked per element
    (130, 13, None),         # chunks of 10
    (384, 3, None),          # chunks of 128, no key mask: the table-free dQ
    (1024, 4, None),         # chunks of 256: two workgroups per chunk, diagonal tiles at two offsets
    (1536, 4, None),         # chunks of 384: diagonal tiles at three offsets
    (512, 1, None),          # one chunk
])
def test_causal_backward_small_parity(oracle_lib, d, L, N, valid):
    dev = device()
    x = inputs(2, 2, L, d, seed=L * 5 + N + d, dtype="bf16", valid_range=valid, with_dout=True)
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    say("causal backward", d, L, N, valid)
    out, lse = rsa.forward(q, k, v, m, N=N, return_lse=True, causal=True)
    dq, dk, dv = rsa.backward(q, k, v, out, g, lse, m, N=N, causal=True)
    torch.cuda.synchronize()
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=N, causal=True)
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert_parity(from_dev(a), b, "bf16", f"causal {name} d={d} L={L} N={N}", grad=True)


def test_causal_long_sequence_sampled_rows(oracle_lib):
    """The long-sequence workload (B=2 H=12 L=8192 d=64 N=16) with the causal
    mask: ~130 sampled rows of two heads."""
    w = rsa_inputs.WORKLOADS["long_seq"]
    dev = device()
    x = rsa_inputs.workload_inputs(w)
    say("causal long_seq")
    out, lse = gpu_forward(x, "bf16", w.N, dev)
    for b, h in ((0, 2), (1, 11)):
        rows = sample_rows(w.L, 128, seed=7 + h)
        want, want_lse = oracle_lib.forward(x["q"][b:b + 1, h:h + 1, rows], x["k"][b:b + 1, h:h + 1],
                                            x["v"][b:b + 1, h:h + 1], None, N=w.N, qpos=rows, causal=True)
        assert_parity(out[b, h, rows], want[0, 0], "bf16", f"causal long_seq b={b} h={h}")
        check_lse(lse[b, h, rows], want_lse[0, 0], "bf16", "causal long_seq")


def test_causal_backward_long_sequence_one_head(oracle_lib):
    """The long-sequence workload (B=2 H=12 L=8192 d=64 N=16, no key mask)
    with the causal mask, the launch the causal bench times: dQ, dK and dV of
    one head element by element against the oracle."""
    w = rsa_inputs.WORKLOADS["long_seq"]
    dev = device()
    x = rsa_inputs.make_inputs(w.B, w.H, w.L, w.d, w.seed, w.dtype, with_dout=True)
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    say("causal long_seq backward")
    out, lse = rsa.forward(q, k, v, None, N=w.N, return_lse=True, causal=True)
    dq, dk, dv = rsa.backward(q, k, v, out, g, lse, None, N=w.N, causal=True)
    torch.cuda.synchronize()
    b, h = 1, 5
    sl = (slice(b, b + 1), slice(h, h + 1))
    want = oracle_lib.backward(x["q"][sl], x["k"][sl], x["v"][sl], x["dout"][sl], None, N=w.N, causal=True)
    for name, a, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert_parity(from_dev(a)[sl], ref, "bf16", f"causal long_seq {name} b={b} h={h}", grad=True)


def test_causal_backward_workload_two_heads(oracle_lib):
    """The backward workload (B=4 H=12 L=4096 d=64 N=8, key padding) with the
    causal mask, checked on two heads element by element."""
    w = rsa_inputs.WORKLOADS["backward"]
    dev = device()
    x = rsa_inputs.workload_inputs(w)
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    say("causal backward workload")
    out, lse = rsa.forward(q, k, v, m, N=w.N, return_lse=True, causal=True)
    dq, dk, dv = rsa.backward(q, k, v, out, g, lse, m, N=w.N, causal=True)
    torch.cuda.synchronize()
    got = [from_dev(t) for t in (dq, dk, dv)]
    for b, h in ((0, 0), (3, 7)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        want = oracle_lib.backward(x["q"][sl], x["k"][sl], x["v"][sl], x["dout"][sl], x["mask"][b:b + 1], N=w.N,
                                   causal=True)
        for name, a, ref in zip(("dq", "dk", "dv"), got, want):
            assert_parity(a[sl], ref, "bf16", f"causal workload {name} b={b} h={h}", grad=True)


def test_causal_longest_key_range(oracle_lib):
    """L = 1048576 with the causal mask: the tile table of a workgroup near
    the end of the sequence classifies 16384 tiles; sampled rows of every
    part of the sequence, key padding at the end."""
    dev = device()
    L, N, d = 64 * 16384, 64, 64
    x = inputs(1, 1, L, d, seed=77, dtype="bf16", valid_range=(L - 3000, L - 1000))
    say("causal longest key range", "valid", x["valid_len"])
    out, lse = gpu_forward(x, "bf16", N, dev)
    rows = sample_rows(L, 14, seed=78)
    want, want_lse = oracle_lib.forward(x["q"][:, :, rows], x["k"], x["v"], x["mask"], N=N, qpos=rows, causal=True)
    assert_parity(out[0, 0, rows], want[0, 0], "bf16", f"causal L={L}")
    check_lse(lse[0, 0, rows], want_lse[0, 0], "bf16", f"causal L={L}")


def test_causal_backward_every_ring_size(oracle_lib):
    """The causal backward does not depend on N (every divisor of L = 256,
    including one token per chunk)."""
    dev = device()
    L, d = 256, 64
    x = inputs(1, 2, L, d, seed=79, dtype="bf16", valid_range=(200, 200), with_dout=True)
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=1, causal=True)
    for N in (1, 2, 4, 16, 64, 256):
        say("causal backward ring size", N)
        out, lse = rsa.forward(q, k, v, m, N=N, return_lse=True, causal=True)
        dq, dk, dv = rsa.backward(q, k, v, out, g, lse, m, N=N, causal=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
            assert_parity(from_dev(a), b, "bf16", f"causal N={N} {name}", grad=True)


def padded_mask(B, L, N, kind):
    """Key masks that leave early query rows without any visible key under the
    causal mask: "left" pads the first keys of the sequence, "hole" pads the
    first keys of every chunk (every other chunk entirely in its first half)."""
    Lc = L // N
    m = np.ones((B, L), np.uint8)
    if kind == "left":
        m[0, :37] = 0
        m[1, :Lc + 5] = 0
    else:
        for c in range(N):
            m[0, c * Lc:c * Lc + min(3, Lc)] = 0
            if c % 2 == 1:
                m[1, c * Lc:c * Lc + max(1, Lc // 2)] = 0
        m[1, :1] = 0
    return m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,N,kind", [(256, 4, "left"), (512, 8, "hole"), (200, 5, "left"), (200, 5, "hole"),
                                      (384, 3, "hole")])
def test_causal_padding_before_visible_keys(oracle_lib, dtype, d, L, N, kind):
    """Causal mask plus key padding at the start of the sequence or of each
    chunk: the first rows see no key at all (output 0, lse -inf), and within
    one wave some rows meet their first visible key while others have seen
    none yet, so a rescale must leave the latter untouched (never NaN). The
    full forward and one rank's share (ring-step groups + merge)."""
    dev = device()
    x = inputs(2, 2, L, d, seed=L + 3 * N + d + (kind == "hole"), dtype=dtype)
    x["mask"] = padded_mask(2, L, N, kind)
    say("causal padded", dtype, d, L, N, kind)
    out, lse = gpu_forward(x, dtype, N, dev)
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=N, causal=True)
    assert np.all(np.isfinite(out)), "non-finite output"
    empty = np.isneginf(want_lse)
    assert empty.any()
    assert np.all(out[empty] == 0.0) and np.all(np.isneginf(lse[empty]))
    assert_parity(out, want, dtype, f"causal padded {kind} {dtype} d={d} L={L} N={N}")
    check_lse(lse, want_lse, dtype, "causal padded lse")
    Lc = L // N
    k, v = to_dev(x["k"], dtype, dev), to_dev(x["v"], dtype, dev)
    m = mask_dev(x["mask"], dev)
    for rank in sorted({0, 1, N - 1}):
        rows = np.arange(rank * Lc, (rank + 1) * Lc)
        ql = to_dev(x["q"][:, :, rows], dtype, dev)
        say("causal padded rank share", dtype, d, L, N, kind, rank)
        o, ls = rsa.forward_rank(ql, k, v, m, N=N, rank=rank, return_lse=True, causal=True)
        torch.cuda.synchronize()
        o, ls = from_dev(o), ls.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(o)), f"rank {rank}: non-finite output"
        assert_parity(o, want[:, :, rows], dtype, f"causal padded rank {rank}")
        check_lse(ls, want_lse[:, :, rows], dtype, f"causal padded rank {rank}")
