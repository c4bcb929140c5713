"""Pins of the oracle's dropout variant (CPU only).

The pages never mention dropout; the reading taken is attention dropout on
the softmax weights: P is the softmax over the full key length (lse is
unchanged), each weight is kept with probability 1 - p and scaled by
1 / (1 - p), and O = (P o Z) V. The keep decisions come from Philox-4x32-10
(Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
3", SC'11) at a counter built from the weight's positions (oracle.c,
dropout_keep).

What pins it:
  * the generator's round structure: the oracle's 32-bit and 64-bit Philox
    are generated from one definition, and the 64-bit instance equals
    numpy's Philox (Philox-4x64-10) block for block; the 32-bit constants
    are the paper's (parity of the 32-bit stream beyond its shared structure
    is unpinned);
  * the stream's statistics: uniform bytes, the keep fraction, and no
    correlation between neighbouring weights, heads, seeds or offsets;
  * where dropout acts: torch fp64 softmax attention with the same keep
    decisions applied to the normalised weights, and torch autograd of it;
  * unbiasedness: the mean over seeds tends to the plain output;
  * p = 0 is the plain result exactly; the result does not depend on N;
  * the backward against central finite differences.
"""

import numpy as np
import pytest
import torch

import oracle
import rsa_inputs


# --------------------------------------------------------------- Philox ---

def test_philox_4x64_matches_numpy_philox():
    """numpy's Philox bit generator draws Philox-4x64-10 blocks at counter + 1
    (it increments before each block, carrying into the next word)."""
    M = 2 ** 64 - 1
    cases = [([0, 0, 0, 0], [0, 0]), ([5, 0, 0, 0], [123, 456]), ([7, 11, 13, 17], [2 ** 63, 99]),
             ([M, 5, 0, 0], [1, 2]), ([M, M, 3, 0], [M, M])]
    for ctr, key in cases:
        bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
        got = bg.random_raw(4).astype(np.uint64)
        nxt = list(ctr)
        for w in range(4):   # counter + 1 with carry
            nxt[w] = (nxt[w] + 1) & M
            if nxt[w] != 0:
                break
        want = oracle.philox4x64_10(nxt, key)
        assert np.array_equal(got, want), (ctr, key)


def test_philox_4x32_bytes_are_uniform():
    counters = np.stack(np.meshgrid(np.arange(40), np.arange(25), [3], [9], indexing="ij"), -1).reshape(-1, 4)
    words = np.concatenate([oracle.philox4x32_10(c, [0x1234, 0xABCD]) for c in counters])
    by = words.view(np.uint8)
    counts = np.bincount(by, minlength=256)
    expect = by.size / 256
    chi2 = ((counts - expect) ** 2 / expect).sum()
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)   # 255 degrees of freedom
    # the generator is a bijection of the counter for a fixed key: no repeats
    assert len({tuple(oracle.philox4x32_10(c, [5, 6])) for c in counters[:300]}) == 300


# ----------------------------------------------------- keep decisions ---

@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_fraction(p):
    p8 = oracle.dropout_p8(p)
    keep = np.concatenate([oracle.dropout_keep((p, 77, 3), bh, 0, 256, 1000, 512).ravel() for bh in range(3)])
    q = 1 - p8 / 256
    sd = np.sqrt(q * (1 - q) / keep.size)
    assert abs(keep.mean() - q) < 5 * sd


def test_keep_decisions_are_uncorrelated():
    d = (0.5, 2024, 1)
    a = oracle.dropout_keep(d, 4, 100, 200, 300, 257).astype(np.float64)
    n = a[:, :-1].size

    def corr(x, y):
        x, y = x.ravel() - x.mean(), y.ravel() - y.mean()
        return float((x * y).mean() / np.sqrt((x * x).mean() * (y * y).mean()))

    bound = 5 / np.sqrt(n)
    assert abs(corr(a[:, :-1], a[:, 1:])) < bound     # neighbouring keys
    assert abs(corr(a[:-1], a[1:])) < bound           # neighbouring queries
    assert abs(corr(a[:, :-4], a[:, 4:])) < bound     # the other half of a 32-key block
    assert abs(corr(a[:, :-32], a[:, 32:])) < bound   # the next 32-key block
    for other in (oracle.dropout_keep(d, 5, 100, 200, 300, 257),          # another head
                  oracle.dropout_keep((0.5, 2025, 1), 4, 100, 200, 300, 257),   # another seed
                  oracle.dropout_keep((0.5, 2024, 2), 4, 100, 200, 300, 257)):  # another offset
        assert abs(corr(a, other.astype(np.float64))) < bound


def test_quantised_probability():
    assert oracle.dropout_p8(0.0) == 0 and oracle.dropout_p8(0.1) == 26 and oracle.dropout_p8(0.5) == 128
    assert oracle.dropout_p8(1 / 512) == 1 and oracle.dropout_p8(0.998) == 255
    with pytest.raises(ValueError):
        oracle.dropout_p8(1.0)
    assert np.all(oracle.dropout_keep((0.0, 1), 0, 0, 64, 0, 64) == 1)


# ------------------------------------------------------- dropout output ---

def small(B=2, H=2, L=48, d=8, seed=0, valid=(30, 48)):
    x = rsa_inputs.make_inputs(B, H, L, d, seed, "f64", valid_range=valid, with_dout=True)
    return x


def keep_tensor(dropout, B, H, L):
    return np.stack([np.stack([oracle.dropout_keep(dropout, b * H + h, 0, L, 0, L) for h in range(H)])
                     for b in range(B)]).astype(np.float64)


def test_p_zero_is_the_plain_result():
    x = small()
    o0, l0 = oracle.forward(x["q"], x["k"], x["v"], x["mask"], N=4)
    o1, l1 = oracle.forward(x["q"], x["k"], x["v"], x["mask"], N=4, dropout=(0.0, 99))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    g0 = oracle.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=4)
    g1 = oracle.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=4, dropout=(0.0, 99))
    for a, b in zip(g0, g1):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_acts_on_the_normalised_weights(causal):
    """torch fp64: O = (softmax(Q K^T / sqrt(d) + M) o Z) V with the same keep
    decisions, and its gradients by autograd; lse is the plain softmax's."""
    x = small(seed=3)
    B, H, L, d = x["q"].shape
    drop = (0.3, 4242, 5)
    p8 = oracle.dropout_p8(drop[0])
    Z = torch.from_numpy(keep_tensor(drop, B, H, L) * (256 / (256 - p8)))
    q, k, v = (torch.from_numpy(x[n]).requires_grad_() for n in ("q", "k", "v"))
    bias = torch.zeros(B, 1, L, L, dtype=torch.float64)
    bias.masked_fill_(torch.from_numpy(x["mask"] == 0)[:, None, None, :], float("-inf"))
    if causal:
        bias = bias + torch.triu(torch.full((L, L), float("-inf"), dtype=torch.float64), 1)
    s = q @ k.transpose(-1, -2) / np.sqrt(d) + bias
    P = torch.softmax(s, dim=-1)
    out = (P * Z) @ v
    (out * torch.from_numpy(x["dout"])).sum().backward()
    got, lse = oracle.forward(x["q"], x["k"], x["v"], x["mask"], N=3, causal=causal, dropout=drop)
    assert np.abs(got - out.detach().numpy()).max() < 1e-12
    assert np.abs(lse - torch.logsumexp(s, dim=-1).detach().numpy()).max() < 1e-12
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=3, causal=causal, dropout=drop)
    for name, a, t in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        assert np.abs(a - t.grad.numpy()).max() < 1e-12, name


def test_dropout_does_not_depend_on_n_or_the_rank_split():
    x = small(B=1, H=2, L=64, d=8, seed=4, valid=(50, 64))
    drop = (0.25, 11, 0)
    ref, _ = oracle.forward(x["q"], x["k"], x["v"], x["mask"], N=1, dropout=drop)
    for N in (2, 4, 8, 16, 64):
        o, _ = oracle.forward(x["q"], x["k"], x["v"], x["mask"], N=N, dropout=drop)
        assert np.abs(o - ref).max() < 1e-13
    rows = np.arange(24, 32)   # rank 3 of N = 8
    o, _ = oracle.forward(x["q"][:, :, rows], x["k"], x["v"], x["mask"], N=8, qpos=rows, dropout=drop)
    assert np.abs(o - ref[:, :, rows]).max() < 1e-13
    g1 = oracle.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=1, dropout=drop)
    g8 = oracle.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=8, dropout=drop)
    for a, b in zip(g1, g8):
        assert np.abs(a - b).max() < 1e-13


def test_mean_over_seeds_tends_to_the_plain_output():
    """E[Z] = 1, so the output averaged over independent masks converges to
    the plain output (checked against the sample's own standard error)."""
    x = small(B=1, H=1, L=32, d=4, seed=5, valid=None)
    plain, _ = oracle.forward(x["q"], x["k"], x["v"], None, N=4)
    outs = np.stack([oracle.forward(x["q"], x["k"], x["v"], None, N=4, dropout=(0.4, s))[0] for s in range(600)])
    mean, se = outs.mean(0), outs.std(0, ddof=1) / np.sqrt(len(outs))
    z = np.abs(mean - plain) / np.maximum(se, 1e-12)
    assert z.max() < 5.5


def test_dropout_backward_finite_differences():
    """Central differences of <O, dO> in fp64 on the B=1 H=1 L=32 d=64 N=8
    slice with key padding (the keep decisions depend on positions only)."""
    w = rsa_inputs.WORKLOADS["backward_fd"]
    x = rsa_inputs.workload_inputs(w)
    drop = (0.2, 31337, 2)
    grads = oracle.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=w.N, dropout=drop)
    h = 1e-6
    rng = np.random.default_rng(0)
    for gi, name in enumerate(("q", "k", "v")):
        flat = x[name].reshape(-1)
        for idx in rng.choice(flat.size, size=40, replace=False):
            vals = []
            for sgn in (1, -1):
                y = {n: x[n].copy() for n in ("q", "k", "v")}
                y[name].reshape(-1)[idx] += sgn * h
                o, _ = oracle.forward(y["q"], y["k"], y["v"], x["mask"], N=w.N, dropout=drop)
                vals.append((o * x["dout"]).sum())
            fd = (vals[0] - vals[1]) / (2 * h)
            an = grads[gi].reshape(-1)[idx]
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, idx, fd, an)
