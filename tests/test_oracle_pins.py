"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

The pages (review of "Sequence Parallelism: Making 4D Parallelism Possible",
ABSTRACT and proposed-method section) state that RSA computes the attention
output by circulating key and value chunks around a ring; they print no
formula and no worked example. The oracle's reading is plain scaled-dot-product
attention with a key-padding mask, evaluated in ring order. These tests pin it
to: hand-derived closed forms (tests/golden), a 50-digit decimal brute force,
torch's fp64 CPU attention and autograd (the N = 1 textbook special case),
invariants of softmax attention, and central finite differences.
"""

import json
import math
import os
import re
from decimal import Decimal, localcontext

import numpy as np
import pytest
import torch

import rsa_inputs
from oracle import brute

HERE = os.path.dirname(os.path.abspath(__file__))


def divisors(n):
    return [x for x in range(1, n + 1) if n % x == 0]


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ----------------------------------------------------------------- golden ---

def _eval_expr(expr: str) -> float:
    """Evaluate a closed form in 50-digit decimal (E = Euler's number)."""
    with localcontext() as ctx:
        ctx.prec = 50
        env = {"E": Decimal(1).exp(), "ln": lambda x: Decimal(x).ln(), "D": Decimal}
        # integer literals become Decimals so that every division is exact to 50 digits
        src = re.sub(r"(?<![\w.])(\d+)(?![\w.])", r"D(\1)", expr)
        return float(eval(src, {"__builtins__": {}}, env))  # noqa: S307


def test_golden_closed_forms(oracle_lib):
    with open(os.path.join(HERE, "golden", "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["k"], dtype=np.float64)
        v = np.array(case["v"], dtype=np.float64)
        mask = None if case["mask"] is None else np.array(case["mask"], dtype=np.uint8)
        qpos = case.get("q_rows")
        for N in case["N"]:
            out, lse = oracle_lib.forward(q, k, v, mask, N=N, qpos=qpos)
            for item in case["out"]:
                want = item["value"]
                assert abs(_eval_expr(item["expr"]) - want) < 1e-15, (case["name"], item)
                assert abs(out[tuple(item["index"])] - want) < 1e-15, (case["name"], N, item)
            for item in case["lse"]:
                want = item["value"]
                assert abs(_eval_expr(item["expr"]) - want) < 1e-15, (case["name"], item)
                assert abs(lse[tuple(item["index"])] - want) < 1e-14, (case["name"], N, item)


# ------------------------------------------------------------ brute force ---

@pytest.mark.parametrize("L,d", [(1, 1), (2, 2), (3, 4), (5, 2), (8, 8), (16, 4)])
def test_forward_matches_decimal_brute_force(oracle_lib, L, d):
    B, H = 2, 2
    q = rand((B, H, L, d), 10 + L)
    k = rand((B, H, L, d), 20 + L)
    v = rand((B, H, L, d), 30 + L)
    rng = np.random.default_rng(40 + L)
    mask = (rng.random((B, L)) < 0.7).astype(np.uint8)
    mask[0, :] = 0
    mask[0, rng.integers(L)] = 1  # exactly one valid key in row 0
    want, want_lse = brute.attention(q, k, v, mask)
    for N in divisors(L):
        out, lse = oracle_lib.forward(q, k, v, mask, N=N)
        scale = max(1.0, np.abs(want).max())
        assert np.abs(out - want).max() <= 1e-13 * scale, N
        fin = np.isfinite(want_lse)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.abs(lse[fin] - want_lse[fin]).max(initial=0.0) <= 1e-13 * max(1.0, np.abs(want_lse[fin]).max(initial=1.0))


def test_fully_masked_rows_are_zero(oracle_lib):
    B, H, L, d = 2, 1, 8, 4
    q, k, v = rand((B, H, L, d), 1), rand((B, H, L, d), 2), rand((B, H, L, d), 3)
    mask = np.ones((B, L), dtype=np.uint8)
    mask[1] = 0
    for N in divisors(L):
        out, lse = oracle_lib.forward(q, k, v, mask, N=N)
        assert np.all(out[1] == 0.0) and np.all(np.isneginf(lse[1]))
        dq, dk, dv = oracle_lib.backward(q, k, v, rand((B, H, L, d), 4), mask, N=N)
        assert np.all(dq[1] == 0) and np.all(dk[1] == 0) and np.all(dv[1] == 0)


# ------------------------------------------- library special case (N = 1) ---

def _torch_attention(q, k, v, mask):
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    am = None
    if mask is not None:
        am = torch.tensor(mask != 0)[:, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am)
    return qt, kt, vt, o


@pytest.mark.parametrize("masked", [False, True])
def test_matches_torch_sdpa_fp64(oracle_lib, masked):
    B, H, L, d = 2, 3, 48, 16
    q, k, v, g = (rand((B, H, L, d), s) for s in (5, 6, 7, 8))
    mask = None
    if masked:
        mask = rsa_inputs.prefix_mask([37, 48], L)
    qt, kt, vt, o = _torch_attention(q, k, v, mask)
    (o * torch.tensor(g)).sum().backward()
    out, _ = oracle_lib.forward(q, k, v, mask, N=1)
    assert np.abs(out - o.detach().numpy()).max() <= 1e-12
    dq, dk, dv = oracle_lib.backward(q, k, v, g, mask, N=1)
    assert np.abs(dq - qt.grad.numpy()).max() <= 1e-12
    assert np.abs(dk - kt.grad.numpy()).max() <= 1e-12
    assert np.abs(dv - vt.grad.numpy()).max() <= 1e-12
    # every ring size gives the same result up to rounding
    for N in (2, 3, 4, 6, 8, 12, 16, 24, 48):
        out_n, _ = oracle_lib.forward(q, k, v, mask, N=N)
        assert np.abs(out_n - out).max() <= 1e-13
        dq_n, dk_n, dv_n = oracle_lib.backward(q, k, v, g, mask, N=N)
        for a, b in ((dq_n, dq), (dk_n, dk), (dv_n, dv)):
            assert np.abs(a - b).max() <= 1e-13


# -------------------------------------------------------------- invariants ---

def test_n_independence_every_divisor(oracle_lib):
    B, H, L, d = 1, 2, 256, 16
    q, k, v = rand((B, H, L, d), 11), rand((B, H, L, d), 12), rand((B, H, L, d), 13)
    mask = rsa_inputs.prefix_mask([201], L)
    ref, ref_lse = oracle_lib.forward(q, k, v, mask, N=1)
    for N in divisors(L):
        out, lse = oracle_lib.forward(q, k, v, mask, N=N)
        assert np.abs(out - ref).max() <= 1e-13, N
        assert np.abs(lse - ref_lse).max() <= 1e-13, N


def test_rows_sum_to_one(oracle_lib):
    """With V = 1 every output entry is the row sum of the attention weights."""
    B, H, L, d = 2, 2, 64, 8
    q, k = rand((B, H, L, d), 21, 3.0), rand((B, H, L, d), 22, 3.0)
    v = np.ones((B, H, L, d))
    mask = rsa_inputs.prefix_mask([64, 9], L)
    for N in (1, 4, 64):
        out, _ = oracle_lib.forward(q, k, v, mask, N=N)
        assert np.abs(out - 1.0).max() <= 1e-14


def test_constant_keys_give_mean_of_valid_values(oracle_lib):
    """All keys equal: every score of a row is the same, so the weights are
    uniform over the valid keys and O_i is the mean of the valid value rows;
    the gradient with respect to Q vanishes."""
    B, H, L, d = 2, 2, 96, 8
    q = rand((B, H, L, d), 31)
    krow = rand((1, 1, 1, d), 32)
    k = np.broadcast_to(krow, (B, H, L, d)).copy()
    v = rand((B, H, L, d), 33)
    valid = [96, 50]
    mask = rsa_inputs.prefix_mask(valid, L)
    for N in (1, 2, 3, 8, 96):
        out, _ = oracle_lib.forward(q, k, v, mask, N=N)
        for b in range(B):
            for h in range(H):
                mean = np.array([math.fsum(v[b, h, :valid[b], x]) / valid[b] for x in range(d)])
                assert np.abs(out[b, h] - mean[None, :]).max() <= 1e-14
        dq, _, _ = oracle_lib.backward(q, k, v, rand((B, H, L, d), 34), mask, N=N)
        assert np.abs(dq).max() <= 1e-13


def test_single_valid_key_copies_its_value(oracle_lib):
    B, H, L, d = 1, 2, 32, 8
    q, k, v = rand((B, H, L, d), 41), rand((B, H, L, d), 42), rand((B, H, L, d), 43)
    j = 19
    mask = np.zeros((B, L), dtype=np.uint8)
    mask[0, j] = 1
    g = rand((B, H, L, d), 44)
    for N in (1, 2, 4, 8, 32):
        out, _ = oracle_lib.forward(q, k, v, mask, N=N)
        assert np.array_equal(out, np.broadcast_to(v[:, :, j:j + 1, :], out.shape))
        dq, dk, dv = oracle_lib.backward(q, k, v, g, mask, N=N)
        others = np.ones(L, bool)
        others[j] = False
        assert np.all(dk[:, :, others] == 0) and np.all(dv[:, :, others] == 0)
        assert np.abs(dv[:, :, j] - g.sum(axis=2)).max() <= 1e-13
        assert np.abs(dk[:, :, j]).max() <= 1e-13  # weight is 1 whatever the score
        assert np.abs(dq).max() <= 1e-13


def test_shift_invariance_of_keys(oracle_lib):
    """K_j -> K_j + u shifts every score of row i by q_i.u/sqrt(d), which the
    softmax removes; a large u stresses the max subtraction."""
    B, H, L, d = 1, 2, 64, 16
    q, k, v = rand((B, H, L, d), 51), rand((B, H, L, d), 52), rand((B, H, L, d), 53)
    u = rand((d,), 54, 40.0)
    mask = rsa_inputs.prefix_mask([50], L)
    ref, _ = oracle_lib.forward(q, k, v, mask, N=4)
    out, _ = oracle_lib.forward(q, k + u, v, mask, N=4)
    assert np.abs(out - ref).max() <= 1e-12


def test_permutation_equivariance(oracle_lib):
    B, H, L, d = 1, 2, 48, 8
    q, k, v = rand((B, H, L, d), 61), rand((B, H, L, d), 62), rand((B, H, L, d), 63)
    mask = rsa_inputs.prefix_mask([40], L)
    ref, _ = oracle_lib.forward(q, k, v, mask, N=6)
    rng = np.random.default_rng(64)
    pk = rng.permutation(L)
    out, _ = oracle_lib.forward(q, k[:, :, pk], v[:, :, pk], mask[:, pk], N=6)
    assert np.abs(out - ref).max() <= 1e-13
    pq = rng.permutation(L)
    out, _ = oracle_lib.forward(q[:, :, pq], k, v, mask, N=6)
    assert np.abs(out - ref[:, :, pq]).max() <= 1e-13


def test_masked_keys_do_not_matter(oracle_lib):
    B, H, L, d = 2, 2, 64, 8
    q, k, v = rand((B, H, L, d), 71), rand((B, H, L, d), 72), rand((B, H, L, d), 73)
    mask = rsa_inputs.prefix_mask([33, 64], L)
    ref, ref_lse = oracle_lib.forward(q, k, v, mask, N=8)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 33:] = 1e4
    v2[0, :, 33:] = -1e4
    out, lse = oracle_lib.forward(q, k2, v2, mask, N=8)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


def test_rank_share_rows_match_full_sequence(oracle_lib):
    """One rank's share (its L/N query rows against all L keys) equals the
    same rows of the full output."""
    B, H, L, d, N = 1, 2, 64, 8, 8
    q, k, v = rand((B, H, L, d), 81), rand((B, H, L, d), 82), rand((B, H, L, d), 83)
    mask = rsa_inputs.prefix_mask([45], L)
    full, full_lse = oracle_lib.forward(q, k, v, mask, N=N)
    Lc = L // N
    for r in range(N):
        rows = np.arange(r * Lc, (r + 1) * Lc)
        out, lse = oracle_lib.forward(q[:, :, rows], k, v, mask, N=N, qpos=rows)
        assert np.array_equal(out, full[:, :, rows]) and np.array_equal(lse, full_lse[:, :, rows])


# ---------------------------------------------------------------- backward ---

def test_backward_finite_differences(oracle_lib):
    """Central differences of the loss <O, dO> on the fp64 slice
    (B=1, H=1, L=32, d=64, N=8, valid length drawn from [24, 32])."""
    w = rsa_inputs.WORKLOADS["backward_fd"]
    x = rsa_inputs.workload_inputs(w)
    q, k, v, g, mask = x["q"], x["k"], x["v"], x["dout"], x["mask"]
    assert x["valid_len"][0] < w.L  # the slice exercises the mask
    dq, dk, dv = oracle_lib.backward(q, k, v, g, mask, N=w.N)
    h = 1e-6

    def loss(qq, kk, vv):
        out, _ = oracle_lib.forward(qq, kk, vv, mask, N=w.N)
        return float(np.sum(out * g))

    for name, base, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus, minus = base.copy(), base.copy()
            plus[idx] += h
            minus[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = plus, minus
            fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                       loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        err = np.abs(fd - grad).max() / np.abs(grad).max()
        assert err <= 1e-7, (name, err)


def test_backward_invariants(oracle_lib):
    B, H, L, d = 2, 2, 64, 16
    q, k, v, g = (rand((B, H, L, d), s) for s in (91, 92, 93, 94))
    valid = [64, 21]
    mask = rsa_inputs.prefix_mask(valid, L)
    dq, dk, dv = oracle_lib.backward(q, k, v, g, mask, N=4)
    # each softmax-Jacobian row sums to zero, so the key gradients sum to zero
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12
    # attention weights of a row sum to one, so the value gradients sum to dO
    assert np.abs(dv.sum(axis=2) - g.sum(axis=2)).max() <= 1e-12
    for b in range(B):
        assert np.all(dk[b, :, valid[b]:] == 0) and np.all(dv[b, :, valid[b]:] == 0)
