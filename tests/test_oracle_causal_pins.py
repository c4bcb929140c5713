"""Pins of the oracle's causal variant (the row at position i sees keys j <= i).

The pages do not describe a causal mask; the variant follows the standard
autoregressive definition. It is pinned to: the 50-digit decimal brute force
evaluated row by row on the keys 0..i only (no mask semantics involved),
torch's fp64 scaled_dot_product_attention with is_causal and its autograd
(the N = 1 library special case), closed forms for the first row and the
last key, the last row equalling the non-causal result, N-independence, and
central finite differences of <O, dO>.
"""

import numpy as np
import pytest
import torch

import rsa_inputs
from oracle import brute


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def divisors(n):
    return [x for x in range(1, n + 1) if n % x == 0]


@pytest.mark.parametrize("L,d,masked", [(1, 2, False), (4, 2, False), (6, 4, True), (12, 4, True)])
def test_causal_matches_rowwise_decimal_brute_force(oracle_lib, L, d, masked):
    B, H = 2, 1
    q, k, v = rand((B, H, L, d), 50 + L), rand((B, H, L, d), 60 + L), rand((B, H, L, d), 70 + L)
    mask = None
    if masked:
        mask = (np.random.default_rng(L).random((B, L)) < 0.7).astype(np.uint8)
        mask[:, 0] = 0   # the first row then has no valid key
    want = np.zeros((B, H, L, d))
    want_lse = np.full((B, H, L), -np.inf)
    for i in range(L):
        sub_mask = None if mask is None else mask[:, :i + 1]
        o, l = brute.attention(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], sub_mask)
        want[:, :, i], want_lse[:, :, i] = o[:, :, 0], l[:, :, 0]
    for N in divisors(L):
        out, lse = oracle_lib.forward(q, k, v, mask, N=N, causal=True)
        assert np.abs(out - want).max() <= 1e-13 * max(1.0, np.abs(want).max()), N
        fin = np.isfinite(want_lse)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.abs(lse[fin] - want_lse[fin]).max(initial=0.0) <= 1e-13 * 10


@pytest.mark.parametrize("masked", [False, True])
def test_causal_matches_torch_sdpa_fp64(oracle_lib, masked):
    B, H, L, d = 2, 2, 40, 8
    q, k, v, g = (rand((B, H, L, d), s) for s in (81, 82, 83, 84))
    mask = rsa_inputs.prefix_mask([33, 40], L) if masked else None
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    if mask is None:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    else:
        allowed = torch.tril(torch.ones(L, L, dtype=torch.bool))[None, None] & torch.tensor(mask != 0)[:, None, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed)
    (o * torch.tensor(g)).sum().backward()
    for N in (1, 2, 5, 8, 40):
        out, _ = oracle_lib.forward(q, k, v, mask, N=N, causal=True)
        assert np.abs(out - o.detach().numpy()).max() <= 1e-12, N
        dq, dk, dv = oracle_lib.backward(q, k, v, g, mask, N=N, causal=True)
        assert np.abs(dq - qt.grad.numpy()).max() <= 1e-12, N
        assert np.abs(dk - kt.grad.numpy()).max() <= 1e-12, N
        assert np.abs(dv - vt.grad.numpy()).max() <= 1e-12, N


def test_causal_closed_forms(oracle_lib):
    B, H, L, d = 1, 2, 16, 4
    q, k, v, g = (rand((B, H, L, d), s) for s in (91, 92, 93, 94))
    out, lse = oracle_lib.forward(q, k, v, None, N=4, causal=True)
    # the first row sees only key 0: its output is v_0, its lse the scaled score
    assert np.abs(out[:, :, 0] - v[:, :, 0]).max() <= 1e-15
    assert np.abs(lse[:, :, 0] - (q[:, :, 0] * k[:, :, 0]).sum(-1) / 2.0).max() <= 1e-14
    # the last row sees every key: the causal and full results coincide there
    full, full_lse = oracle_lib.forward(q, k, v, None, N=4)
    assert np.abs(out[:, :, -1] - full[:, :, -1]).max() <= 1e-14
    assert np.abs(out[:, :, :-1] - full[:, :, :-1]).max() > 1e-3
    # only the last row sees the last key: dV of that key is P * dO of that row
    dq, dk, dv = oracle_lib.backward(q, k, v, g, None, N=4, causal=True)
    p_last = np.exp((q[:, :, -1] * k[:, :, -1]).sum(-1) / 2.0 - full_lse[:, :, -1])
    assert np.abs(dv[:, :, -1] - p_last[..., None] * g[:, :, -1]).max() <= 1e-13


def test_causal_finite_differences(oracle_lib):
    B, H, L, d, N = 1, 1, 12, 4, 3
    q, k, v, g = (rand((B, H, L, d), s, 0.7) for s in (101, 102, 103, 104))
    mask = rsa_inputs.prefix_mask([10], L)
    dq, dk, dv = oracle_lib.backward(q, k, v, g, mask, N=N, causal=True)

    def loss(qq, kk, vv):
        o, _ = oracle_lib.forward(qq, kk, vv, mask, N=N, causal=True)
        return float((o * g).sum())

    eps = 1e-6
    rng = np.random.default_rng(5)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(rng.integers(s) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
