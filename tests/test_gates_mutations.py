"""The parity gates reject plausible mistakes at full workload sizes.

Each planted mistake is written here, in plain numpy on the CPU, as a wrong
variant of attention (a dropped ring step, the scale 1/d instead of
1/sqrt(d), an ignored key mask, softmax normalised per chunk, an online
softmax that never rescales, a zero output). The oracle gives the right
answer on sampled query rows of one head; each mistaken answer, rounded to
bf16 as a GPU output would be, must fail the gates, while the oracle's own
answer rounded to bf16 must pass them.
"""

import numpy as np
import pytest

import rsa_inputs
from gates import passes

ROWS = 128


def _head(w, b=0, h=0):
    x = rsa_inputs.workload_inputs(w)
    mask = x["mask"][b] if x["mask"] is not None else np.ones(w.L, np.uint8)
    return x["q"][b, h].astype(np.float64), x["k"][b, h].astype(np.float64), \
        x["v"][b, h].astype(np.float64), mask, x


def _positions(w):
    rng = np.random.default_rng(123)
    if w.rank is not None:
        base = w.rank * w.Lc
        return np.sort(rng.choice(w.Lc, ROWS, replace=False)), base
    return np.sort(rng.choice(w.L, ROWS, replace=False)), 0


def _mistakes(q, k, v, mask, pos, w):
    """Wrong attention variants for query rows q (absolute positions pos)."""
    d, N, Lc = w.d, w.N, w.Lc
    valid = mask != 0
    s = (q @ k.T) / np.sqrt(d)
    chunk_of = np.arange(w.L) // Lc

    def softmax_v(scores, keep):
        sc = np.where(keep, scores, -np.inf)
        m = sc.max(axis=1, keepdims=True)
        e = np.where(keep, np.exp(sc - m), 0.0)
        return (e / e.sum(axis=1, keepdims=True)) @ v

    out = {}
    out["zero output"] = np.zeros((len(pos), d))
    n = pos // Lc
    # drop the first ring step whose chunk holds a valid key (a rank can own,
    # or first receive, a chunk that is all padding)
    dropped = np.empty(len(pos), dtype=np.int64)
    for i in range(len(pos)):
        for t in range(N):
            c = (n[i] - t) % N
            if valid[chunk_of == c].any():
                dropped[i] = c
                break
    skip = chunk_of[None, :] != dropped[:, None]
    out["skip one ring step"] = softmax_v(s, valid[None, :] & skip)
    out["scale 1/d"] = softmax_v((q @ k.T) / d, np.broadcast_to(valid, s.shape))
    if not valid.all():
        out["ignore mask"] = softmax_v(s, np.ones_like(s, bool))
    # softmax normalised within each chunk, then averaged over the chunks
    acc = np.zeros((len(pos), d))
    used = 0
    for c in range(N):
        keep = valid & (chunk_of == c)
        if keep.any():
            acc += softmax_v(s, np.broadcast_to(keep, s.shape))
            used += 1
    out["per-chunk softmax"] = acc / used
    # online softmax over the ring that never rescales what it has summed
    o = np.zeros((len(pos), d))
    l = np.zeros((len(pos), 1))
    m = np.full((len(pos), 1), -np.inf)
    for i in range(len(pos)):
        for t in range(N):
            c = (n[i] - t) % N
            keep = valid & (chunk_of == c)
            if not keep.any():
                continue
            sc = s[i, keep]
            m[i] = max(m[i, 0], sc.max())
            e = np.exp(sc - m[i])
            l[i] += e.sum()
            o[i] += e @ v[keep]
    out["online softmax without rescale"] = o / l
    return out


@pytest.mark.parametrize("name", ["bert_base", "long_seq", "rank_share"])
def test_forward_mistakes_fail_the_gates(oracle_lib, name):
    w = rsa_inputs.WORKLOADS[name]
    q_all, k, v, mask, _ = _head(w)
    rows, base = _positions(w)
    q = q_all[rows]
    pos = rows + base
    want, _ = oracle_lib.forward(q[None, None], k[None, None], v[None, None],
                                 mask[None], N=w.N, qpos=pos)
    want = want[0, 0]
    assert passes(rsa_inputs.bf16_round(want.astype(np.float32)), want, "bf16")
    for label, wrong in _mistakes(q, k, v, mask, pos, w).items():
        assert not passes(rsa_inputs.bf16_round(wrong.astype(np.float32)), want, "bf16"), label


def _backward_mistakes(q, k, v, g, mask, w):
    d, N, Lc = w.d, w.N, w.Lc
    valid = mask != 0
    s = np.where(valid[None, :], (q @ k.T) / np.sqrt(d), -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o = p @ v
    D = (g * o).sum(axis=1, keepdims=True)
    dp = g @ v.T
    scale = 1.0 / np.sqrt(d)
    chunk_of = np.arange(w.L) // Lc
    qchunk = np.arange(w.L) // Lc
    out = {}
    ds = p * (dp - D)
    out["dq: no D term"] = scale * (p * dp) @ k
    out["dk: no D term"] = scale * (p * dp).T @ q
    out["dk: scale 1/d"] = (ds.T @ q) / d
    out["dv: skip one query chunk"] = (p * (qchunk[:, None] != 1)).T @ g
    out["dq: skip one ring step"] = scale * (ds * (chunk_of[None, :] != ((qchunk - 1) % N)[:, None])) @ k
    return out, {"dq": scale * ds @ k, "dk": scale * ds.T @ q, "dv": p.T @ g}


def test_backward_mistakes_fail_the_gates(oracle_lib):
    w = rsa_inputs.WORKLOADS["backward"]
    x = rsa_inputs.workload_inputs(w)
    b, h = 1, 5
    q, k, v, g = (x[n][b, h].astype(np.float64) for n in ("q", "k", "v", "dout"))
    mask = x["mask"][b]
    dq, dk, dv = oracle_lib.backward(q[None, None], k[None, None], v[None, None],
                                     g[None, None], mask[None], N=w.N)
    want = {"dq": dq[0, 0], "dk": dk[0, 0], "dv": dv[0, 0]}
    wrong, dense = _backward_mistakes(q, k, v, g, mask, w)
    for key in want:  # the dense numpy gradients agree with the oracle
        assert np.abs(dense[key] - want[key]).max() <= 1e-10
        assert passes(rsa_inputs.bf16_round(want[key].astype(np.float32)), want[key], "bf16", grad=True)
    for label, val in wrong.items():
        key = label.split(":")[0]
        assert not passes(rsa_inputs.bf16_round(val.astype(np.float32)), want[key], "bf16", grad=True), label
