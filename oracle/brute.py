"""Dense attention in 50-digit decimal arithmetic -- test infrastructure only.

An independent evaluation of the definition the oracle follows (review page
of "Sequence Parallelism: Making 4D Parallelism Possible", ABSTRACT: the
method computes the ordinary self-attention output): for every query row,
O = softmax(q K^T / sqrt(d) + M) V over the whole key length at once, with no
chunking and no ring. Python's ``decimal`` gives correctly rounded sqrt and
exp, so for tiny inputs the result is exact to far below fp64 rounding.
"""

from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np


def attention(q, k, v, mask=None, digits: int = 50):
    """Return (out, lse) as float64 arrays; q [B,H,Lq,d], k, v [B,H,L,d].

    Rows without a valid key give out = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    L = k.shape[2]
    out = np.zeros((B, H, Lq, d), dtype=np.float64)
    lse = np.full((B, H, Lq), -np.inf, dtype=np.float64)
    with localcontext() as ctx:
        ctx.prec = digits
        scale = Decimal(1) / Decimal(d).sqrt()
        for b in range(B):
            valid = [True] * L if mask is None else [bool(mask[b][j]) for j in range(L)]
            for h in range(H):
                K = [[Decimal(float(x)) for x in k[b, h, j]] for j in range(L)]
                V = [[Decimal(float(x)) for x in v[b, h, j]] for j in range(L)]
                for i in range(Lq):
                    Q = [Decimal(float(x)) for x in q[b, h, i]]
                    s = {j: sum(Q[x] * K[j][x] for x in range(d)) * scale
                         for j in range(L) if valid[j]}
                    if not s:
                        continue
                    m = max(s.values())
                    e = {j: (s[j] - m).exp() for j in s}
                    total = sum(e.values())
                    for x in range(d):
                        out[b, h, i, x] = float(sum(e[j] * V[j][x] for j in s) / total)
                    lse[b, h, i] = float(m + total.ln())
    return out, lse
