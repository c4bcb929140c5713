"""fp64 CPU oracle of the sequence-parallel layer around RSA -- test
infrastructure only (the test suite, the smoke check and the bench's CPU
baseline may import it; the HIP library never does).

What it computes. The review page of "Sequence Parallelism: Making 4D
Parallelism Possible" (ABSTRACT) places RSA inside a Transformer, each device
holding one chunk of the sequence; every step of the layer other than the
attention acts on one token at a time, so it runs on each chunk without any
exchange. The page "一文捋順千億模型訓練技術：流水線并行、張量并行和3D并行"
(section 二, 1D tensor parallelism, parts (2) and (3)) describes the other
two blocks of the layer: two fully connected layers with a GeLU between them,
and multi-head attention whose heads are independent. The residual sums and
the layer normalisations are not on the pages; the oracle takes the plainest
reading, the post-normalisation encoder layer of BERT:

    Q, K, V = split_heads(x W_qkv^T + b_qkv)
    O       = attention(Q, K, V, key_mask)          RSA, oracle.forward
    A1      = merge_heads(O) W_o^T + b_o + x
    h1      = LayerNorm(A1; gamma1, beta1)
    F1      = GeLU(h1 W_1^T + b_1)                  GeLU(z) = z Phi(z), exact erf form
    A2      = F1 W_2^T + b_2 + h1
    y       = LayerNorm(A2; gamma2, beta2)

LayerNorm(z) = (z - mean(z)) / sqrt(var(z) + eps) * gamma + beta over the
hidden dimension, var the population variance, eps = 1e-12 (BERT's).

Every step is evaluated in fp64 with numpy (a matmul, a sum, erf). With
``store="bf16"`` the activations the layer keeps between its steps (Q, K, V,
O, A1, h1, F1, A2, y) are rounded to bf16 (nearest, ties to even) exactly
where a bf16 implementation stores them; with ``store=None`` nothing is
rounded (the plain definition, which the pins check).
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np
from scipy.special import erf

from . import forward as attention_forward

LN_EPS = 1e-12


def round_bf16(x) -> np.ndarray:
    """fp64 values rounded to the nearest bf16 value (8 significant bits,
    ties to even), returned as fp64. Written from the definition: x = m 2^e
    with 0.5 <= |m| < 1, and m is rounded to a multiple of 2^-8."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def linear(a, w, b) -> np.ndarray:
    """a [..., K] times w [N, K] transposed, plus b [N] (a fully connected layer)."""
    return np.asarray(a, np.float64) @ np.asarray(w, np.float64).T + np.asarray(b, np.float64)


def gelu(z) -> np.ndarray:
    """GeLU(z) = z * Phi(z) = z/2 * (1 + erf(z / sqrt 2))."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def layernorm(z, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    """Normalise over the last axis to zero mean and unit (population)
    variance, then scale by gamma and shift by beta."""
    z = np.asarray(z, dtype=np.float64)
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    return (z - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def split_heads(t, H: int) -> np.ndarray:
    """[B, L, E] -> [B, H, L, d]: head h takes features h*d .. h*d + d - 1."""
    B, L, E = t.shape
    return np.ascontiguousarray(t.reshape(B, L, H, E // H).transpose(0, 2, 1, 3))


def merge_heads(o) -> np.ndarray:
    """[B, H, L, d] -> [B, L, H*d], the inverse of split_heads."""
    B, H, L, d = o.shape
    return np.ascontiguousarray(o.transpose(0, 2, 1, 3).reshape(B, L, H * d))


def qkv_projection(x, w_qkv, b_qkv, H: int, store: Optional[str] = "bf16"):
    """Q, K, V [B, H, L, d] from x [B, L, E]."""
    E = x.shape[-1]
    t = linear(x, w_qkv, b_qkv)
    q, k, v = (split_heads(t[..., i * E:(i + 1) * E], H) for i in range(3))
    if store == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


def layer_forward(inp: dict, H: int, N: int, store: Optional[str] = "bf16", rows=None,
                  eps: float = LN_EPS) -> dict:
    """The layer's output y [B, L, E] and its intermediates.

    inp holds x and the weights (names as in the seeded layer inputs) and
    mask [B, L] or None. ``rows`` (optional) restricts everything after the
    key/value projection to those token positions of every batch row: K and V
    still cover the whole sequence, so the rows' attention is exact.
    """
    rnd = round_bf16 if store == "bf16" else (lambda a: np.asarray(a, np.float64))
    x = np.asarray(inp["x"], np.float64)
    B, L, E = x.shape
    q, k, v = qkv_projection(x, inp["w_qkv"], inp["b_qkv"], H, store)
    qpos = None
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q = q[:, :, rows]
        x = x[:, rows]
        qpos = rows
    o, lse = attention_forward(q, k, v, inp.get("mask"), N=N, qpos=qpos)
    o = rnd(o)
    a1 = rnd(linear(merge_heads(o), inp["w_o"], inp["b_o"]) + x)
    h1 = rnd(layernorm(a1, inp["ln1_gamma"], inp["ln1_beta"], eps))
    f1 = rnd(gelu(linear(h1, inp["w_ff1"], inp["b_ff1"])))
    a2 = rnd(linear(f1, inp["w_ff2"], inp["b_ff2"]) + h1)
    y = rnd(layernorm(a2, inp["ln2_gamma"], inp["ln2_beta"], eps))
    return {"q": q, "k": k, "v": v, "o": o, "lse": lse, "a1": a1, "h1": h1, "f1": f1, "a2": a2, "y": y}
