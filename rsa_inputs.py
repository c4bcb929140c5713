"""Seeded synthetic inputs for Ring Self-Attention workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
bench. It holds none of the attention arithmetic: only random draws, a
bf16 round-to-nearest-even helper that turns fp32 draws into bf16-representable
values, the key-padding-mask constructor and the named workload shapes.

The review page of "Sequence Parallelism: Making 4D Parallelism Possible"
(ABSTRACT; proposed-method section) names no dataset: the method splits a
sequence of attention embeddings into chunks. The workloads below stand in
for those embeddings with i.i.d. normal draws at the shapes used to exercise
and measure the method.

Recipe (identical for every caller):
  * generator ``numpy.random.Generator(PCG64(seed))``;
  * ``standard_normal`` fp64 draws, in the order Q, K, V, then dO if asked;
  * each draw multiplied by the workload's scale (exact for 0.5) and cast to
    fp32; bf16 workloads are then rounded to bf16 by RNE (kept as fp32 values
    that are exactly representable in bf16);
  * if a valid-length range ``[lo, hi]`` is given, one integer per batch row
    is drawn with ``integers(lo, hi + 1, size=B)`` after the tensors, and key
    j of row b is valid iff ``j < valid_len[b]``.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits",
    "bits_to_f32",
    "Workload",
    "WORKLOADS",
    "make_inputs",
    "prefix_mask",
    "LayerShape",
    "LAYERS",
    "make_layer_inputs",
]


def bf16_round(x) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even).

    Returns fp32 values that are exactly representable in bf16. Inputs must be
    finite (the generator never produces NaN or Inf).
    """
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)
    return r.astype(np.uint32).view(np.float32).reshape(x32.shape)


def bf16_bits(x) -> np.ndarray:
    """The 16-bit patterns of bf16-representable fp32 values (upper halves)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-representable; call bf16_round first")
    return (u >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 values exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def prefix_mask(valid_len, L: int) -> np.ndarray:
    """Key-padding mask [B, L] uint8: key j of row b is valid iff j < valid_len[b]."""
    vl = np.asarray(valid_len, dtype=np.int64).reshape(-1, 1)
    return (np.arange(L, dtype=np.int64)[None, :] < vl).astype(np.uint8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named RSA workload: shapes, element type, scale, mask and seed."""

    name: str
    B: int
    H: int
    L: int
    d: int
    N: int
    dtype: str  # "f32" or "bf16"
    seed: int
    scale: float = 1.0
    valid_range: Optional[Tuple[int, int]] = None
    rank: Optional[int] = None  # one rank's share only (Q holds L/N rows)
    backward: bool = False
    description: str = ""

    @property
    def Lc(self) -> int:
        return self.L // self.N

    @property
    def Lq(self) -> int:
        return self.Lc if self.rank is not None else self.L


# Named workloads. "share" workloads hold only one rank's query rows (L/N of
# them) against all L keys, exactly as one device of the ring sees them.
WORKLOADS = {
    "fp32_small": Workload(
        "fp32_small", B=1, H=2, L=256, d=64, N=4, dtype="f32", seed=1,
        description="fp32, B=1 H=2 L=256 d=64, N=4 chunks of 64, no mask"),
    "bert_base": Workload(
        "bert_base", B=8, H=12, L=512, d=64, N=4, dtype="bf16", seed=2,
        valid_range=(384, 512),
        description="bf16 BERT-Base-shaped, B=8 H=12 L=512 d=64, N=4, key padding"),
    "long_seq": Workload(
        "long_seq", B=2, H=12, L=8192, d=64, N=16, dtype="bf16", seed=3,
        description="bf16 long sequence, B=2 H=12 L=8192 d=64, N=16 chunks of 512, no mask"),
    "rank_share": Workload(
        "rank_share", B=1, H=16, L=32768, d=128, N=64, dtype="bf16", seed=4,
        scale=0.5, valid_range=(24576, 32768), rank=0,
        description="bf16 one rank's share: 512 query rows vs 32768 keys in 64 chunks, "
                    "H=16 d=128, N(0,1)*0.5, key padding"),
    "backward": Workload(
        "backward", B=4, H=12, L=4096, d=64, N=8, dtype="bf16", seed=5,
        valid_range=(3072, 4096), backward=True,
        description="bf16 backward, B=4 H=12 L=4096 d=64, N=8, key padding"),
    "backward_fd": Workload(
        "backward_fd", B=1, H=1, L=32, d=64, N=8, dtype="f64", seed=6,
        valid_range=(24, 32), backward=True,
        description="fp64 finite-difference slice, B=1 H=1 L=32 d=64, N=8"),
}


def plant_score_jumps(x: dict, jump: float, positions) -> dict:
    """Keys that outscore every other key by a chosen margin.

    With n = len(positions) (at most d), every query row gets q[..., :n] = 2
    and the key at positions[i] gets k[..., positions[i], i] =
    (jump + i) * sqrt(d) / 2, so its score (after the 1/sqrt(d) scale)
    exceeds the row's other scores by about jump + i natural units when Q
    and K are otherwise drawn small (scale 0.5). Each planted key is large in
    its own component: keys that shared one large component would make dQ a
    small difference of large terms, which no bf16 dS operand resolves.
    Values stay bf16-representable. Modifies and returns x.
    """
    d = x["q"].shape[-1]
    n = len(positions)
    if n > d:
        raise ValueError("at most d planted keys")
    x["q"][..., :n] = 2.0
    for i, pos in enumerate(positions):
        x["k"][..., pos, i] = (jump + i) * np.sqrt(d) / 2.0
    x["q"] = bf16_round(x["q"])
    x["k"] = bf16_round(x["k"])
    return x


def make_inputs(B: int, H: int, L: int, d: int, seed: int, dtype: str = "bf16",
                scale: float = 1.0, valid_range: Optional[Tuple[int, int]] = None,
                Lq: Optional[int] = None, with_dout: bool = False) -> dict:
    """Draw seeded Q, K, V (and dO) following the module's recipe.

    Q is [B, H, Lq, d] (Lq defaults to L); K and V are [B, H, L, d]; dO has
    Q's shape. Returns numpy arrays: fp32 for "f32" and
    "bf16" (bf16-representable values for the latter), fp64 for "f64". The
    mask is None when ``valid_range`` is None.
    """
    if dtype not in ("f32", "bf16", "f64"):
        raise ValueError(f"unknown dtype {dtype!r}")
    Lq = L if Lq is None else Lq
    rng = np.random.Generator(np.random.PCG64(seed))

    def draw(shape):
        x = rng.standard_normal(shape) * scale
        if dtype == "f64":
            return x
        x = x.astype(np.float32)
        return bf16_round(x) if dtype == "bf16" else x

    out = {"q": draw((B, H, Lq, d)), "k": draw((B, H, L, d)), "v": draw((B, H, L, d))}
    out["dout"] = draw((B, H, Lq, d)) if with_dout else None
    if valid_range is not None:
        lo, hi = valid_range
        valid_len = rng.integers(lo, hi + 1, size=B)
        out["valid_len"] = valid_len
        out["mask"] = prefix_mask(valid_len, L)
    else:
        out["valid_len"] = None
        out["mask"] = None
    return out


def workload_inputs(w: Workload) -> dict:
    """Inputs of a named workload, following the module's recipe."""
    return make_inputs(w.B, w.H, w.L, w.d, w.seed, w.dtype, w.scale, w.valid_range,
                       Lq=w.Lq, with_dout=w.backward)


# ---------------------------------------------------------------------------
# The sequence-parallel layer around RSA: the token-local steps on either side
# of the attention (QKV projection, output projection, two fully connected
# layers with GeLU, residual sums and layer normalisation). Inputs are a
# hidden-state tensor x [B, L, E] and random-initialised weights in the
# shapes of a BERT-style encoder layer (E = H * d, F = 4 E):
#   w_qkv [3E, E], b_qkv [3E]   rows 0..E-1 give Q, E..2E-1 K, 2E..3E-1 V,
#                               head h owning rows h*d .. h*d + d - 1 of each
#   w_o   [E, E],  b_o   [E]
#   ln1_gamma, ln1_beta [E]
#   w_ff1 [F, E],  b_ff1 [F]
#   w_ff2 [E, F],  b_ff2 [E]
#   ln2_gamma, ln2_beta [E]
# Recipe: generator PCG64(seed); standard-normal fp64 draws in the order x,
# w_qkv, b_qkv, w_o, b_o, ln1_gamma, ln1_beta, w_ff1, b_ff1, w_ff2, b_ff2,
# ln2_gamma, ln2_beta; x is N(0,1), weight matrices and biases N(0,1) * 0.02,
# gammas 1 + N(0,1) * 0.1, betas N(0,1) * 0.1; matrices and x are rounded to
# bf16 (fp32 holders), vectors stay fp32. Then the valid lengths, as for
# make_inputs.


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One named layer workload: B, L, hidden size E, heads H, FFN width F, N."""

    name: str
    B: int
    L: int
    E: int
    H: int
    F: int
    N: int
    seed: int
    valid_range: Optional[Tuple[int, int]] = None
    description: str = ""

    @property
    def d(self) -> int:
        return self.E // self.H


LAYERS = {
    "layer_bert_base": LayerShape(
        "layer_bert_base", B=8, L=512, E=768, H=12, F=3072, N=4, seed=12, valid_range=(384, 512),
        description="BERT-Base-shaped layer, B=8 L=512 E=768 H=12 F=3072, N=4, key padding"),
    "layer_long_seq": LayerShape(
        "layer_long_seq", B=2, L=8192, E=768, H=12, F=3072, N=16, seed=13,
        description="long-sequence layer, B=2 L=8192 E=768 H=12 (d=64) F=3072, N=16, no mask"),
}


def make_layer_inputs(B: int, L: int, E: int, H: int, F: int, seed: int,
                      valid_range: Optional[Tuple[int, int]] = None) -> dict:
    """Draw the layer's input x and weights following the recipe above."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def mat(shape, scale):
        return bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))

    def vec(n, scale, offset=0.0):
        return (offset + rng.standard_normal(n) * scale).astype(np.float32)

    out = {"x": mat((B, L, E), 1.0)}
    out["w_qkv"] = mat((3 * E, E), 0.02)
    out["b_qkv"] = vec(3 * E, 0.02)
    out["w_o"] = mat((E, E), 0.02)
    out["b_o"] = vec(E, 0.02)
    out["ln1_gamma"] = vec(E, 0.1, 1.0)
    out["ln1_beta"] = vec(E, 0.1)
    out["w_ff1"] = mat((F, E), 0.02)
    out["b_ff1"] = vec(F, 0.02)
    out["w_ff2"] = mat((E, F), 0.02)
    out["b_ff2"] = vec(E, 0.02)
    out["ln2_gamma"] = vec(E, 0.1, 1.0)
    out["ln2_beta"] = vec(E, 0.1)
    if valid_range is not None:
        lo, hi = valid_range
        out["valid_len"] = rng.integers(lo, hi + 1, size=B)
        out["mask"] = prefix_mask(out["valid_len"], L)
    else:
        out["valid_len"] = None
        out["mask"] = None
    return out


def layer_inputs(w: LayerShape) -> dict:
    """Inputs of a named layer workload."""
    return make_layer_inputs(w.B, w.L, w.E, w.H, w.F, w.seed, w.valid_range)
