"""Parity gates: how GPU outputs are compared with the fp64 oracle.

Two gates, both required:
  * max-abs: max |got - want| over every element, at most 1e-4 for fp32
    inputs and 2e-2 for bf16 inputs;
  * relative Frobenius: ||got - want||_F / ||want||_F, at most 1e-5 for fp32
    and 5e-3 for bf16 outputs (1e-2 for bf16 gradients, whose dS operand is
    rounded to bf16 before two further contractions).

The max-abs bound alone is vacuous where outputs are small (a one-rank share
at d = 128 with inputs scaled by 0.5 has max |O| near 0.015); the relative
gate is what rejects a dropped ring step, a wrong scale, an ignored mask or
per-chunk softmax normalisation (test_gates_mutations.py shows each of them
failing). Expected bf16 errors from rounding P and the output to bf16 are
near 1.5e-3 relative. Any NaN or Inf fails.
"""

from __future__ import annotations

import numpy as np

MAX_ABS = {"f32": 1e-4, "bf16": 2e-2}
# lse (natural log). The bf16 kernels sum the row's weights after rounding
# each to bf16 (so that the weights used sum to exactly the normaliser);
# round-to-nearest-even has a relative error of at most 2^-8 (7 stored
# fraction bits), so the sum, and with it exp(lse), is off by at most that
# factor: |d lse| <= -ln(1 - 2^-8) = 3.91e-3, reached only by rows with few
# visible keys. fp32: accumulation rounding only.
LSE_TOL = {"f32": 1e-5, "bf16": 4e-3}
REL_FRO = {"f32": 1e-5, "bf16": 5e-3}
REL_FRO_GRAD = {"f32": 1e-5, "bf16": 1e-2}


def errors(got, want) -> dict:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if got.shape != want.shape:
        raise ValueError(f"shape mismatch {got.shape} vs {want.shape}")
    finite = bool(np.all(np.isfinite(got)))
    diff = got - want
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(want.ravel()))
    num = float(np.linalg.norm(diff.ravel()))
    rel = num / denom if denom > 0 else (0.0 if num == 0 else np.inf)
    return {"finite": finite, "max_abs": max_abs, "rel_fro": rel}


def passes(got, want, dtype: str, grad: bool = False) -> bool:
    e = errors(got, want)
    rel_tol = (REL_FRO_GRAD if grad else REL_FRO)[dtype]
    return e["finite"] and e["max_abs"] <= MAX_ABS[dtype] and e["rel_fro"] <= rel_tol


def assert_parity(got, want, dtype: str, what: str = "", grad: bool = False) -> dict:
    e = errors(got, want)
    rel_tol = (REL_FRO_GRAD if grad else REL_FRO)[dtype]
    assert e["finite"], f"{what}: non-finite values"
    assert e["max_abs"] <= MAX_ABS[dtype], f"{what}: max-abs {e['max_abs']:.3e} > {MAX_ABS[dtype]}"
    assert e["rel_fro"] <= rel_tol, f"{what}: rel-Frobenius {e['rel_fro']:.3e} > {rel_tol}"
    return e
