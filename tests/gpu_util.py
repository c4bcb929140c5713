"""Helpers for the GPU parity tests: upload seeded inputs, run the oracle on
the same rounded values, and sample rows at full workload sizes."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import rsa_inputs


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*args):
    """Name the case before a GPU step (flushed, so a hang still shows it)."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


PARITY_REPORT = []


def report(what: str, e: dict):
    """Record a parity result (errors() dict) for the end-of-run summary."""
    PARITY_REPORT.append((what, e["max_abs"], e["rel_fro"]))
    say(what, f"max-abs {e['max_abs']:.3e} rel-fro {e['rel_fro']:.3e}")


def to_dev(x: np.ndarray, dtype: str, dev) -> torch.Tensor:
    """Exact upload: fp32 values (bf16-representable for "bf16")."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(dev).contiguous()


def mask_dev(mask, dev):
    return None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).to(dev)


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def sample_rows(L: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct rows, always including the first and last."""
    rng = np.random.default_rng(seed)
    picks = rng.choice(L, size=min(count, L), replace=False)
    return np.unique(np.concatenate([picks, [0, L - 1]]))


def inputs(B, H, L, d, seed, dtype, scale=1.0, valid_range=None, Lq=None, with_dout=False):
    return rsa_inputs.make_inputs(B, H, L, d, seed, dtype, scale, valid_range, Lq=Lq, with_dout=with_dout)
