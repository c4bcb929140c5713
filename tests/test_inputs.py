"""The seeded input module: determinism, bf16 rounding and masks."""

import numpy as np
import torch

import rsa_inputs


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 3,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 65504.0, 1e-40, -3.4e38], np.float32),
    ])
    # values exactly half-way between two bf16 numbers exercise ties-to-even
    halfway = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, halfway, -halfway])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = rsa_inputs.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_bf16_bits_roundtrip():
    x = rsa_inputs.bf16_round(np.random.default_rng(1).standard_normal(1000).astype(np.float32))
    assert np.array_equal(rsa_inputs.bits_to_f32(rsa_inputs.bf16_bits(x)), x)


def test_inputs_are_deterministic_and_follow_the_recipe():
    a = rsa_inputs.make_inputs(2, 3, 64, 8, seed=7, dtype="bf16", valid_range=(40, 64), with_dout=True)
    b = rsa_inputs.make_inputs(2, 3, 64, 8, seed=7, dtype="bf16", valid_range=(40, 64), with_dout=True)
    for key in ("q", "k", "v", "dout", "mask", "valid_len"):
        assert np.array_equal(a[key], b[key])
    rng = np.random.Generator(np.random.PCG64(7))
    q = rng.standard_normal((2, 3, 64, 8)).astype(np.float32)
    assert np.array_equal(a["q"], rsa_inputs.bf16_round(q))
    for _ in ("k", "v", "dout"):
        rng.standard_normal((2, 3, 64, 8))
    vl = rng.integers(40, 65, size=2)
    assert np.array_equal(a["valid_len"], vl)
    assert np.array_equal(a["mask"].sum(axis=1), vl)
    assert a["mask"].dtype == np.uint8 and a["mask"].shape == (2, 64)


def test_workloads_are_consistent():
    for w in rsa_inputs.WORKLOADS.values():
        assert w.L % w.N == 0
        if w.valid_range is not None:
            lo, hi = w.valid_range
            assert 0 <= lo <= hi <= w.L
    share = rsa_inputs.WORKLOADS["rank_share"]
    assert share.Lq == share.L // share.N == 512
