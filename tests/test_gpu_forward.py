"""GPU parity of the RSA forward (full sequence and one rank's share)
against the fp64 oracle, through the C ABI.

Small cases compare every element and span several tiles plus a ragged tail;
the full-size workloads run in the launch configuration the bench times and
are checked on sampled query rows, which the oracle computes one by one
(rows are independent given all keys)."""

import numpy as np
import pytest
import torch

import rsa_inputs
import sequence_transformer_attention_rsa_amd as rsa
from gates import LSE_TOL, MAX_ABS, assert_parity
from gpu_util import device, report, from_dev, inputs, mask_dev, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu



def divisors(n):
    return [x for x in range(1, n + 1) if n % x == 0]


def gpu_forward(x, dtype, N, dev, return_lse=True):
    q, k, v = (to_dev(x[n], dtype, dev) for n in ("q", "k", "v"))
    out, lse = rsa.forward(q, k, v, mask_dev(x["mask"], dev), N=N, return_lse=True)
    torch.cuda.synchronize()
    return from_dev(out), lse.cpu().numpy().astype(np.float64)


def check_lse(got, want, dtype, what):
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: lse finiteness differs"
    if fin.any():
        err = np.abs(got[fin] - want[fin]).max()
        assert err <= LSE_TOL[dtype], f"{what}: lse max-abs {err:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,N,valid", [
    (256, 4, None),          # four chunks of one 64-key tile each
    (200, 5, (150, 200)),    # chunks of 40 keys: tiles straddle chunks, ragged tail
    (320, 8, (1, 320)),      # very short valid lengths possible
    (130, 13, None),         # chunks of 10 keys, 130 = 2 query tiles + 2 rows
    (64, 64, None),          # one key per chunk
    (128, 2, (90, 128)),     # two key tiles, one query tile
])
def test_forward_small_parity(oracle_lib, dtype, d, L, N, valid):
    dev = device()
    x = inputs(2, 3, L, d, seed=L + d + N, dtype=dtype, valid_range=valid)
    say("forward", dtype, d, L, N, valid)
    out, lse = gpu_forward(x, dtype, N, dev)
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=N)
    assert_parity(out, want, dtype, f"out {dtype} d={d} L={L} N={N}")
    check_lse(lse, want_lse, dtype, f"lse {dtype} d={d} L={L} N={N}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_every_ring_size(oracle_lib, dtype):
    """The result does not depend on N: every divisor of L = 256."""
    dev = device()
    L, d = 256, 64
    x = inputs(1, 2, L, d, seed=77, dtype=dtype, valid_range=(190, 190))
    want, _ = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=1)
    outs = []
    for N in divisors(L):
        say("forward ring size", dtype, N)
        out, _ = gpu_forward(x, dtype, N, dev)
        assert_parity(out, want, dtype, f"N={N}")
        outs.append(out)
    spread = max(np.abs(o - outs[0]).max() for o in outs)
    assert spread <= MAX_ABS[dtype] / 4


def test_fully_masked_rows_give_zeros(oracle_lib):
    dev = device()
    L, d = 192, 64
    x = inputs(2, 2, L, d, seed=5, dtype="bf16")
    mask = np.ones((2, L), np.uint8)
    mask[1] = 0
    x["mask"] = mask
    say("fully masked batch row")
    out, lse = gpu_forward(x, "bf16", 3, dev)
    assert np.all(out[1] == 0.0) and np.all(np.isneginf(lse[1]))
    want, _ = oracle_lib.forward(x["q"], x["k"], x["v"], mask, N=3)
    assert_parity(out, want, "bf16", "fully masked")


def test_masked_garbage_is_ignored_bitwise():
    dev = device()
    L, d = 384, 128
    x = inputs(2, 2, L, d, seed=6, dtype="bf16", valid_range=(100, 300))
    say("masked garbage")
    ref, ref_lse = gpu_forward(x, "bf16", 6, dev)
    for b, vl in enumerate(x["valid_len"]):
        x["k"][b, :, vl:] = 1.0e4
        x["v"][b, :, vl:] = -1.0e4
    out, lse = gpu_forward(x, "bf16", 6, dev)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unit_values_give_unit_output(dtype):
    """V = 1: each output entry is the sum of the weights actually used.
    fp32: the MFMA sum and the row sum round differently, at most about
    2 * 448 * 2^-24 = 5e-5 apart; bf16 adds the output rounding (2^-9)."""
    dev = device()
    L, d = 448, 64
    x = inputs(1, 2, L, d, seed=8, dtype=dtype, scale=2.0, valid_range=(300, 448))
    x["v"] = np.ones_like(x["v"])
    say("unit values", dtype)
    out, _ = gpu_forward(x, dtype, 7, dev)
    assert np.abs(out - 1.0).max() <= (2e-5 if dtype == "f32" else 4e-3)


def test_constant_keys_give_mean_of_values():
    dev = device()
    L, d = 320, 64
    x = inputs(2, 2, L, d, seed=9, dtype="bf16", valid_range=(200, 320))
    x["k"] = np.broadcast_to(x["k"][:, :, :1, :], x["k"].shape).copy()
    say("constant keys")
    out, _ = gpu_forward(x, "bf16", 4, dev)
    for b, vl in enumerate(x["valid_len"]):
        mean = x["v"][b, :, :vl].astype(np.float64).mean(axis=1)
        assert np.abs(out[b] - mean[:, None, :]).max() <= 2e-3


def test_large_scores_stress(oracle_lib):
    """Q scaled by 8: scores span about +-60, stressing the running max."""
    dev = device()
    L, d = 512, 64
    x = inputs(1, 2, L, d, seed=10, dtype="bf16")
    x["q"] = rsa_inputs.bf16_round(x["q"] * 8.0)
    say("large scores")
    out, lse = gpu_forward(x, "bf16", 8, dev)
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], None, N=8)
    assert_parity(out, want, "bf16", "large scores")
    assert np.abs(lse - want_lse).max() <= 2e-2


@pytest.mark.parametrize("jump", [25.0, 60.0, 200.0])
@pytest.mark.parametrize("H,L,d,causal", [
    (2, 1024, 64, False),    # small grid: 64-row workgroups, keys split between wave pairs
    (40, 2048, 64, False),   # 128-row workgroups
    (2, 1024, 128, False),
    (2, 1024, 64, True),
])
def test_late_score_jumps(oracle_lib, jump, H, L, d, causal):
    """Three late keys outscore every other key by jump, jump + 1 and
    jump + 2 natural units (positions in different tiles and chunks, met
    after other tiles by most ranks). The weights of those tiles against
    the running base are 2^36 to 2^289 (the largest overflow to infinity):
    the base must move to the new maximum and the earlier tiles' sums and
    products be rescaled, without losing either."""
    dev = device()
    N = 4
    x = inputs(1, H, L, d, seed=int(jump) + L + d, dtype="bf16", scale=0.5)
    rsa_inputs.plant_score_jumps(x, jump, [L - 400, L - 200, L - 30])
    say("late score jumps", jump, H, L, d, "causal" if causal else "")
    q, k, v = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v"))
    out, lse = rsa.forward(q, k, v, None, N=N, return_lse=True, causal=causal)
    torch.cuda.synchronize()
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], None, N=N, causal=causal)
    report(f"late score jumps {jump} H={H} L={L} d={d} causal={causal}",
           assert_parity(from_dev(out), want, "bf16", f"jump {jump}"))
    check_lse(lse.cpu().numpy().astype(np.float64), want_lse, "bf16", f"jump {jump}")


@pytest.mark.parametrize("jump", [25.0, 60.0])
def test_late_score_jumps_rank_share(oracle_lib, jump):
    """The same planted keys in one rank's share, split over ring-step
    groups (each group's partial has its own base before the merge)."""
    dev = device()
    B, H, L, d, N = 1, 2, 4096, 64, 8
    Lc = L // N
    x = inputs(B, H, L, d, seed=int(jump) + 7, dtype="bf16", scale=0.5)
    rsa_inputs.plant_score_jumps(x, jump, [1000, 2100, 3900])
    k, v = to_dev(x["k"], "bf16", dev), to_dev(x["v"], "bf16", dev)
    for rank in (0, 3, 7):
        rows = np.arange(rank * Lc, (rank + 1) * Lc)
        ql = to_dev(x["q"][:, :, rows], "bf16", dev)
        say("late score jumps, rank share", jump, rank)
        out, lse = rsa.forward_rank(ql, k, v, None, N=N, rank=rank, return_lse=True)
        torch.cuda.synchronize()
        want, want_lse = oracle_lib.forward(x["q"][:, :, rows], x["k"], x["v"], None, N=N, qpos=rows)
        assert_parity(from_dev(out), want, "bf16", f"jump {jump} rank {rank}")
        check_lse(lse.cpu().numpy().astype(np.float64), want_lse, "bf16", f"jump {jump} rank {rank}")


def test_forward_is_deterministic():
    dev = device()
    x = inputs(2, 4, 1024, 64, seed=11, dtype="bf16", valid_range=(700, 1024))
    say("determinism")
    a, la = gpu_forward(x, "bf16", 4, dev)
    b, lb = gpu_forward(x, "bf16", 4, dev)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


# --------------------------------------------------------- named workloads ---

@pytest.mark.parametrize("name", ["fp32_small", "bert_base"])
def test_workload_full_parity(oracle_lib, name):
    w = rsa_inputs.WORKLOADS[name]
    dev = device()
    x = rsa_inputs.workload_inputs(w)
    say("workload", name)
    out, lse = gpu_forward(x, w.dtype, w.N, dev)
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=w.N)
    report(f"{name} forward out", assert_parity(out, want, w.dtype, name))
    check_lse(lse, want_lse, w.dtype, name)


def test_long_sequence_full_parity(oracle_lib):
    """B=2, H=12, L=8192, d=64, N=16 (the bench's forward launch): every
    output element of all 24 heads against the oracle, plus each (rank,
    head) slice on its own so that a fault confined to one rank or head
    cannot hide in the whole."""
    w = rsa_inputs.WORKLOADS["long_seq"]
    dev = device()
    x = rsa_inputs.workload_inputs(w)
    say("workload long_seq, all heads")
    out, lse = gpu_forward(x, w.dtype, w.N, dev)
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], None, N=w.N)
    report("long_seq forward out (24 heads)", assert_parity(out, want, "bf16", "long_seq"))
    check_lse(lse, want_lse, "bf16", "long_seq")
    for b in range(w.B):
        for h in range(w.H):
            for n in range(w.N):
                sl = (b, h, slice(n * w.Lc, (n + 1) * w.Lc))
                assert_parity(out[sl], want[sl], "bf16", f"long_seq b={b} h={h} rank {n}")


@pytest.mark.parametrize("rank", [0, 31, 63])
def test_rank_share_full_parity(oracle_lib, rank):
    """One rank's 512 rows against 32768 keys (H=16, d=128, N=64, key
    padding), split over ring-step groups and merged: every row of all 16
    heads. Rank 63 starts its ring on a chunk that can be all padding."""
    w = rsa_inputs.WORKLOADS["rank_share"]
    dev = device()
    x = rsa_inputs.make_inputs(w.B, w.H, w.L, w.d, w.seed, w.dtype, w.scale, w.valid_range, Lq=w.Lc)
    q, k, v = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v"))
    say("rank share", rank, "valid", x["valid_len"])
    out, lse = rsa.forward_rank(q, k, v, mask_dev(x["mask"], dev), N=w.N, rank=rank, return_lse=True)
    torch.cuda.synchronize()
    out, lse = from_dev(out), lse.cpu().numpy()
    base = rank * w.Lc
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=w.N,
                                        qpos=base + np.arange(w.Lc))
    report(f"rank_share rank {rank} out (16 heads)", assert_parity(out, want, "bf16", f"rank {rank}"))
    check_lse(lse, want_lse, "bf16", f"rank {rank}")
    for h in range(w.H):
        assert_parity(out[0, h], want[0, h], "bf16", f"rank {rank} h={h}")


@pytest.mark.parametrize("d", [64, 128])
def test_unmasked_matches_all_ones_mask_bitwise(d):
    """Without a key mask (chunk-aligned tiles, not causal) the forward runs an
    instance that builds no tile table; with an all-ones mask every tile is
    whole, so the general instance must give the same bits: full forward and
    one rank's share (split over ring-step groups)."""
    dev = device()
    B, H, L, N = 2, 3, 1024, 8
    x = inputs(B, H, L, d, seed=90 + d, dtype="bf16")
    q, k, v = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v"))
    ones = torch.ones(B, L, dtype=torch.uint8, device=dev)
    say("unmasked vs all-ones mask", d)
    a, la = rsa.forward(q, k, v, None, N=N, return_lse=True)
    b, lb = rsa.forward(q, k, v, ones, N=N, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    Lc = L // N
    for rank in (0, N - 1):
        ql = q[:, :, rank * Lc:(rank + 1) * Lc].contiguous()
        a, la = rsa.forward_rank(ql, k, v, None, N=N, rank=rank, return_lse=True)
        b, lb = rsa.forward_rank(ql, k, v, ones, N=N, rank=rank, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(la, lb), rank


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L,N,d", [(256, 4, 64), (1024, 32, 128), (600, 6, 64), (96, 96, 128),
                                   # 12 chunks of 128 in 8 ring-step groups: groups take every 8th
                                   # step, so four of them hold two steps and four hold one
                                   (1536, 12, 64), (1536, 12, 128)])
def test_rank_share_matches_oracle_small(oracle_lib, dtype, L, N, d):
    dev = device()
    x = inputs(2, 2, L, d, seed=L + N, dtype=dtype, valid_range=(L // 3, L))
    Lc = L // N
    k, v = to_dev(x["k"], dtype, dev), to_dev(x["v"], dtype, dev)
    m = mask_dev(x["mask"], dev)
    for rank in sorted({0, N // 2, N - 1}):
        rows = np.arange(rank * Lc, (rank + 1) * Lc)
        ql = to_dev(x["q"][:, :, rows], dtype, dev)
        say("rank share small", dtype, L, N, d, rank)
        out, lse = rsa.forward_rank(ql, k, v, m, N=N, rank=rank, return_lse=True)
        torch.cuda.synchronize()
        want, want_lse = oracle_lib.forward(x["q"][:, :, rows], x["k"], x["v"], x["mask"], N=N, qpos=rows)
        assert_parity(from_dev(out), want, dtype, f"rank {rank}")
        check_lse(lse.cpu().numpy().astype(np.float64), want_lse, dtype, f"rank {rank}")


@pytest.mark.parametrize("rank", [0, 1])
def test_rank_share_one_group(oracle_lib, rank):
    """A rank share with 512 query tiles (B=1, H=16, L=8192, N=2: 4096 rows
    per rank) runs in one ring-step group, in the instance with 64-row
    workgroups whose wave pairs split each tile's keys; rank 1 starts half
    way down the sequence. Key padding; 96 sampled rows of every head
    against the oracle."""
    B, H, L, d, N = 1, 16, 8192, 64, 2
    Lc = L // N
    dev = device()
    x = inputs(B, H, L, d, seed=8192 + rank, dtype="bf16", valid_range=(5000, 7000))
    k, v = to_dev(x["k"], "bf16", dev), to_dev(x["v"], "bf16", dev)
    rows = np.arange(rank * Lc, (rank + 1) * Lc)
    ql = to_dev(x["q"][:, :, rows], "bf16", dev)
    say("rank share one group", rank, "valid", x["valid_len"])
    out, lse = rsa.forward_rank(ql, k, v, mask_dev(x["mask"], dev), N=N, rank=rank, return_lse=True)
    torch.cuda.synchronize()
    out, lse = from_dev(out), lse.cpu().numpy().astype(np.float64)
    pick = sample_rows(Lc, 96, seed=rank)
    want, want_lse = oracle_lib.forward(x["q"][:, :, rows[pick]], x["k"], x["v"], x["mask"], N=N, qpos=rows[pick])
    report(f"rank share one group, rank {rank} (96 rows x 16 heads)",
           assert_parity(out[:, :, pick], want, "bf16", f"one-group rank {rank}"))
    check_lse(lse[:, :, pick], want_lse, "bf16", f"one-group rank {rank}")


@pytest.mark.parametrize("d", [64, 128])
def test_forward_longest_key_range(oracle_lib, d):
    """L = 1048576, the longest key range one launch covers (its tile table
    holds 16384 tiles of 64 keys), with key padding; sampled rows of every
    part of the sequence against the oracle."""
    dev = device()
    L, N = 64 * 16384, 64
    x = inputs(1, 1, L, d, seed=40 + d, dtype="bf16", valid_range=(L - 5000, L - 1000))
    say("forward longest key range", d, "valid", x["valid_len"])
    out, lse = gpu_forward(x, "bf16", N, dev)
    rows = sample_rows(L, 14, seed=41)
    want, want_lse = oracle_lib.forward(x["q"][:, :, rows], x["k"], x["v"], x["mask"], N=N, qpos=rows)
    assert_parity(out[0, 0, rows], want[0, 0], "bf16", f"L={L} d={d}")
    check_lse(lse[0, 0, rows], want_lse[0, 0], "bf16", f"L={L} d={d}")
