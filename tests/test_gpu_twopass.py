"""GPU parity of the two-stage forward (score rows materialised, then the
row softmax, then the weighted sum of V) against the fp64 oracle, through
the C ABI, and its agreement with the fused forward."""

import numpy as np
import pytest
import torch

import rsa_inputs
import sequence_transformer_attention_rsa_amd as rsa
from gates import LSE_TOL as _LSE_TOL, MAX_ABS, assert_parity
from gpu_util import device, from_dev, inputs, mask_dev, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu

LSE_TOL = _LSE_TOL["bf16"]


def run(x, N, dev, fused=False):
    q, k, v = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v"))
    m = mask_dev(x["mask"], dev)
    fn = rsa.forward if fused else rsa.forward_twopass
    out, lse = fn(q, k, v, m, N=N, return_lse=True)
    torch.cuda.synchronize()
    return from_dev(out), lse.cpu().numpy().astype(np.float64)


def check_lse(got, want, what):
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: lse finiteness differs"
    if fin.any():
        err = np.abs(got[fin] - want[fin]).max()
        assert err <= LSE_TOL, f"{what}: lse max-abs {err:.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,N,valid", [
    (256, 4, None),          # two 128-row score tiles per side
    (200, 5, (150, 200)),    # ragged score tile, ragged 64-key value tile
    (135, 5, (60, 135)),     # odd L: rows start on 4-byte boundaries only
    (130, 13, None),         # chunks of 10 keys
    (1, 1, None),            # one query, one key
    (520, 8, (1, 520)),      # PAIRS = 2 in the softmax pass
])
def test_twopass_small_parity(oracle_lib, d, L, N, valid):
    dev = device()
    x = inputs(2, 3, L, d, seed=L * 3 + d + N, dtype="bf16", valid_range=valid)
    say("twopass", d, L, N, valid)
    out, lse = run(x, N, dev)
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=N)
    assert_parity(out, want, "bf16", f"twopass d={d} L={L} N={N}")
    check_lse(lse, want_lse, f"twopass lse d={d} L={L} N={N}")


def test_twopass_matches_fused_and_ignores_n():
    """Both forms compute the same attention: within the bf16 gate of each
    other; the materialised form sums in its own order, so N does not
    change a single bit of it."""
    dev = device()
    L, d = 768, 64
    x = inputs(2, 2, L, d, seed=31, dtype="bf16", valid_range=(500, 768))
    say("twopass vs fused")
    ref, ref_lse = run(x, 1, dev)
    for N in (2, 3, 8, 768):
        out, lse = run(x, N, dev)
        assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse), f"N={N}"
    fused, fused_lse = run(x, 8, dev, fused=True)
    assert np.abs(fused - ref).max() <= MAX_ABS["bf16"]
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(fused_lse), fin)
    assert np.abs(fused_lse[fin] - ref_lse[fin]).max() <= LSE_TOL


def test_twopass_fully_masked_and_garbage():
    dev = device()
    L, d = 384, 128
    x = inputs(2, 2, L, d, seed=32, dtype="bf16", valid_range=(100, 300))
    x["mask"][1] = 0
    say("twopass fully masked + garbage")
    ref, ref_lse = run(x, 4, dev)
    assert np.all(ref[1] == 0.0) and np.all(np.isneginf(ref_lse[1]))
    vl = x["valid_len"][0]
    x["k"][0, :, vl:] = 1.0e4
    x["v"][0, :, vl:] = -1.0e4
    out, lse = run(x, 4, dev)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


def test_twopass_workspace_reuse_and_determinism():
    dev = device()
    B, H, L, d, N = 1, 4, 1024, 64, 8
    x = inputs(B, H, L, d, seed=33, dtype="bf16", valid_range=(700, 1024))
    q, k, v = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v"))
    m = mask_dev(x["mask"], dev)
    ws = torch.full((rsa.forward_twopass_workspace_bytes(B, H, L, d, N),), 0x7F, dtype=torch.uint8, device=dev)
    say("twopass workspace reuse")
    a = rsa.forward_twopass(q, k, v, m, N=N, workspace=ws)
    b = rsa.forward_twopass(q, k, v, m, N=N, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(rsa.RSAError):
        rsa.forward_twopass(q, k, v, m, N=N, workspace=ws[:-16])


def test_twopass_bert_base_full(oracle_lib):
    w = rsa_inputs.WORKLOADS["bert_base"]
    dev = device()
    x = rsa_inputs.workload_inputs(w)
    say("twopass workload bert_base")
    out, lse = run(x, w.N, dev)
    want, want_lse = oracle_lib.forward(x["q"], x["k"], x["v"], x["mask"], N=w.N)
    assert_parity(out, want, "bf16", "twopass bert_base")
    check_lse(lse, want_lse, "twopass bert_base")


def test_twopass_long_sequence_sampled_rows(oracle_lib):
    """B=2, H=12, L=8192, d=64, N=16 (6 GiB of score rows), checked on two
    heads x ~200 sampled rows."""
    w = rsa_inputs.WORKLOADS["long_seq"]
    dev = device()
    x = rsa_inputs.workload_inputs(w)
    say("twopass workload long_seq")
    out, lse = run(x, w.N, dev)
    for b, h in ((0, 3), (1, 8)):
        rows = sample_rows(w.L, 192, seed=b * 10 + h)
        want, want_lse = oracle_lib.forward(x["q"][b:b + 1, h:h + 1, rows], x["k"][b:b + 1, h:h + 1],
                                            x["v"][b:b + 1, h:h + 1], None, N=w.N, qpos=rows)
        assert_parity(out[b, h, rows], want[0, 0], "bf16", f"twopass long_seq b={b} h={h}")
        check_lse(lse[b, h, rows], want_lse[0, 0], "twopass long_seq")


@pytest.mark.parametrize("L,N,valid", [
    (16384, 16, (12000, 16384)),   # the longest row the softmax pass holds in registers
    (16896, 16, (16500, 16896)),   # the shortest row of the two-pass-per-row kernel
    (17000, 17, (9000, 17000)),    # a row that ends inside a 512-element chunk
    (65536, 64, None),             # 16 GiB of score rows
])
def test_twopass_long_rows(oracle_lib, L, N, valid):
    dev = device()
    x = inputs(1, 1, L, 64, seed=34 + L % 97, dtype="bf16", valid_range=valid)
    say("twopass long rows", L, N, valid)
    out, lse = run(x, N, dev)
    rows = sample_rows(L, 64, seed=34)
    want, want_lse = oracle_lib.forward(x["q"][:, :, rows], x["k"], x["v"], x["mask"], N=N, qpos=rows)
    assert_parity(out[0, 0, rows], want[0, 0], "bf16", f"twopass L={L}")
    check_lse(lse[0, 0, rows], want_lse[0, 0], f"twopass L={L}")
