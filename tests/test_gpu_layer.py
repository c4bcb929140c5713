"""GPU parity of the layer around RSA (bf16 matrix products with their fused
head split / head merge / bias / GeLU / residual, layer normalisation, and
the whole encoder layer) against the fp64 layer oracle, through the C ABI.

Gates. A product accumulates in fp32, whose rounding error is at most about
K * 2^-24 * S with S = sum_k |a_k w_k| + |bias| + |residual| (the standard
bound for a K-term sum), and its result is rounded once to bf16 (relative
error <= 2^-9); each element must satisfy
|got - want| <= 2^-8 |want| + K * 2^-24 * S.
The layer normalisation: 2^-8 |want| + 2^-16 (fp32 statistics).
The whole layer is checked three ways: it equals, bit for bit, the chain
of the individual entry points; every step of that chain meets its own
gate above given the GPU's input to that step; and the layer output agrees
with the oracle that rounds the same kept activations to bf16. In the last
comparison the two sides differ wherever a kept value falls on different
sides of a rounding boundary (one bf16 unit at that value, up to 2^-6 for
the second residual sum, which reaches magnitude 4) and through the
attention's bf16 weights (about 2e-3 relative); those one-unit differences
add along the chain of nine kept activations, so each element must satisfy
|got - want| <= 2^-4 and the relative Frobenius error must stay below 5e-3.
"""

import numpy as np
import pytest
import torch

import rsa_inputs
import sequence_transformer_attention_rsa_amd as rsa
from gpu_util import device, from_dev, mask_dev, sample_rows, say

pytestmark = pytest.mark.gpu


def bf(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(dev)


def f32(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def check_product(got, want, S, K, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    err = np.abs(got - want)
    tol = 2.0 ** -8 * np.abs(want) + K * 2.0 ** -24 * S
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of bound, worst excess {float((err - tol).max()):.3e}"


def check_layer(got, want, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    err = float(np.abs(got - want).max())
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    print(f"[{what}] max-abs {err:.3e} rel-Frobenius {rel:.3e}")
    assert err <= 2.0 ** -4, f"{what}: max-abs {err:.3e}"
    assert rel <= 5e-3, f"{what}: rel-Frobenius {rel:.3e}"
    return err, float(rel)


def check_norm(got, want, what):
    err = np.abs(got - want)
    assert (err <= 2.0 ** -8 * np.abs(want) + 2.0 ** -16).all(), f"{what}: {float(err.max()):.3e}"


@pytest.mark.parametrize("M,N,K,act,bias,res", [
    (256, 128, 64, "none", False, False),     # one contraction step
    (200, 256, 192, "gelu", True, False),     # ragged M, three steps
    (1, 384, 768, "none", True, True),        # a single row
    (129, 128, 128, "gelu", True, True),      # ragged by one row, two steps
    (1000, 768, 3072, "none", True, True),    # the second MLP product's width (256 x 192 tiles)
    (300, 1152, 256, "gelu", True, True),     # 192-column tiles, ragged M, GeLU
])
def test_linear_parity(oracle_lib, M, N, K, act, bias, res):
    from oracle import layer as OL
    dev = device()
    rng = np.random.default_rng(M * 7 + N + K)
    a = rsa_inputs.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    w = rsa_inputs.bf16_round((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    b = (rng.standard_normal(N) * 0.1).astype(np.float32) if bias else None
    r = rsa_inputs.bf16_round(rng.standard_normal((M, N)).astype(np.float32)) if res else None
    say("linear", M, N, K, act, bias, res)
    out = rsa.linear(bf(a, dev), bf(w, dev), None if b is None else f32(b, dev),
                     None if r is None else bf(r, dev), activation=act)
    torch.cuda.synchronize()
    z = OL.linear(a, w, np.zeros(N) if b is None else b)
    want = OL.gelu(z) if act == "gelu" else z
    if r is not None:
        want = want + r
    S = np.abs(a.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    S += 0 if b is None else np.abs(b)
    S += 0 if r is None else np.abs(r)
    check_product(from_dev(out), want, S, K, f"linear {M}x{N}x{K}")


@pytest.mark.parametrize("B,L,E,H", [
    (2, 96, 256, 4),      # 256-column tiles (E % 256 == 0, E % 192 != 0)
    (1, 130, 512, 4),     # d = 128, ragged rows
    (3, 64, 768, 12),     # BERT-base widths (192-column tiles)
    (2, 80, 384, 6),      # 192-column tiles (E % 256 != 0)
    (2, 70, 640, 10),     # 128-column tiles (E divisible by neither 256 nor 192)
])
def test_qkv_and_output_projection(oracle_lib, B, L, E, H):
    from oracle import layer as OL
    dev = device()
    x = rsa_inputs.make_layer_inputs(B, L, E, H, 4 * E, seed=B + L + E)
    say("qkv/output projection", B, L, E, H)
    q, k, v = rsa.qkv_projection(bf(x["x"], dev), bf(x["w_qkv"], dev), f32(x["b_qkv"], dev), H)
    torch.cuda.synchronize()
    wq, wk, wv = OL.qkv_projection(x["x"], x["w_qkv"], x["b_qkv"], H, store=None)
    S = np.abs(x["x"].astype(np.float64)) @ np.abs(x["w_qkv"].astype(np.float64)).T + np.abs(x["b_qkv"])
    Sq, Sk, Sv = (OL.split_heads(S[..., i * E:(i + 1) * E], H) for i in range(3))
    for name, got, want, s in (("q", q, wq, Sq), ("k", k, wk, Sk), ("v", v, wv, Sv)):
        check_product(from_dev(got), want, s, E, f"qkv {name}")
    # output projection of a random head-layout operand, with the residual
    rng = np.random.default_rng(L)
    o = rsa_inputs.bf16_round(rng.standard_normal((B, H, L, E // H)).astype(np.float32))
    out = rsa.output_projection(bf(o, dev), bf(x["w_o"], dev), f32(x["b_o"], dev), bf(x["x"], dev))
    torch.cuda.synchronize()
    om = OL.merge_heads(o)
    want = OL.linear(om, x["w_o"], x["b_o"]) + x["x"]
    S = np.abs(om) @ np.abs(x["w_o"].astype(np.float64)).T + np.abs(x["b_o"]) + np.abs(x["x"])
    check_product(from_dev(out), want, S, E, "output projection")


@pytest.mark.parametrize("rows,E", [(1, 768), (37, 768), (300, 1024), (5, 4096), (8, 64)])
def test_layernorm_parity(oracle_lib, rows, E):
    from oracle import layer as OL
    dev = device()
    rng = np.random.default_rng(rows + E)
    x = rsa_inputs.bf16_round((rng.standard_normal((rows, E)) * 3 + 1).astype(np.float32))
    g = (1 + rng.standard_normal(E) * 0.1).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    say("layernorm", rows, E)
    y = rsa.layernorm(bf(x, dev), f32(g, dev), f32(b, dev))
    torch.cuda.synchronize()
    check_norm(from_dev(y), OL.layernorm(x, g, b), f"layernorm {rows}x{E}")


def test_gelu_is_the_exact_erf_form():
    """Pre-activations z exact (one nonzero product per output): the GPU
    output must be bf16(GeLU(z)) of the erf form for (almost) every z on a
    fine grid; the tanh approximation rounds differently on many of them."""
    from oracle import layer as OL
    dev = device()
    z = rsa_inputs.bf16_round(np.linspace(-5.0, 5.0, 4001).astype(np.float32))
    a = np.zeros((z.size, 64), np.float32)
    a[:, 0] = z
    w = np.zeros((128, 64), np.float32)
    w[:, 0] = 1.0
    say("gelu grid")
    out = from_dev(rsa.linear(bf(a, dev), bf(w, dev), activation="gelu"))
    torch.cuda.synchronize()
    want = OL.round_bf16(OL.gelu(z.astype(np.float64)))
    assert np.array_equal(out, np.repeat(out[:, :1], 128, axis=1))
    agree = np.mean(out[:, 0] == want)
    tanh = OL.round_bf16(0.5 * z * (1 + np.tanh(np.sqrt(2 / np.pi) * (z + 0.044715 * z.astype(np.float64) ** 3))))
    assert np.mean(tanh == want) < 0.95      # the grid tells the two forms apart
    assert agree >= 0.995, agree


@pytest.mark.parametrize("B,L,E,H,F,N,valid", [
    (2, 192, 256, 4, 1024, 3, (100, 192)),   # chunks of 64, key padding
    (1, 130, 512, 4, 512, 5, None),          # L not a multiple of 64 (chunks of 26 keys)
    (2, 256, 512, 4, 2048, 4, None),         # d = 128
    (1, 1024, 1024, 8, 4096, 4, (700, 1024)),   # d = 128, E = 1024: 256-column product tiles
])
def test_layer_small_parity(oracle_lib, B, L, E, H, F, N, valid):
    from oracle import layer as OL
    dev = device()
    x = rsa_inputs.make_layer_inputs(B, L, E, H, F, seed=L + E + N, valid_range=valid)
    say("layer", B, L, E, H, F, N, valid)
    w = {n: (bf(x[n], dev) if n.startswith("w_") else f32(x[n], dev)) for n in rsa.LAYER_WEIGHTS}
    xd, m = bf(x["x"], dev), mask_dev(x["mask"], dev)
    y = rsa.layer_forward(xd, w, H=H, N=N, key_mask=m)
    # the same steps through the individual entry points
    q, k, v = rsa.qkv_projection(xd, w["w_qkv"], w["b_qkv"], H)
    o = rsa.forward(q, k, v, m, N=N)
    a1 = rsa.output_projection(o, w["w_o"], w["b_o"], xd)
    h1 = rsa.layernorm(a1, w["ln1_gamma"], w["ln1_beta"])
    f1 = rsa.linear(h1.view(B * L, E), w["w_ff1"], w["b_ff1"], activation="gelu")
    a2 = rsa.linear(f1, w["w_ff2"], w["b_ff2"], residual=h1.view(B * L, E))
    y2 = rsa.layernorm(a2, w["ln2_gamma"], w["ln2_beta"]).view(B, L, E)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    # each step against the oracle, given the GPU's input to that step
    o_, a1_, h1_, f1_, a2_ = (from_dev(t) for t in (o, a1, h1, f1, a2))
    om = OL.merge_heads(o_)
    S = np.abs(om) @ np.abs(x["w_o"].astype(np.float64)).T + np.abs(x["b_o"]) + np.abs(x["x"])
    check_product(a1_, OL.linear(om, x["w_o"], x["b_o"]) + x["x"], S, E, "layer output projection")
    check_norm(h1_, OL.layernorm(a1_, x["ln1_gamma"], x["ln1_beta"]), "layer norm 1")
    h1m = h1_.reshape(B * L, E)
    S = np.abs(h1m) @ np.abs(x["w_ff1"].astype(np.float64)).T + np.abs(x["b_ff1"])
    check_product(f1_, OL.gelu(OL.linear(h1m, x["w_ff1"], x["b_ff1"])), S, E, "layer ff1")
    S = np.abs(f1_) @ np.abs(x["w_ff2"].astype(np.float64)).T + np.abs(x["b_ff2"]) + np.abs(h1m)
    check_product(a2_, OL.linear(f1_, x["w_ff2"], x["b_ff2"]) + h1m, S, F, "layer ff2")
    check_norm(from_dev(y).reshape(B * L, E), OL.layernorm(a2_, x["ln2_gamma"], x["ln2_beta"]), "layer norm 2")
    want = OL.layer_forward(x, H, N, store="bf16")["y"]
    check_layer(from_dev(y), want, f"layer L={L} E={E}")


def _run_layer(shape, dev):
    x = rsa_inputs.layer_inputs(shape)
    w = {n: (bf(x[n], dev) if n.startswith("w_") else f32(x[n], dev)) for n in rsa.LAYER_WEIGHTS}
    y = rsa.layer_forward(bf(x["x"], dev), w, H=shape.H, N=shape.N, key_mask=mask_dev(x["mask"], dev))
    torch.cuda.synchronize()
    return x, from_dev(y)


def test_layer_bert_base_full(oracle_lib):
    from oracle import layer as OL
    shape = rsa_inputs.LAYERS["layer_bert_base"]
    dev = device()
    say("layer workload", shape.name)
    x, y = _run_layer(shape, dev)
    want = OL.layer_forward(x, shape.H, shape.N, store="bf16")["y"]
    check_layer(y, want, shape.name)


def test_layer_long_seq_sampled_rows(oracle_lib):
    """B=2, L=8192, E=768 (12 heads of 64), F=3072, N=16: every token's K and V
    enter the oracle's attention; ~130 sampled rows per batch row are checked."""
    from oracle import layer as OL
    shape = rsa_inputs.LAYERS["layer_long_seq"]
    dev = device()
    say("layer workload", shape.name)
    x, y = _run_layer(shape, dev)
    rows = sample_rows(shape.L, 128, seed=21)
    want = OL.layer_forward(x, shape.H, shape.N, store="bf16", rows=rows)["y"]
    check_layer(y[:, rows], want, shape.name)


def test_layer_workspace_reuse_is_deterministic():
    shape = rsa_inputs.LAYERS["layer_bert_base"]
    dev = device()
    x = rsa_inputs.layer_inputs(shape)
    w = {n: (bf(x[n], dev) if n.startswith("w_") else f32(x[n], dev)) for n in rsa.LAYER_WEIGHTS}
    need = rsa.layer_forward_workspace_bytes(shape.B, shape.L, shape.E, shape.H, shape.F, shape.N)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev)
    xin = bf(x["x"], dev)
    m = mask_dev(x["mask"], dev)
    say("layer workspace reuse")
    a = rsa.layer_forward(xin, w, H=shape.H, N=shape.N, key_mask=m, workspace=ws)
    b = rsa.layer_forward(xin, w, H=shape.H, N=shape.N, key_mask=m, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(rsa.RSAError):
        rsa.layer_forward(xin, w, H=shape.H, N=shape.N, key_mask=m, workspace=ws[:-2])
