"""Pins of the fp64 layer oracle (oracle/layer.py) against facts fixed outside it.

The layer around RSA (QKV projection, attention, output projection, residual
sums, layer normalisations, two fully connected layers with GeLU) is pinned
to: torch's own fp64 Transformer encoder layer (the post-normalisation,
GeLU encoder layer is a library routine there), torch's fp64 linear,
layer-norm and exact GeLU, a pure-Python triple loop, printed values of the
standard normal CDF, a bit-level bf16 rounding, and invariants (independence
of the chunk count N, token locality, masked keys).
"""

import math

import numpy as np
import pytest
import torch

import rsa_inputs
from oracle import layer as L


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def small_inputs(B=2, Ls=12, E=16, H=2, F=24, seed=0, valid=None):
    x = rsa_inputs.make_layer_inputs(B, Ls, E, H, F, seed, valid)
    # larger weights than the workload's 0.02 so that attention is far from uniform
    rng = np.random.default_rng(seed + 100)
    for name in ("w_qkv", "w_o", "w_ff1", "w_ff2"):
        x[name] = rsa_inputs.bf16_round(rng.standard_normal(x[name].shape).astype(np.float32) * 0.4)
    return x


# ----------------------------------------------------------- bf16 rounding ---

def test_round_bf16_matches_bit_level_rounding():
    v = np.concatenate([rand(20000, 1), rand(2000, 2, 1e-3), rand(2000, 3, 1e3)]).astype(np.float32)
    # exact ties: 1 + 2^-8 (halfway between 1 and 1 + 2^-7) and neighbours
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 + 2 ** -7, 1.5 + 2 ** -8], np.float32)
    v = np.concatenate([v, ties])
    got = L.round_bf16(v.astype(np.float64))
    want = rsa_inputs.bf16_round(v).astype(np.float64)
    assert np.array_equal(got, want)
    assert L.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0            # tie to even (down)
    assert L.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6  # tie to even (up)
    assert L.round_bf16(np.array([0.0]))[0] == 0.0


# ------------------------------------------------------------------ pieces ---

def test_linear_matches_triple_loop_and_torch():
    a, w, b = rand((3, 5), 4), rand((7, 5), 5), rand(7, 6)
    want = [[sum(a[i, k] * w[j, k] for k in range(5)) + b[j] for j in range(7)] for i in range(3)]
    got = L.linear(a, w, b)
    assert np.allclose(got, np.array(want), rtol=0, atol=1e-13)
    t = torch.nn.functional.linear(torch.from_numpy(a), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    assert np.allclose(got, t, rtol=0, atol=1e-13)


def test_gelu_printed_normal_cdf_values():
    # Phi(1) = 0.841344746068543, Phi(2) = 0.977249868051821, Phi(0.5) = 0.691462461274013
    pts = np.array([0.0, 1.0, -1.0, 2.0, 0.5, -0.5])
    want = np.array([0.0, 0.841344746068543, -(1 - 0.841344746068543), 2 * 0.977249868051821,
                     0.5 * 0.691462461274013, -0.5 * (1 - 0.691462461274013)])
    assert np.allclose(L.gelu(pts), want, rtol=0, atol=1e-14)
    assert abs(L.gelu(np.array([10.0]))[0] - 10.0) < 1e-20
    assert abs(L.gelu(np.array([-10.0]))[0]) < 1e-21


def test_gelu_is_the_exact_form_not_tanh():
    z = np.linspace(-6, 6, 2001)
    t = torch.nn.functional.gelu(torch.from_numpy(z), approximate="none").numpy()
    assert np.allclose(L.gelu(z), t, rtol=0, atol=1e-15)
    tanh = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.abs(L.gelu(z) - tanh).max() > 1e-4


def test_layernorm_torch_and_moments():
    z, g, b = rand((5, 32), 7, 3.0) + 2.0, 1 + rand(32, 8, 0.1), rand(32, 9, 0.1)
    t = torch.nn.functional.layer_norm(torch.from_numpy(z), (32,), torch.from_numpy(g),
                                       torch.from_numpy(b), eps=1e-12).numpy()
    assert np.allclose(L.layernorm(z, g, b), t, rtol=0, atol=1e-12)
    y = L.layernorm(z, np.ones(32), np.zeros(32))
    assert np.allclose(y.mean(axis=-1), 0.0, atol=1e-13)
    assert np.allclose((y ** 2).mean(axis=-1), 1.0, atol=1e-12)     # population variance
    # a constant row normalises to beta
    assert np.allclose(L.layernorm(np.full((1, 32), 3.5), g, b), b[None, :], atol=1e-12)


def test_head_split_order():
    t = np.arange(2 * 3 * 8, dtype=np.float64).reshape(2, 3, 8)    # B=2, L=3, E=8
    s = L.split_heads(t, 2)                                          # d = 4
    assert s.shape == (2, 2, 3, 4)
    assert np.array_equal(s[1, 0, 2], t[1, 2, 0:4]) and np.array_equal(s[1, 1, 2], t[1, 2, 4:8])
    assert np.array_equal(L.merge_heads(s), t)


# ------------------------------------------------------------- whole layer ---

def torch_layer(inp, H, mask):
    x = torch.from_numpy(np.asarray(inp["x"], np.float64))
    E = x.shape[-1]
    F = inp["w_ff1"].shape[0]
    m = torch.nn.TransformerEncoderLayer(E, H, dim_feedforward=F, dropout=0.0, activation="gelu",
                                         layer_norm_eps=1e-12, batch_first=True, norm_first=False,
                                         dtype=torch.float64)
    sd = {"self_attn.in_proj_weight": inp["w_qkv"], "self_attn.in_proj_bias": inp["b_qkv"],
          "self_attn.out_proj.weight": inp["w_o"], "self_attn.out_proj.bias": inp["b_o"],
          "linear1.weight": inp["w_ff1"], "linear1.bias": inp["b_ff1"],
          "linear2.weight": inp["w_ff2"], "linear2.bias": inp["b_ff2"],
          "norm1.weight": inp["ln1_gamma"], "norm1.bias": inp["ln1_beta"],
          "norm2.weight": inp["ln2_gamma"], "norm2.bias": inp["ln2_beta"]}
    m.load_state_dict({k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in sd.items()})
    m.train()   # no fused inference path; dropout is 0
    kpm = None if mask is None else torch.from_numpy(np.asarray(mask) == 0)
    with torch.no_grad():
        return m(x, src_key_padding_mask=kpm).numpy()


@pytest.mark.parametrize("valid", [None, (5, 12)])
def test_layer_matches_torch_encoder_layer(valid):
    inp = small_inputs(valid=valid)
    got = L.layer_forward(inp, H=2, N=3, store=None)["y"]
    want = torch_layer(inp, 2, inp["mask"])
    assert np.abs(got - want).max() < 1e-10


def test_layer_independent_of_n_and_token_local():
    inp = small_inputs(B=1, Ls=24, seed=3, valid=(17, 17))
    ref = L.layer_forward(inp, H=2, N=1, store=None)
    for N in (2, 3, 4, 6, 8, 12, 24):
        assert np.abs(L.layer_forward(inp, H=2, N=N, store=None)["y"] - ref["y"]).max() < 1e-12
    rows = np.array([0, 5, 16, 17, 23])
    part = L.layer_forward(inp, H=2, N=4, store=None, rows=rows)
    assert np.abs(part["y"] - ref["y"][:, rows]).max() < 1e-12


def test_layer_padded_tokens_only_change_themselves():
    inp = small_inputs(B=1, Ls=16, seed=4, valid=(10, 10))
    ref = L.layer_forward(inp, H=2, N=2, store=None)["y"]
    inp2 = dict(inp)
    x2 = np.array(inp["x"], copy=True)
    x2[:, 10:] = rand(x2[:, 10:].shape, 5, 5.0)
    inp2["x"] = x2
    y2 = L.layer_forward(inp2, H=2, N=2, store=None)["y"]
    assert np.abs(y2[:, :10] - ref[:, :10]).max() < 1e-12
    assert np.abs(y2[:, 10:] - ref[:, 10:]).max() > 1e-3


def test_zero_qkv_weights_give_uniform_attention():
    # Q = K = V = bias for every token: the attention output is v's bias part
    inp = small_inputs(B=1, Ls=8, seed=6)
    inp["w_qkv"] = np.zeros_like(inp["w_qkv"])
    r = L.layer_forward(inp, H=2, N=2, store=None)
    E = inp["x"].shape[-1]
    vb = inp["b_qkv"][2 * E:].astype(np.float64)
    assert np.allclose(L.merge_heads(r["o"]), np.broadcast_to(vb, (1, 8, E)), atol=1e-14)


def test_bf16_store_mode_rounds_every_kept_activation():
    inp = small_inputs(seed=8, valid=(6, 12))
    r = L.layer_forward(inp, H=2, N=2, store="bf16")
    for name in ("q", "k", "v", "o", "a1", "h1", "f1", "a2", "y"):
        assert np.array_equal(r[name], L.round_bf16(r[name])), name
    exact = L.layer_forward(inp, H=2, N=2, store=None)["y"]
    # nine rounding points of relative size 2^-9 each, through O(1) layer gains
    assert np.abs(r["y"] - exact).max() < 0.1
    assert np.linalg.norm(r["y"] - exact) / np.linalg.norm(exact) < 2e-2


# ------------------------------------------------- bf16 store mode, exactly ---

POINTS = ("q", "k", "v", "o", "a1", "h1", "f1", "a2", "y")


def torch_layer_bf16(inp, H, drop=(), move=None):
    """The layer written independently with torch fp64 operations (linear,
    scaled_dot_product_attention with a boolean key mask, layer_norm, exact
    GeLU), rounding to bf16 with torch's own conversion at the nine points
    where a bf16 implementation stores an activation: Q, K, V, O, A1, h1, F1,
    A2, y. `drop` removes roundings; `move` places one elsewhere:
      "gelu_in"   F1 rounded before the GeLU instead of after it,
      "a1_prod"   A1's product rounded before the residual sum instead of after,
      "a2_prod"   the same for A2,
      "a1_twice"  A1's product rounded before the residual sum and A1 after it,
      "a2_twice"  the same for A2."""
    f = torch.nn.functional
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    bf = lambda t: t.to(torch.bfloat16).to(torch.float64)
    r = lambda name, t: t if name in drop else bf(t)
    x = T(inp["x"])
    B, Ls, E = x.shape
    d = E // H
    t = f.linear(x, T(inp["w_qkv"]), T(inp["b_qkv"]))
    heads = lambda u: u.reshape(B, Ls, H, d).transpose(1, 2)
    q, k, v = (r(n, heads(t[..., i * E:(i + 1) * E])) for i, n in enumerate(("q", "k", "v")))
    mask = None if inp["mask"] is None else T(inp["mask"]).bool()[:, None, None, :]
    o = r("o", f.scaled_dot_product_attention(q, k, v, attn_mask=mask))
    z1 = f.linear(o.transpose(1, 2).reshape(B, Ls, E), T(inp["w_o"]), T(inp["b_o"]))
    if move in ("a1_prod", "a1_twice"):
        z1 = bf(z1)
    a1 = z1 + x if move == "a1_prod" else r("a1", z1 + x)
    h1 = r("h1", f.layer_norm(a1, (E,), T(inp["ln1_gamma"]), T(inp["ln1_beta"]), eps=1e-12))
    z = f.linear(h1, T(inp["w_ff1"]), T(inp["b_ff1"]))
    f1 = f.gelu(bf(z)) if move == "gelu_in" else r("f1", f.gelu(z))
    z2 = f.linear(f1, T(inp["w_ff2"]), T(inp["b_ff2"]))
    if move in ("a2_prod", "a2_twice"):
        z2 = bf(z2)
    a2 = z2 + h1 if move == "a2_prod" else r("a2", z2 + h1)
    y = r("y", f.layer_norm(a2, (E,), T(inp["ln2_gamma"]), T(inp["ln2_beta"]), eps=1e-12))
    return {"q": q, "k": k, "v": v, "o": o, "a1": a1, "h1": h1, "f1": f1, "a2": a2, "y": y}


def test_bf16_store_mode_equals_torch_at_the_nine_points():
    """The oracle's bf16 store mode equals, value for value, an independent
    torch evaluation that rounds with torch's bf16 conversion at exactly the
    nine kept activations; every plausible misplacement of a rounding (one
    left out, one moved before the GeLU or before a residual sum, one applied
    twice around a residual sum) changes the result, so the equality pins
    the placement."""
    inp = small_inputs(seed=8, valid=(6, 12))
    got = L.layer_forward(inp, H=2, N=3, store="bf16")
    want = torch_layer_bf16(inp, 2)
    for name in POINTS:
        w = want[name].numpy()
        if name in ("q", "k", "v", "o"):
            w = np.ascontiguousarray(w)
        assert np.array_equal(got[name], w), name
    variants = [dict(drop=(p,)) for p in POINTS] + [dict(move=m) for m in
                                                    ("gelu_in", "a1_prod", "a2_prod", "a1_twice", "a2_twice")]
    for var in variants:
        alt = torch_layer_bf16(inp, 2, **var)
        diff = [n for n in POINTS if not np.array_equal(got[n], alt[n].numpy())]
        assert "y" in diff, f"{var}: the misplaced rounding leaves y unchanged"
