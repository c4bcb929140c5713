"""The backward entry point that allocates nothing (rsa_backward_noalloc),
called through the C ABI, against the ordinary rsa_backward_ex on the same
inputs: the two run the same kernels, so the gradients must agree bit for
bit, and both must meet the parity gates against the fp64 oracle. Two calls
in a row, the second with a smaller input, so that the second runs over what
the first left in the shared static array."""

import ctypes

import pytest
import torch

import sequence_transformer_attention_rsa_amd as rsa
from gates import assert_parity
from gpu_util import device, from_dev, inputs, mask_dev, say, to_dev

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def run_both(x, N, causal, dev):
    q, k, v, g = (to_dev(x[n], "bf16", dev) for n in ("q", "k", "v", "dout"))
    m = mask_dev(x["mask"], dev)
    B, H, L, d = q.shape
    out, lse = rsa.forward(q, k, v, m, N=N, return_lse=True, causal=causal)
    ref = rsa.backward(q, k, v, out, g, lse, m, N=N, causal=causal)
    # outputs preallocated and poisoned: the call below allocates nothing
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = rsa.load().rsa_backward_noalloc(_p(q), _p(k), _p(v), _p(out), _p(g), _p(lse), _p(m),
                                         B, H, L, d, N, rsa.RSA_BF16, rsa.RSA_CAUSAL if causal else 0,
                                         stream, _p(got[0]), _p(got[1]), _p(got[2]))
    assert st == 0, rsa.status_string(st)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_backward_on_two_calls(oracle_lib):
    dev = device()
    cases = [  # the second call is smaller than the first
        dict(B=2, H=3, L=1024, d=64, N=8, valid=(600, 1024), causal=False, seed=301),
        dict(B=1, H=2, L=256, d=128, N=4, valid=None, causal=True, seed=302),
    ]
    for c in cases:
        x = inputs(c["B"], c["H"], c["L"], c["d"], seed=c["seed"], dtype="bf16", valid_range=c["valid"],
                   with_dout=True)
        say("noalloc backward", c)
        ref, got = run_both(x, c["N"], c["causal"], dev)
        want = oracle_lib.backward(x["q"], x["k"], x["v"], x["dout"], x["mask"], N=c["N"], causal=c["causal"])
        for name, a, b, w in zip(("dq", "dk", "dv"), ref, got, want):
            assert torch.equal(a, b), f"{name}: differs from rsa_backward_ex"
            assert_parity(from_dev(b), w, "bf16", f"noalloc {name}", grad=True)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """B*H*L above 2097152 rows: RSA_ERR_SCRATCH, before any launch."""
    dev = device()
    t = torch.zeros(64, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(16, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = rsa.load().rsa_backward_noalloc(_p(t), _p(t), _p(t), _p(t), _p(t), _p(lse), None,
                                         1, 3, 1048576, 64, 64, rsa.RSA_BF16, 0, stream, _p(t), _p(t), _p(t))
    assert st == 7, rsa.status_string(st)
