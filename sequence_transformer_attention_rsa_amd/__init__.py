"""Ring Self-Attention (RSA) on AMD Instinct MI355X -- Python binding.

A thin ctypes layer over ``librsa.so`` (C ABI in ``include/rsa.h``). It only
marshals arguments: shapes and dtypes are checked, outputs are allocated with
torch on the inputs' device, and the library is called on the current HIP
stream. Every step of the computation runs in the library's HIP kernels; if
the library is not built, every call raises.

    out = rsa.forward(q, k, v, key_mask=None, N=4)
    out, lse = rsa.forward(q, k, v, N=4, return_lse=True)
    out_local = rsa.forward_rank(q_local, k, v, N=64, rank=3)
    out = rsa.forward_twopass(q, k, v, N=4)      # score rows materialised
    dq, dk, dv = rsa.backward(q, k, v, out, dout, lse, N=8)
    y = rsa.layer_forward(x, weights, H=12, N=16)  # the encoder layer around RSA

Shapes: q, k, v, out, dout: [B, H, L, d] contiguous (q_local and out_local:
[B, H, L/N, d]); key_mask: [B, L] bool or uint8 (nonzero = valid key);
lse: [B, H, rows] fp32. dtypes: torch.float32 or torch.bfloat16.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "RSAError", "lib_path", "load", "forward", "forward_rank", "forward_twopass", "backward",
    "backward_preprocess", "backward_dq", "backward_dkdv",
    "forward_rank_workspace_bytes", "forward_twopass_workspace_bytes", "backward_workspace_bytes",
    "status_string", "linear", "qkv_projection", "output_projection", "layernorm", "layer_forward",
    "layer_forward_workspace_bytes", "LAYER_WEIGHTS",
    "backward_noalloc", "NOALLOC_SCRATCH_BYTES",
    "RSA_F32", "RSA_BF16",
]

RSA_F32 = 0
RSA_BF16 = 1
RSA_CAUSAL = 1
NOALLOC_SCRATCH_BYTES = 16 << 20   # RSA_NOALLOC_SCRATCH_BYTES

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librsa.so")
_lib = None

_vp = ctypes.c_void_p
_ci = ctypes.c_int
_sz = ctypes.c_size_t

# (name, restype, argtypes) for every symbol of include/rsa.h
SIGNATURES = {
    "rsa_forward": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _vp, _vp]),
    "rsa_forward_ex": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _vp, _vp]),
    "rsa_forward_rank": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _sz, _vp, _vp, _vp]),
    "rsa_forward_rank_ex": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _sz, _vp, _vp,
                                  _vp]),
    "rsa_forward_rank_workspace_bytes": (_sz, [_ci, _ci, _ci, _ci, _ci]),
    "rsa_forward_twopass": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _sz, _vp, _vp, _vp]),
    "rsa_forward_twopass_workspace_bytes": (_sz, [_ci, _ci, _ci, _ci, _ci]),
    "rsa_backward": (_ci, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci,
                           _vp, _sz, _vp, _vp, _vp, _vp]),
    "rsa_backward_ex": (_ci, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci,
                              _vp, _sz, _vp, _vp, _vp, _vp]),
    "rsa_backward_workspace_bytes": (_sz, [_ci, _ci, _ci, _ci, _ci, _ci]),
    "rsa_backward_noalloc": (_ci, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci,
                                   _vp, _vp, _vp, _vp]),
    "rsa_forward_dropout": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _vp, _vp, _vp]),
    "rsa_forward_rank_dropout": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _vp, _sz,
                                       _vp, _vp, _vp]),
    "rsa_backward_dropout": (_ci, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp,
                                   _vp, _sz, _vp, _vp, _vp, _vp]),
    "rsa_backward_preprocess": (_ci, [_vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _vp, _vp]),
    "rsa_backward_dq": (_ci, [_vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _vp]),
    "rsa_backward_dkdv": (_ci, [_vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _vp, _vp]),
    "rsa_linear": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _vp, _vp]),
    "rsa_qkv_projection": (_ci, [_vp, _vp, _vp, _ci, _ci, _ci, _ci, _vp, _vp, _vp, _vp]),
    "rsa_output_projection": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _vp, _vp]),
    "rsa_layernorm": (_ci, [_vp, _vp, _vp, _ci, _ci, ctypes.c_float, _vp, _vp]),
    "rsa_layer_forward": (_ci, [_vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _sz, _vp, _vp]),
    "rsa_layer_forward_workspace_bytes": (_sz, [_ci, _ci, _ci, _ci, _ci, _ci]),
    "rsa_status_string": (ctypes.c_char_p, [_ci]),
}

# Field order of struct rsa_layer_weights (matrices bf16, vectors fp32).
LAYER_WEIGHTS = ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_gamma", "ln1_beta",
                 "w_ff1", "b_ff1", "w_ff2", "b_ff2", "ln2_gamma", "ln2_beta")


class _LayerWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in LAYER_WEIGHTS]


class _Dropout(ctypes.Structure):
    """struct rsa_dropout: drop probability, fourth counter word, Philox key."""
    _fields_ = [("p", ctypes.c_float), ("offset", ctypes.c_uint32), ("seed", ctypes.c_uint64)]


def _dropout(dropout):
    """None, or (p, seed[, offset]) -> a struct rsa_dropout (kept alive by the caller)."""
    if dropout is None:
        return None
    p, seed = float(dropout[0]), int(dropout[1])
    offset = int(dropout[2]) if len(dropout) > 2 else 0
    return _Dropout(p, offset & 0xFFFFFFFF, seed & 0xFFFFFFFFFFFFFFFF)


def _ref(s):
    return None if s is None else ctypes.byref(s)


class RSAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load librsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built; run `python -m sequence_transformer_attention_rsa_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().rsa_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RSA_F32
    if t.dtype == torch.bfloat16:
        return RSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.float32 or torch.bfloat16")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _mask(key_mask, B, L, device):
    if key_mask is None:
        return None
    if key_mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError("key_mask must be bool or uint8")
    _need(key_mask, "key_mask", (B, L), key_mask.dtype, device)
    return key_mask


def forward(q, k, v, key_mask=None, N: int = 1, return_lse: bool = False, out=None, lse=None,
            causal: bool = False, dropout=None):
    """RSA forward over all N ranks: softmax(q k^T / sqrt(d) + mask) v
    (causal: the row at position i sees keys j <= i only; dropout: None or
    (p, seed[, offset]), dropout of the softmax weights, see rsa.h)."""
    B, H, L, d = q.shape
    dev = q.device
    _need(q, "q", (B, H, L, d), q.dtype, dev)
    _need(k, "k", (B, H, L, d), q.dtype, dev)
    _need(v, "v", (B, H, L, d), q.dtype, dev)
    m = _mask(key_mask, B, L, dev)
    code = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", (B, H, L, d), q.dtype, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (B, H, L), torch.float32, dev)
    if dropout is not None:
        dr = _dropout(dropout)
        st = load().rsa_forward_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(m), B, H, L, d, int(N), code,
                                        RSA_CAUSAL if causal else 0, _ref(dr), _stream(dev), _ptr(out), _ptr(lse))
    elif causal:
        st = load().rsa_forward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(m), B, H, L, d, int(N), code, RSA_CAUSAL,
                                   _stream(dev), _ptr(out), _ptr(lse))
    else:
        st = load().rsa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(m), B, H, L, d, int(N), code,
                                _stream(dev), _ptr(out), _ptr(lse))
    if st != 0:
        raise RSAError(st, "rsa_forward")
    return (out, lse) if (return_lse or lse is not None) else out


def forward_rank_workspace_bytes(B: int, H: int, L: int, d: int, N: int) -> int:
    return int(load().rsa_forward_rank_workspace_bytes(B, H, L, d, N))


def forward_rank(q_local, k, v, key_mask=None, N: int = 1, rank: int = 0, return_lse: bool = False,
                 out=None, lse=None, workspace=None, causal: bool = False, dropout=None):
    """One rank's share: q_local [B,H,L/N,d] against all L keys in that rank's ring order."""
    B, H, L, d = k.shape
    dev = k.device
    if N <= 0 or L % N != 0:
        raise ValueError("N must divide L")
    Lc = L // N
    _need(q_local, "q_local", (B, H, Lc, d), k.dtype, dev)
    _need(v, "v", (B, H, L, d), k.dtype, dev)
    m = _mask(key_mask, B, L, dev)
    code = _dtype_code(k)
    if out is None:
        out = torch.empty_like(q_local)
    _need(out, "out", (B, H, Lc, d), k.dtype, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Lc), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (B, H, Lc), torch.float32, dev)
    need = forward_rank_workspace_bytes(B, H, L, d, N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if dropout is not None:
        dr = _dropout(dropout)
        st = load().rsa_forward_rank_dropout(_ptr(q_local), _ptr(k), _ptr(v), _ptr(m), B, H, L, d, int(N), int(rank),
                                             code, RSA_CAUSAL if causal else 0, _ref(dr), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(dev), _ptr(out),
                                             _ptr(lse))
    elif causal:
        st = load().rsa_forward_rank_ex(_ptr(q_local), _ptr(k), _ptr(v), _ptr(m), B, H, L, d, int(N), int(rank),
                                        code, RSA_CAUSAL, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(dev), _ptr(out),
                                        _ptr(lse))
    else:
        st = load().rsa_forward_rank(_ptr(q_local), _ptr(k), _ptr(v), _ptr(m), B, H, L, d, int(N), int(rank),
                                     code, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(dev), _ptr(out), _ptr(lse))
    if st != 0:
        raise RSAError(st, "rsa_forward_rank")
    return (out, lse) if (return_lse or lse is not None) else out


def forward_twopass_workspace_bytes(B: int, H: int, L: int, d: int, N: int) -> int:
    return int(load().rsa_forward_twopass_workspace_bytes(B, H, L, d, N))


def forward_twopass(q, k, v, key_mask=None, N: int = 1, return_lse: bool = False, out=None, lse=None,
                    workspace=None):
    """The forward with every score row materialised (fp32 [B,H,L,L] in the
    workspace), softmax over each row, then the weighted sum of v. bf16 only."""
    B, H, L, d = q.shape
    dev = q.device
    _need(q, "q", (B, H, L, d), q.dtype, dev)
    _need(k, "k", (B, H, L, d), q.dtype, dev)
    _need(v, "v", (B, H, L, d), q.dtype, dev)
    m = _mask(key_mask, B, L, dev)
    code = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", (B, H, L, d), q.dtype, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (B, H, L), torch.float32, dev)
    if workspace is None:
        need = forward_twopass_workspace_bytes(B, H, L, d, N)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = load().rsa_forward_twopass(_ptr(q), _ptr(k), _ptr(v), _ptr(m), B, H, L, d, int(N), code,
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(dev), _ptr(out), _ptr(lse))
    if st != 0:
        raise RSAError(st, "rsa_forward_twopass")
    return (out, lse) if (return_lse or lse is not None) else out


def backward_workspace_bytes(B: int, H: int, L: int, d: int, N: int, dtype: int = RSA_BF16) -> int:
    return int(load().rsa_backward_workspace_bytes(B, H, L, d, N, dtype))


def backward_preprocess(out, dout, lse, rowstats=None):
    """Stage 1 of the backward: row statistics, fp32 [2, B, H, L]
    (-rowsum(dout * out), -lse * log2(e))."""
    B, H, L, d = out.shape
    dev = out.device
    _need(out, "out", (B, H, L, d), out.dtype, dev)
    _need(dout, "dout", (B, H, L, d), out.dtype, dev)
    _need(lse, "lse", (B, H, L), torch.float32, dev)
    if rowstats is None:
        rowstats = torch.empty((2, B, H, L), dtype=torch.float32, device=dev)
    _need(rowstats, "rowstats", (2, B, H, L), torch.float32, dev)
    st = load().rsa_backward_preprocess(_ptr(out), _ptr(dout), _ptr(lse), B, H, L, d, _dtype_code(out),
                                        _stream(dev), _ptr(rowstats))
    if st != 0:
        raise RSAError(st, "rsa_backward_preprocess")
    return rowstats


def _stage_args(q, k, v, dout, rowstats, key_mask):
    B, H, L, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _need(t, name, (B, H, L, d), q.dtype, dev)
    _need(rowstats, "rowstats", (2, B, H, L), torch.float32, dev)
    return B, H, L, d, dev, _mask(key_mask, B, L, dev)


def backward_dq(q, k, v, dout, rowstats, key_mask=None, N: int = 1, dq=None):
    """Stage 2 of the backward: dq."""
    B, H, L, d, dev, m = _stage_args(q, k, v, dout, rowstats, key_mask)
    dq = torch.empty_like(q) if dq is None else dq
    _need(dq, "dq", (B, H, L, d), q.dtype, dev)
    st = load().rsa_backward_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(rowstats), _ptr(m),
                                B, H, L, d, int(N), _dtype_code(q), _stream(dev), _ptr(dq))
    if st != 0:
        raise RSAError(st, "rsa_backward_dq")
    return dq


def backward_dkdv(q, k, v, dout, rowstats, key_mask=None, N: int = 1, dk=None, dv=None):
    """Stage 3 of the backward: dk and dv."""
    B, H, L, d, dev, m = _stage_args(q, k, v, dout, rowstats, key_mask)
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _need(dk, "dk", (B, H, L, d), q.dtype, dev)
    _need(dv, "dv", (B, H, L, d), q.dtype, dev)
    st = load().rsa_backward_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(rowstats), _ptr(m),
                                  B, H, L, d, int(N), _dtype_code(q), _stream(dev), _ptr(dk), _ptr(dv))
    if st != 0:
        raise RSAError(st, "rsa_backward_dkdv")
    return dk, dv


def backward(q, k, v, out, dout, lse, key_mask=None, N: int = 1, dq=None, dk=None, dv=None, workspace=None,
             causal: bool = False, dropout=None):
    """Gradients (dq, dk, dv) of <out, dout>; out and lse come from forward()
    with the same causal and dropout settings."""
    B, H, L, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _need(t, name, (B, H, L, d), q.dtype, dev)
    _need(lse, "lse", (B, H, L), torch.float32, dev)
    m = _mask(key_mask, B, L, dev)
    code = _dtype_code(q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, name, (B, H, L, d), q.dtype, dev)
    need = backward_workspace_bytes(B, H, L, d, N, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if dropout is not None:
        dr = _dropout(dropout)
        st = load().rsa_backward_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(m),
                                         B, H, L, d, int(N), code, RSA_CAUSAL if causal else 0, _ref(dr),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(dev), _ptr(dq), _ptr(dk), _ptr(dv))
    elif causal:
        st = load().rsa_backward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(m),
                                    B, H, L, d, int(N), code, RSA_CAUSAL, _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(dev),
                                    _ptr(dq), _ptr(dk), _ptr(dv))
    else:
        st = load().rsa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(m),
                                 B, H, L, d, int(N), code, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev),
                                 _ptr(dq), _ptr(dk), _ptr(dv))
    if st != 0:
        raise RSAError(st, "rsa_backward")
    return dq, dk, dv


def backward_noalloc(q, k, v, out, dout, lse, key_mask=None, N: int = 1, dq=None, dk=None, dv=None,
                     causal: bool = False):
    """backward() without a workspace: the library keeps the row statistics in
    its static device array (at most B*H*L = 2097152 rows; calls that overlap
    on one GPU race). Pass dq, dk and dv to allocate nothing at all."""
    B, H, L, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _need(t, name, (B, H, L, d), q.dtype, dev)
    _need(lse, "lse", (B, H, L), torch.float32, dev)
    m = _mask(key_mask, B, L, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, name, (B, H, L, d), q.dtype, dev)
    st = load().rsa_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(m),
                                     B, H, L, d, int(N), _dtype_code(q), RSA_CAUSAL if causal else 0,
                                     _stream(dev), _ptr(dq), _ptr(dk), _ptr(dv))
    if st != 0:
        raise RSAError(st, "rsa_backward_noalloc")
    return dq, dk, dv


# ------------------------------------------------ the layer around RSA ---

def _bf16(t, name, shape, device):
    _need(t, name, shape, torch.bfloat16, device)


def _vec(t, name, n, device, optional=True):
    if t is None and optional:
        return None
    _need(t, name, (n,), torch.float32, device)
    return t


def linear(a, w, bias=None, residual=None, activation: str = "none", out=None):
    """out = act(a w^T + bias) + residual; a [M,K], w [N,K] bf16, bias [N] fp32;
    activation "none" or "gelu" (applied before the residual)."""
    M, K = a.shape
    N = w.shape[0]
    dev = a.device
    _bf16(a, "a", (M, K), dev)
    _bf16(w, "w", (N, K), dev)
    _vec(bias, "bias", N, dev)
    if residual is not None:
        _bf16(residual, "residual", (M, N), dev)
    act = {"none": 0, "gelu": 1}[activation]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    _bf16(out, "out", (M, N), dev)
    st = load().rsa_linear(_ptr(a), _ptr(w), _ptr(bias), _ptr(residual), M, N, K, act, _stream(dev), _ptr(out))
    if st != 0:
        raise RSAError(st, "rsa_linear")
    return out


def qkv_projection(x, w_qkv, b_qkv, H: int):
    """Q, K, V [B,H,L,d] from x [B,L,E] (head split fused into the product)."""
    B, L, E = x.shape
    dev = x.device
    _bf16(x, "x", (B, L, E), dev)
    _bf16(w_qkv, "w_qkv", (3 * E, E), dev)
    _vec(b_qkv, "b_qkv", 3 * E, dev)
    if E % H != 0:
        raise ValueError("H must divide E")
    q, k, v = (torch.empty((B, H, L, E // H), dtype=torch.bfloat16, device=dev) for _ in range(3))
    st = load().rsa_qkv_projection(_ptr(x), _ptr(w_qkv), _ptr(b_qkv), B, L, E, H, _stream(dev),
                                   _ptr(q), _ptr(k), _ptr(v))
    if st != 0:
        raise RSAError(st, "rsa_qkv_projection")
    return q, k, v


def output_projection(o, w_o, b_o=None, residual=None):
    """merge(o) w_o^T + b_o + residual, o [B,H,L,d] -> [B,L,E]."""
    B, H, L, d = o.shape
    E = H * d
    dev = o.device
    _bf16(o, "o", (B, H, L, d), dev)
    _bf16(w_o, "w_o", (E, E), dev)
    _vec(b_o, "b_o", E, dev)
    if residual is not None:
        _bf16(residual, "residual", (B, L, E), dev)
    out = torch.empty((B, L, E), dtype=torch.bfloat16, device=dev)
    st = load().rsa_output_projection(_ptr(o), _ptr(w_o), _ptr(b_o), _ptr(residual), B, L, E, H, _stream(dev),
                                      _ptr(out))
    if st != 0:
        raise RSAError(st, "rsa_output_projection")
    return out


def layernorm(x, gamma, beta, eps: float = 1e-12):
    """Layer normalisation over the last axis of a bf16 tensor."""
    E = x.shape[-1]
    rows = x.numel() // E
    dev = x.device
    _bf16(x, "x", tuple(x.shape), dev)
    _vec(gamma, "gamma", E, dev, optional=False)
    _vec(beta, "beta", E, dev, optional=False)
    y = torch.empty_like(x)
    st = load().rsa_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), rows, E, float(eps), _stream(dev), _ptr(y))
    if st != 0:
        raise RSAError(st, "rsa_layernorm")
    return y


def layer_forward_workspace_bytes(B: int, L: int, E: int, H: int, F: int, N: int) -> int:
    return int(load().rsa_layer_forward_workspace_bytes(B, L, E, H, F, N))


def layer_forward(x, weights: dict, H: int, N: int = 1, key_mask=None, out=None, workspace=None):
    """The encoder layer around RSA: x [B,L,E] bf16 -> y [B,L,E] bf16.

    weights: dict with the LAYER_WEIGHTS names; matrices bf16 (w_qkv [3E,E],
    w_o [E,E], w_ff1 [F,E], w_ff2 [E,F]), vectors fp32 (biases may be None).
    """
    B, L, E = x.shape
    dev = x.device
    _bf16(x, "x", (B, L, E), dev)
    F = weights["w_ff1"].shape[0]
    _bf16(weights["w_qkv"], "w_qkv", (3 * E, E), dev)
    _bf16(weights["w_o"], "w_o", (E, E), dev)
    _bf16(weights["w_ff1"], "w_ff1", (F, E), dev)
    _bf16(weights["w_ff2"], "w_ff2", (E, F), dev)
    for name, n in (("b_qkv", 3 * E), ("b_o", E), ("b_ff1", F), ("b_ff2", E)):
        _vec(weights.get(name), name, n, dev)
    for name in ("ln1_gamma", "ln1_beta", "ln2_gamma", "ln2_beta"):
        _vec(weights[name], name, E, dev, optional=False)
    m = _mask(key_mask, B, L, dev)
    ws = _LayerWeights(*[None if weights.get(n) is None else weights[n].data_ptr() for n in LAYER_WEIGHTS])
    y = torch.empty_like(x) if out is None else out
    _bf16(y, "out", (B, L, E), dev)
    if workspace is None:
        need = layer_forward_workspace_bytes(B, L, E, H, F, N)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = load().rsa_layer_forward(_ptr(x), _ptr(m), ctypes.addressof(ws), B, L, E, H, F, int(N), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(dev), _ptr(y))
    if st != 0:
        raise RSAError(st, "rsa_layer_forward")
    return y
