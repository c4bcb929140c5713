"""fp64 CPU oracle for Ring Self-Attention -- test infrastructure only.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this package. It shares no code with the HIP library: ``oracle.c`` is
compiled by gcc into ``liboracle.so`` and called through ctypes here;
``brute.py`` evaluates the dense definition in 50-digit decimal arithmetic.

What the oracle computes is stated at the top of ``oracle.c``: plain
scaled-dot-product attention with a key-padding mask, evaluated through the
two ring-ordered stages of Ring Self-Attention (review page of "Sequence
Parallelism: Making 4D Parallelism Possible", ABSTRACT and proposed-method
section), and its gradients.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (fp64, OpenMP, no -ffast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i64p = ctypes.POINTER(ctypes.c_int64)
        ci = ctypes.c_int
        u64, u32 = ctypes.c_uint64, ctypes.c_uint32
        lib.oracle_forward.argtypes = [dp, dp, dp, u8p, ci, ci, ci, ci, ci, ci, i64p, ci, ci, u64, u32, dp, dp]
        lib.oracle_forward.restype = ci
        lib.oracle_backward.argtypes = [dp, dp, dp, dp, u8p, ci, ci, ci, ci, ci, ci, ci, u64, u32, dp, dp, dp]
        lib.oracle_backward.restype = ci
        lib.oracle_philox4x32_10.argtypes = [ctypes.POINTER(u32), ctypes.POINTER(u32), ctypes.POINTER(u32)]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_philox4x64_10.argtypes = [ctypes.POINTER(u64), ctypes.POINTER(u64), ctypes.POINTER(u64)]
        lib.oracle_philox4x64_10.restype = None
        lib.oracle_dropout_keep.argtypes = [ci, u64, u32, ctypes.c_int64, ctypes.c_int64, ci, ctypes.c_int64, ci,
                                            u8p]
        lib.oracle_dropout_keep.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ci
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: Optional[np.ndarray], ctype):
    if a is None:
        return ctypes.POINTER(ctype)()
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def num_threads() -> int:
    """OpenMP threads the oracle uses (set OMP_NUM_THREADS before loading)."""
    return int(_load().oracle_num_threads())


def dropout_p8(p: float) -> int:
    """The dropout probability quantised to 1/256 steps: p is taken as fp32,
    p8 = floor(256 p + 1/2), and the weights are dropped with probability
    p8 / 256. p8 must lie in [0, 256)."""
    p32 = float(np.float32(p))
    p8 = int(np.floor(p32 * 256.0 + 0.5))
    if not (0 <= p8 < 256):
        raise ValueError(f"dropout probability {p} outside [0, 1 - 1/512)")
    return p8


def _dropout_args(dropout):
    """(p8, seed, offset) from None or (p, seed[, offset])."""
    if dropout is None:
        return 0, 0, 0
    p, seed = dropout[0], int(dropout[1])
    offset = int(dropout[2]) if len(dropout) > 2 else 0
    return dropout_p8(p), seed & (2 ** 64 - 1), offset & (2 ** 32 - 1)


def philox4x32_10(counter, key) -> np.ndarray:
    """Philox-4x32-10 of a 4-word counter and a 2-word key (uint32 words)."""
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    _load().oracle_philox4x32_10(c.ctypes.data_as(u32p), k.ctypes.data_as(u32p), out.ctypes.data_as(u32p))
    return out


def philox4x64_10(counter, key) -> np.ndarray:
    """Philox-4x64-10 of a 4-word counter and a 2-word key (uint64 words)."""
    c = np.ascontiguousarray(counter, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.empty(4, dtype=np.uint64)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    _load().oracle_philox4x64_10(c.ctypes.data_as(u64p), k.ctypes.data_as(u64p), out.ctypes.data_as(u64p))
    return out


def dropout_keep(dropout, bh: int, i0: int, ni: int, j0: int, nj: int) -> np.ndarray:
    """Keep decisions [ni, nj] (1 = kept) of the weights of query positions
    i0.. and key positions j0.. of head bh = b * H + h; dropout = (p, seed[,
    offset])."""
    p8, seed, offset = _dropout_args(dropout)
    out = np.empty((ni, nj), dtype=np.uint8)
    _load().oracle_dropout_keep(p8, seed, offset, bh, i0, ni, j0, nj, _ptr(out, ctypes.c_uint8))
    return out


def forward(q, k, v, mask=None, N: int = 1, qpos=None, causal: bool = False,
            dropout=None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 attention output and natural-log lse through RSA's ring stages.

    q: [B,H,Lq,d]; k, v: [B,H,L,d]; mask: [B,L] (nonzero = valid) or None;
    qpos: absolute positions of q's rows (default 0..Lq-1), which fix each
    row's rank and so its ring order; causal: the row at position i sees
    keys j <= i only; dropout: None or (p, seed[, offset]) -- the softmax
    weights of head b*H + h are dropped as oracle.c's dropout_keep() decides
    (the heads' indices come from q's [B,H] layout). Returns
    (out [B,H,Lq,d], lse [B,H,Lq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Lq, d = q.shape
    L = k.shape[2]
    if k.shape != (B, H, L, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B,H,L,d] matching q")
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    if m is not None and m.shape != (B, L):
        raise ValueError("mask must be [B,L]")
    pos = None
    if qpos is not None:
        pos = np.ascontiguousarray(qpos, dtype=np.int64)
        if pos.shape != (Lq,) or np.any(pos < 0) or np.any(pos >= L):
            raise ValueError("qpos must hold Lq positions in [0, L)")
    elif Lq != L:
        raise ValueError("qpos is required when q does not hold all L rows")
    out = np.empty((B, H, Lq, d), dtype=np.float64)
    lse = np.empty((B, H, Lq), dtype=np.float64)
    st = _load().oracle_forward(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                _ptr(v, ctypes.c_double), _ptr(m, ctypes.c_uint8),
                                B, H, L, d, N, Lq, _ptr(pos, ctypes.c_int64), int(bool(causal)),
                                *_dropout_args(dropout), _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if st != 0:
        raise ValueError(f"oracle_forward failed with status {st}")
    return out, lse


def backward(q, k, v, dout, mask=None, N: int = 1, causal: bool = False,
             dropout=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """fp64 gradients (dQ, dK, dV) of <O, dO>, all [B,H,L,d] (causal and
    dropout as in forward)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, L, d = q.shape
    for name, a in (("k", k), ("v", v), ("dout", g)):
        if a.shape != q.shape:
            raise ValueError(f"{name} must be [B,H,L,d] like q")
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    if m is not None and m.shape != (B, L):
        raise ValueError("mask must be [B,L]")
    dq = np.empty_like(q)
    dk = np.empty_like(q)
    dv = np.empty_like(q)
    st = _load().oracle_backward(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                 _ptr(v, ctypes.c_double), _ptr(g, ctypes.c_double),
                                 _ptr(m, ctypes.c_uint8), B, H, L, d, N, int(bool(causal)),
                                 *_dropout_args(dropout), _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double),
                                 _ptr(dv, ctypes.c_double))
    if st != 0:
        raise ValueError(f"oracle_backward failed with status {st}")
    return dq, dk, dv
