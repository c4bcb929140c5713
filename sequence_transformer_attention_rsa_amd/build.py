"""Build librsa.so: the HIP kernels and the C ABI, compiled for gfx950.

    python -m sequence_transformer_attention_rsa_amd.build

Every HIP source is compiled with hipcc for gfx950 only. Packed fp32 vector
instructions are disabled in device code (`-packed-fp32-ops`); hipcc's host
pass warns that it does not know that feature, which is harmless.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librsa.so")

SOURCES = ["rsa_fwd.hip", "rsa_twopass.hip", "rsa_bwd.hip", "rsa_layer.hip", "rsa_static.hip", "rsa_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build librsa.so")
    return path


def _flags():
    return ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # the kernels never form a NaN from finite inputs (non-finite inputs
            # are outside the contract), so max/min need no NaN canonicalisation
            "-fno-honor-nans",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking librsa.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
