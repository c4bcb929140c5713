"""Build librsa.so: the HIP kernels and the C ABI, compiled for gfx950.

    python -m sequence_transformer_attention_rsa_amd.build

Every HIP source is compiled with hipcc for gfx950 only. Packed fp32 vector
instructions are disabled in device code (`-packed-fp32-ops`); hipcc's host
pass warns that it does not know that feature, which is harmless.
"""

from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librsa.so")

SOURCES = ["rsa_fwd.hip", "rsa_twopass.hip", "rsa_bwd.hip", "rsa_bwd_f32.hip", "rsa_layer.hip", "rsa_static.hip",
           "rsa_api.cpp"]
ARCH = "gfx950"
# Sources whose kernels issue HBM->LDS copies from inline assembly that sets
# m0 (rsa_tiles.h: dma_copy16, dma_copy4). The compiler does not know the
# assembly writes m0, so those kernels must contain no compiler-generated
# instruction that reads or writes m0; m0_violations() checks the device
# assembly of every build.
UNTRACKED_COPY_SOURCES = ["rsa_fwd.hip", "rsa_bwd.hip", "rsa_layer.hip"]


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


# Instructions that use m0 without naming it: relative register moves,
# messages, GWS/append/ordered LDS operations, and copies into LDS.
_IMPLICIT_M0 = re.compile(r"^(v_movrel|s_movrel|s_sendmsg|ds_gws|ds_append|ds_consume|ds_ordered|"
                          r"global_load_lds|scratch_load_lds|buffer_load\S*\s.*\blds\b)")


def m0_violations(asm: str) -> list:
    """Functions of a device assembly listing that write m0 from inline
    assembly (between ;;#ASMSTART and ;;#ASMEND) and also contain a
    compiler-generated instruction that names m0 or uses it implicitly.
    Returns "function: instruction" strings (empty when the listing is safe)."""
    funcs = set(re.findall(r"^\s*\.type\s+([^,\s]+),@function", asm, flags=re.M))
    out = []
    name, in_asm, writes, others = None, False, False, []
    for raw in asm.splitlines():
        line = raw.split(";;")[0].strip() if not raw.strip().startswith(";;#ASM") else raw.strip()
        if name is None:
            m = re.match(r"^([^\s:]+):", line)
            if m and m.group(1) in funcs:
                name, in_asm, writes, others = m.group(1), False, False, []
            continue
        if line.startswith(".Lfunc_end"):
            if writes and others:
                out += [f"{name}: {o}" for o in others]
            name = None
            continue
        if line == ";;#ASMSTART":
            in_asm = True
            continue
        if line == ";;#ASMEND":
            in_asm = False
            continue
        if not line or line.startswith((".", ";")) or line.endswith(":"):
            continue
        touches = re.search(r"\bm0\b", line) is not None or _IMPLICIT_M0.match(line) is not None
        if in_asm:
            writes |= re.match(r"^s_mov_b32\s+m0\b", line) is not None
        elif touches:
            others.append(line)
    return out


def _device_asm(src: str, extra=()) -> str:
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "dev.s")
        cmd = [hipcc(), *_flags(), *extra, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"device assembly of {src} failed:\n{r.stdout}\n{r.stderr}")
        return open(out).read()


def check_untracked_copies(extra=(), executor=None) -> None:
    """Fail the build if a kernel that writes m0 from inline assembly also has
    compiler-generated code that uses m0."""
    ex = executor or concurrent.futures.ThreadPoolExecutor(max_workers=len(UNTRACKED_COPY_SOURCES))
    bad = []
    for src, asm in zip(UNTRACKED_COPY_SOURCES, ex.map(lambda s: _device_asm(s, extra), UNTRACKED_COPY_SOURCES)):
        bad += [f"{src}: {v}" for v in m0_violations(asm)]
    if bad:
        raise RuntimeError("compiler-generated m0 use in kernels with untracked copies:\n" + "\n".join(bad[:20]))


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + len(UNTRACKED_COPY_SOURCES)) as ex:
        guard = ex.submit(check_untracked_copies, extra, ex)
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
        guard.result()
    tmp = LIB + ".tmp"
    # every symbol resolved at link time: a kernel source missing from SOURCES fails here
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking librsa.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
