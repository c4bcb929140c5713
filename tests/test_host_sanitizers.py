"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two native programs are built with gcc/g++ and run:
  * tests/native/oracle_check.c with oracle/oracle.c: the fp64 oracle on
    small cases (every ring size, key padding with rows that see no key, one
    rank's rows through explicit positions, the causal variant, the
    backward);
  * tests/native/api_host_check.cpp with the library's C ABI
    (csrc/rsa_api.cpp) compiled without device code: argument validation,
    workspace sizing and carving and dispatch, with the launch functions
    replaced by stubs that check every pointer derived from a caller's
    workspace stays inside it.
Any sanitizer report aborts the program (-fno-sanitize-recover=all), and
leaks are reported at exit.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "sequence_transformer_attention_rsa_amd", "csrc")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_check")
    run(["gcc", "-std=c11", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(NATIVE, "oracle_check.c"), "-lm", "-o", exe])
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    assert "oracle checks passed" in run([exe], env)


def test_abi_host_logic_under_sanitizers(tmp_path):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers not available")
    exe = str(tmp_path / "api_check")
    run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "rsa_api.cpp"),
         os.path.join(NATIVE, "api_host_check.cpp"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    assert "host checks passed" in run([exe], env)
