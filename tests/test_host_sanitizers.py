"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each run in a child process with its sanitizer runtime preloaded
(the Python interpreter itself is not instrumented):

* the oracle, built by gcc with -fsanitize=address,undefined, against the
  oracle's quick pins (tests/mutant_check.py);
* the library's host side (argument validation, descriptor analysis, the
  planner with its footprint sizing and tile table, workspace sizing, the
  gradient shape mapping), built by hipcc's host pass only with the same
  sanitizers and CONV_I8_HOST_ONLY (no device code, launches compiled out),
  against tests/test_boundary.py loaded through CONV_I8_LIB.

A sanitizer report, or any failure, fails the test.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from oracle import build as oracle_build  # noqa: E402

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
CSRC = os.path.join(ROOT, "int8_convolution_forward_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1"}


def _runtime(compiler, name):
    path = subprocess.run([compiler, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_clean(cmd, env):
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-6000:]
    assert "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    rt = _runtime("gcc", "libasan.so")
    if rt is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = str(tmp_path / "liboracle_asan.so")
    oracle_build.compile_oracle(out=lib, extra=("-O1", "-g", "-fno-omit-frame-pointer",
                                                "-fsanitize=address,undefined",
                                                "-fno-sanitize-recover=undefined"))
    env = dict(os.environ, LD_PRELOAD=rt, OMP_NUM_THREADS="4", **SAN_ENV)
    out = _run_clean([sys.executable, os.path.join(HERE, "mutant_check.py"), lib], env)
    assert "all pins hold" in out


def test_library_host_side_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("no hipcc")
    rt = _runtime(CLANG, "libclang_rt.asan-x86_64.so")
    if rt is None:
        pytest.skip("clang has no AddressSanitizer runtime here")
    lib = str(tmp_path / "libconv_i8_host_asan.so")
    cmd = [HIPCC, "--offload-host-only", "-DCONV_I8_HOST_ONLY", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Wno-inline-asm", "-Wno-unused-variable",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libsan",
           "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, "conv_i8.hip"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=rt, CONV_I8_LIB=lib, **SAN_ENV)
    env.pop("CONV_I8_TILE", None)
    out = _run_clean([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                      os.path.join(HERE, "test_boundary.py")], env)
    assert " passed" in out and " failed" not in out
