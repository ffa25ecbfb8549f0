"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The host half of libkda (kda_api.hip: argument checks, the workspace query,
  status strings, test hooks) is rebuilt with the sanitizers and linked with
  the library's kernel objects into tests/sanitize/host_checks.c, which calls
  every entry point with bad arguments (all rejected before any HIP call, so
  no GPU is needed).
- The fp64 oracle (oracle/kda_oracle.c) is built with the sanitizers into
  tests/sanitize/oracle_checks.c, which runs a ragged batch with each initial
  state kind and several thread counts.

Only the host side is instrumented (no GPU sanitizer).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_tok_amd", "csrc")
BUILD = os.path.join(ROOT, "gated_delta_rule_tok_amd", "_build")
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-pthread", os.path.join(ROOT, "oracle", "kda_oracle.c"),
          os.path.join(SAN, "oracle_checks.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV)
    assert "0 failures" in r.stdout


def test_library_host_code_under_sanitizers(tmp_path):
    from gated_delta_rule_tok_amd import build as B
    hipcc = B.hipcc()
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    kernels = [o for o in sorted(glob.glob(os.path.join(BUILD, "*.hip.o")))
               if not o.endswith("kda_api.hip.o")]
    if not os.path.exists(clang) or len(kernels) < 5:
        pytest.skip("the library's objects are not built (python -m gated_delta_rule_tok_amd.build)")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    api = str(tmp_path / "api_san.o")
    _run([hipcc, f"--offload-arch={B.ARCH}", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
          *san, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "kda_api.hip"),
          "-o", api])
    drv = str(tmp_path / "host_checks.o")
    _run([clang, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(SAN, "host_checks.c"), "-o", drv])
    exe = str(tmp_path / "host_checks")
    _run([hipcc, f"--offload-arch={B.ARCH}", *san, api, drv, *kernels, "-o", exe])
    r = _run([exe], env=ENV)
    assert "0 failures" in r.stdout
