"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer.

* The CPU oracle (oracle/dspark_oracle.c), built with gcc and both
  sanitizers, run by tests/sanitize/oracle_driver.c on inputs that reach its
  edge cases (NaN padding rows, greedy rows, forced tokens, K = 0 and 1, tiny
  vocabularies, empty residuals, out-of-range tokens).
* The host code of the C-ABI library, built by hipcc with the sanitizers on
  the host side only (the device code is compiled as usual and never runs
  here), run by tests/sanitize/abi_driver.c: the workspace-size functions over
  a grid of sizes past every limit, and the argument checks of every entry
  point, none of which reaches a HIP call.

A sanitizer report makes the program abort, so a nonzero exit fails the test.
"""

from __future__ import annotations

import os
import subprocess

import pytest

from ancestral_draft_token_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-o", exe,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "dspark_oracle.c"), "-lm"])
    r = _run([exe], env=SAN_ENV)
    assert "oracle driver ok" in r.stdout


def test_abi_host_code_under_sanitizers(tmp_path):
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    if not (os.path.exists(_build.hipcc()) and os.path.exists(clang)):
        pytest.skip("hipcc / clang not available")
    lib = str(tmp_path / "libdspark_san.so")
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-O3", "-Wall")]
    # the sanitizers apply to the host side only: each flag behind -Xarch_host
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([_build.hipcc(), *flags, "-O1", "-g", *host_san, f"-I{_build.INCLUDE}", "-o", lib, *_build.SOURCES])
    exe = str(tmp_path / "abi_driver")
    _run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          f"-I{_build.INCLUDE}", "-o", exe, os.path.join(HERE, "abi_driver.c"), lib,
          f"-Wl,-rpath,{tmp_path}"])
    r = _run([exe], env=SAN_ENV)
    assert "abi driver ok" in r.stdout
