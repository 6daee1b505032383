"""CPU sanitizer runs: AddressSanitizer and UndefinedBehaviorSanitizer over the
fp64 oracle and over the HIP library's host-side argument checks.

* The oracle (oracle/spec_oracle.c) is compiled with gcc and both sanitizers
  into a driver (tests/sanitize/oracle_driver.c) that calls every oracle
  function on small seeded inputs: both dtypes, V = 1, a ragged chunk, -inf
  logits, out-of-range draft tokens, malformed tree parents and node counts.
* The library's host code is compiled with the sanitizers (device code as
  usual for gfx950) and driven by tests/sanitize/abi_driver.cpp, which calls
  every entry point with arguments it must reject before anything is
  enqueued, and the size queries.  No kernel is launched; no GPU is needed.

Both run with leak detection and abort on the first report.  Nothing here is
marked gpu.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fopenmp", "-I" + os.path.join(ROOT, "oracle"), "-o", exe,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "spec_oracle.c"),
          "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "all calls returned" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="ROCm toolchain not available")
def test_library_host_checks_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libspecverify_asan.so")
    # the sanitizers apply to the host pass only (device code is built as usual)
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-I" + os.path.join(ROOT, "include"), "-o", lib,
          os.path.join(ROOT, "draft_verification_row_amd", "csrc", "spec_verify.hip")])
    exe = str(tmp_path / "abi_driver")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"), "-o", exe,
          os.path.join(HERE, "abi_driver.cpp"), "-L" + str(tmp_path), "-lspecverify_asan",
          "-Wl,-rpath," + str(tmp_path)])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
