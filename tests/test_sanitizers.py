"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The C ABI's host side (combine_expert_amd/csrc/api.hip: argument checks and
  the choice of launches) is built with both sanitizers into a driver that
  replaces the kernel launchers with recorders (tests/sanitize/api_driver.cpp);
  no GPU is touched.
- The oracle is built with both sanitizers and the oracle pin suite runs on
  that build in a subprocess with the ASan runtime preloaded.

A sanitizer report makes the program exit non-zero (recovery is off).
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
PIN_FILES = ["tests/test_oracle_numbers.py", "tests/test_oracle_route.py",
             "tests/test_oracle_dispatch_combine.py", "tests/test_oracle_scaled.py",
             "tests/test_oracle_gemm.py", "tests/test_golden.py"]


def runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def symbols(path, dynamic=False):
    args = ["nm", "-D", path] if dynamic else ["nm", path]
    return subprocess.run(args, capture_output=True, text=True).stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_api_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_driver")
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *host_san,
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "combine_expert_amd", "csrc"),
           os.path.join(ROOT, "combine_expert_amd", "csrc", "api.hip"),
           os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    syms = symbols(exe)
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "not instrumented"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0 and "all passed" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]


@pytest.mark.skipif(runtime("libasan.so") is None or runtime("libubsan.so") is None,
                    reason="gcc sanitizer runtimes not installed")
def test_oracle_pins_under_sanitizers(tmp_path):
    lib = obuild.build(lib=str(tmp_path / "libmoe_oracle_san.so"), extra=SAN)
    assert "__asan_report" in symbols(lib, dynamic=True), "not instrumented"
    env = dict(os.environ, MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="2",
               LD_PRELOAD=f"{runtime('libasan.so')}:{runtime('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0")  # the interpreter's own allocations stay alive
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
