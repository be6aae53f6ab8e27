"""Build libmoe_expert.so (the HIP kernels and the C ABI of the MoE path) and
libmoe_calib.so (the measurement kernels of include/moe_calib.h), for gfx950
only.

    python -m combine_expert_amd.build

hipcc cross-compiles without a GPU.  Packed-fp32 instruction selection is
switched off for device code (-packed-fp32-ops); the host pass warns that it
does not know the feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_expert.so")
CALIB_DIR = os.path.join(PKG, "calib")
CALIB_LIB = os.path.join(PKG, "libmoe_calib.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def calib_sources():
    return sorted(glob.glob(os.path.join(CALIB_DIR, "*.hip")))


def headers():
    return sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [os.path.join(INCLUDE, "moe_expert.h"),
                                                           os.path.join(INCLUDE, "moe_calib.h")]


FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-command-line-argument", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops"]
OBJDIR = os.path.join(PKG, "_build")


def _filter(text: str) -> str:
    return "\n".join(line for line in text.splitlines()
                     if "packed-fp32-ops" not in line and "not a recognized feature" not in line)


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, _filter(r.stdout + r.stderr)


def _compile_link(srcs, lib, verbose):
    """Compile sources to objects in parallel, then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = []
    for src in srcs:
        obj = os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".o")
        jobs.append((src, obj, [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, src]))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(lambda j: (j, _run(j[2])), jobs))
    for (src, _, cmd), (rc, out) in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = lib + ".tmp%d" % os.getpid()
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
            *[j[1] for j in jobs]]
    rc, out = _run(link)
    if verbose:
        print(" ".join(link), flush=True)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip to an object (in parallel: the dispatch kernels
    are split by quantisation mode across several files) and link the library;
    then the same for the measurement kernels in calib/."""
    _compile_link(sources(), LIB, verbose)
    _compile_link(calib_sources(), CALIB_LIB, verbose)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB) or not os.path.exists(CALIB_LIB):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(CALIB_LIB))
    return any(os.path.getmtime(p) > t for p in sources() + calib_sources() + headers())


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
