"""The measurement library without a GPU: libmoe_calib.so loads, exports every
function include/moe_calib.h declares, and rejects bad arguments on the host
before anything is enqueued (no pointer is ever dereferenced by these calls).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_calib.h")
P = 0x10000  # a 16-byte aligned stand-in address; never dereferenced here


def declared_functions():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_calib_\w+)\s*\(", src, re.M)))


def test_header_declares_the_measurement_kernels():
    assert declared_functions() == ["moe_calib_gather_shape", "moe_calib_scatter_shape",
                                    "moe_calib_stream"]


def test_library_exports_every_declared_symbol():
    from combine_expert_amd import calib
    out = subprocess.run(["nm", "-D", "--defined-only", calib.library_path()],
                         capture_output=True, text=True, check=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, re.M), name
    assert sorted(calib.EXPORTS) == declared_functions()


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


@pytest.mark.skipif(not _no_gpu(), reason="validation-only calls are made without a GPU")
def test_bad_arguments_are_rejected_before_launch():
    from combine_expert_amd import calib
    L = calib.raw()
    assert L.moe_calib_stream(None, 16, P, 16, 1, None) == 1
    assert L.moe_calib_stream(P + 8, 16, P, 16, 1, None) == 1          # misaligned
    assert L.moe_calib_stream(P, 15, P, 16, 1, None) == 1              # not a multiple of 16
    assert L.moe_calib_stream(P, 0, P, 0, 1, None) == 1                # nothing to move
    assert L.moe_calib_stream(P, (1 << 31) + 16, P, 16, 1, None) == 1  # too large
    assert L.moe_calib_stream(P, 16, P, 16, 3, None) == 1              # no such policy
    assert L.moe_calib_scatter_shape(P, P, 512, 7168, 8, 4096 + 1, P, 1, None) == 1  # rows > Bs*K
    assert L.moe_calib_scatter_shape(P, P, 513, 7168, 8, 4096, P, 1, None) == 1
    assert L.moe_calib_scatter_shape(P, P, 512, 7200 + 16, 8, 4096, P, 1, None) == 1  # H % 32
    assert L.moe_calib_scatter_shape(P, P, 512, 7168, 8, 4096, P, -1, None) == 1
    assert L.moe_calib_gather_shape(P, P, P, P, P, 512, 7168, 17, 4096, P, P, 1, None) == 1
    assert L.moe_calib_gather_shape(P, P, P, P, None, 512, 7168, 8, 4096, P, P, 1, None) == 1
