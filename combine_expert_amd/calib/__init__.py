"""ctypes binding of libmoe_calib.so (include/moe_calib.h): measurement
kernels that move bytes in the shapes of the dispatch and combine kernels
with none of their arithmetic, used by bench.py to report the ceilings the
method's kernels are measured against.  Not part of the dispatch / combine
path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

from .. import build as _build

EXPORTS = ("moe_calib_stream", "moe_calib_scatter_shape", "moe_calib_gather_shape")

if not os.path.exists(_build.CALIB_LIB):
    raise ImportError(f"{_build.CALIB_LIB} is not built: run `python -m combine_expert_amd.build`")

_lib = C.CDLL(_build.CALIB_LIB)
_P, _I, _S = C.c_void_p, C.c_int, C.c_size_t
_lib.moe_calib_stream.argtypes = [_P, _S, _P, _S, _I, _P]
_lib.moe_calib_scatter_shape.argtypes = [_P, _P, _I, _I, _I, _I, _P, _I, _P]
_lib.moe_calib_gather_shape.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P]

STORE_PLAIN, STORE_STREAM, STORE_DEVICE = 0, 1, 2
POLICIES = {"plain": STORE_PLAIN, "non-temporal": STORE_STREAM, "write-through": STORE_DEVICE}
for _n in EXPORTS:
    getattr(_lib, _n).restype = C.c_int


def library_path() -> str:
    return _build.CALIB_LIB


def raw():
    return _lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(name, rc):
    if rc != 0:
        raise RuntimeError(f"{name} returned {rc}")


def stream(src: torch.Tensor, read_bytes: int, dst: torch.Tensor, write_bytes: int,
           policy: int = STORE_STREAM):
    assert src.is_cuda and dst.is_cuda
    assert src.numel() * src.element_size() >= read_bytes
    assert dst.numel() * dst.element_size() >= write_bytes
    _check("moe_calib_stream", _lib.moe_calib_stream(src.data_ptr(), read_bytes, dst.data_ptr(),
                                                     write_bytes, policy, _stream()))


def scatter_shape(x: torch.Tensor, assist: torch.Tensor, n_rows: int, out: torch.Tensor,
                  policy: int = STORE_STREAM):
    Bs, H = x.shape
    K = assist.numel() // Bs
    assert x.dtype == torch.bfloat16 and assist.dtype == torch.int32 and out.dtype == torch.uint8
    assert out.numel() >= n_rows * H and assist.numel() == Bs * K
    _check("moe_calib_scatter_shape",
           _lib.moe_calib_scatter_shape(x.data_ptr(), assist.data_ptr(), Bs, H, K, n_rows,
                                        out.data_ptr(), policy, _stream()))


def gather_shape(rows: torch.Tensor, assist: torch.Tensor, a: torch.Tensor, b, gamma: torch.Tensor,
                 n_rows: int, out1: torch.Tensor, out2: torch.Tensor, policy: int = STORE_STREAM):
    """b may be None: the combine's shape without a shared expert."""
    Bs, H = a.shape
    K = assist.numel() // Bs
    for t in (rows, a, b, gamma, out1, out2):
        assert t is None or (t.dtype == torch.bfloat16 and t.is_cuda and t.is_contiguous())
    assert rows.numel() >= n_rows * H and assist.numel() == Bs * K
    _check("moe_calib_gather_shape",
           _lib.moe_calib_gather_shape(rows.data_ptr(), assist.data_ptr(), a.data_ptr(),
                                       None if b is None else b.data_ptr(), gamma.data_ptr(),
                                       Bs, H, K, n_rows, out1.data_ptr(), out2.data_ptr(),
                                       policy, _stream()))
