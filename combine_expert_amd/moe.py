"""Thin ctypes binding of libmoe_expert.so (include/moe_expert.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the path runs in the library's kernels.
Output tensors may be passed in (nothing is allocated then) or are allocated
with torch.empty.  There is no fallback: importing this module raises if the
library is missing, and each call raises MoeError on a non-zero status.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

from . import build as _build

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_ELAUNCH = 0, 1, 2, 3
QUANT_NONE, QUANT_STATIC, QUANT_INT8_TOKEN, QUANT_INT8_TILE, QUANT_MXFP8 = 0, 1, 2, 3, 4
QUANT_MXFP8_GM = 5   # the mxfp8 codes, exponents group-major [ceil(H/512), rows, 16]
QUANT_STATIC_E4M3 = 6  # static, E4M3 codes of x * one coefficient (no expand_scales)
_MX = (QUANT_MXFP8, QUANT_MXFP8_GM)
SCALES_NONE, SCALES_ONE, SCALES_ROW, SCALES_EXPERT = 0, 1, 2, 3
SHARED_PAGE, SHARED_ADD = 0, 1
ERR_ID, ERR_TABLE, ERR_MASK1D, ERR_ROW, ERR_OFFSETS = 1, 2, 4, 8, 16

EXPORTS = ("moe_update_expert", "moe_dispatch", "moe_update_dispatch", "moe_combine_add_rmsnorm",
           "moe_expert_gemm", "moe_expert_swiglu", "moe_status_string")

if not os.path.exists(_build.LIB):
    raise ImportError(f"{_build.LIB} is not built: run `python -m combine_expert_amd.build`")

_lib = C.CDLL(_build.LIB)
_P, _I = C.c_void_p, C.c_int
_lib.moe_update_expert.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P]
_lib.moe_dispatch.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P,
                              _P, _P, _P, _P, _P]
_lib.moe_update_dispatch.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                     _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.moe_combine_add_rmsnorm.argtypes = [_P, _P, _P, _P, _P, _P, C.c_float, _I, _I, _I, _I,
                                         _P, _P, _P, _P, _P]
_lib.moe_expert_gemm.argtypes = [_P, _P, _P, _I, _I, _P, _P, _I, _I, _I, _P, _P, _P]
_lib.moe_expert_swiglu.argtypes = [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P]
for _f in (_lib.moe_update_expert, _lib.moe_dispatch, _lib.moe_update_dispatch,
           _lib.moe_combine_add_rmsnorm, _lib.moe_expert_gemm, _lib.moe_expert_swiglu):
    _f.restype = C.c_int
_lib.moe_status_string.argtypes = [_I]
_lib.moe_status_string.restype = C.c_char_p


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {moe_status_string(status)}")
        self.status = status


def library_path() -> str:
    return _build.LIB


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


_BYTE_TYPES = (torch.uint8, torch.int8, torch.bool)


def _arg(t: Optional[torch.Tensor], name: str, dtypes, numel: int, required: bool = True):
    """Checks a tensor argument before its pointer goes to the library: a CUDA tensor,
    contiguous, of one of `dtypes`, holding at least `numel` elements.  The kernels trust
    the sizes they are given, so an undersized or host tensor is refused here."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; at least {numel} are needed")


_I32, _F32, _BF16 = (torch.int32,), (torch.float32,), (torch.bfloat16,)


def _dispatch_args(x, expert_ids, Bs, H, K, E, quant_mode, tile, quant_scales, out,
                   dev_err, ids_name="expert_ids"):
    _arg(x, "x", _BF16, Bs * H)
    _arg(expert_ids, ids_name, _I32, Bs * K)
    if quant_scales is not None:
        _arg(quant_scales, "quant_scales", _F32, 1)
    N = Bs * K
    _arg(out["expand_x"], "expand_x", _BF16 if quant_mode == QUANT_NONE else _BYTE_TYPES[:2],
         N * H)
    ns = n_scale_entries(quant_mode, H, tile) if quant_mode != QUANT_INT8_TILE or tile > 0 else 0
    _arg(out.get("expand_scales"), "expand_scales",
         (torch.uint8,) if quant_mode in _MX else _F32, N * ns, required=ns > 0)
    _arg(out["expert_counts"], "expert_counts", _I32, E)
    _arg(out["expert_offsets"], "expert_offsets", _I32, E + 1)
    _arg(out["expand_src"], "expand_src", _I32, N)
    _arg(out["assist_dst"], "assist_dst", _I32, N)
    _arg(dev_err, "dev_err", _I32, 1, required=False)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def n_scale_entries(quant_mode: int, H: int, tile: int = 0) -> int:
    """Scale entries per expand_x row for a quantisation mode."""
    if quant_mode == QUANT_INT8_TOKEN:
        return 1
    if quant_mode in (QUANT_STATIC, QUANT_STATIC_E4M3):
        return 0
    if quant_mode == QUANT_INT8_TILE:
        return -(-H // tile)
    if quant_mode == QUANT_MXFP8:
        return H // 32
    if quant_mode == QUANT_MXFP8_GM:
        return -(-H // 512) * 16   # padded to whole groups of 16 exponents
    return 0


def moe_update_expert(expert_ids, table, n_instances: int, expert_scales=None, prune_thr=None,
                      token_mask=None, balanced_ids=None, balanced_mask=None, dev_err=None,
                      stream=None):
    Bs, K = expert_ids.shape
    n_logical, F = table.shape
    dev = expert_ids.device
    if balanced_ids is None:
        balanced_ids = torch.empty((Bs, K), dtype=torch.int32, device=dev)
    if balanced_mask is None:
        balanced_mask = torch.empty((Bs, K), dtype=torch.uint8, device=dev)
    _arg(expert_ids, "expert_ids", _I32, Bs * K)
    _arg(table, "table", _I32, n_logical * F)
    _arg(expert_scales, "expert_scales", _F32, Bs * K, required=False)
    _arg(prune_thr, "prune_thr", _F32, K, required=False)
    _arg(token_mask, "token_mask", _BYTE_TYPES, Bs, required=False)
    _arg(balanced_ids, "balanced_ids", _I32, Bs * K)
    _arg(balanced_mask, "balanced_mask", _BYTE_TYPES, Bs * K)
    _arg(dev_err, "dev_err", _I32, 1, required=False)
    rc = _lib.moe_update_expert(_ptr(expert_ids), _ptr(expert_scales), _ptr(table),
                                _ptr(prune_thr), _ptr(token_mask), Bs, K, n_logical, F,
                                n_instances, _ptr(balanced_ids), _ptr(balanced_mask),
                                _ptr(dev_err), _stream(stream))
    _check("moe_update_expert", rc)
    return balanced_ids, balanced_mask


def dispatch_buffers(Bs: int, H: int, K: int, E: int, quant_mode: int, tile: int = 0,
                     device="cuda"):
    """Allocate the dispatch outputs for a shape (capacity Bs*K rows)."""
    N = Bs * K
    dt = {QUANT_NONE: torch.bfloat16, QUANT_STATIC: torch.int8, QUANT_INT8_TOKEN: torch.int8,
          QUANT_INT8_TILE: torch.int8, QUANT_MXFP8: torch.uint8,
          QUANT_MXFP8_GM: torch.uint8, QUANT_STATIC_E4M3: torch.uint8}[quant_mode]
    ns = n_scale_entries(quant_mode, H, tile)
    sdt = torch.uint8 if quant_mode in _MX else torch.float32
    sshape = (ns // 16, N, 16) if quant_mode == QUANT_MXFP8_GM else (N, ns)
    return dict(
        expand_x=torch.empty((N, H), dtype=dt, device=device),
        expand_scales=torch.empty(sshape, dtype=sdt, device=device) if ns else None,
        expert_counts=torch.empty((E,), dtype=torch.int32, device=device),
        expert_offsets=torch.empty((E + 1,), dtype=torch.int32, device=device),
        expand_src=torch.empty((N,), dtype=torch.int32, device=device),
        assist_dst=torch.empty((N,), dtype=torch.int32, device=device),
    )


def scales_kind(quant_scales, H: int, E: int) -> int:
    """The shape name of a scales tensor: [1], [H] or [E, H]."""
    if quant_scales is None:
        return SCALES_NONE
    if quant_scales.dim() == 2 and tuple(quant_scales.shape) == (E, H):
        return SCALES_EXPERT
    if quant_scales.dim() == 1 and quant_scales.numel() == H:
        return SCALES_ROW
    if quant_scales.numel() == 1:
        return SCALES_ONE
    raise ValueError(f"scales of shape {tuple(quant_scales.shape)}: expected [1], [H] or [E, H]")


def moe_dispatch(x, expert_ids, n_ranks: int, local_experts: int, quant_mode: int = 0,
                 tile: int = 0, active_mask=None, quant_scales=None,
                 out: Optional[dict] = None, dev_err=None, stream=None,
                 token_mask=None) -> dict:
    Bs, H = x.shape
    K = expert_ids.shape[1]
    E = n_ranks * local_experts
    if out is None:
        out = dispatch_buffers(Bs, H, K, E, quant_mode, tile, x.device)
    _dispatch_args(x, expert_ids, Bs, H, K, E, quant_mode, tile, quant_scales, out, dev_err)
    _arg(active_mask, "active_mask", _BYTE_TYPES, Bs * K, required=False)
    _arg(token_mask, "token_mask", _BYTE_TYPES, Bs, required=False)
    rc = _lib.moe_dispatch(_ptr(x), _ptr(expert_ids), _ptr(active_mask), _ptr(token_mask), Bs,
                           H, K, n_ranks,
                           local_experts, quant_mode, tile, _ptr(quant_scales),
                           scales_kind(quant_scales, H, E), _ptr(out["expand_x"]),
                           _ptr(out.get("expand_scales")), _ptr(out["expert_counts"]),
                           _ptr(out["expert_offsets"]), _ptr(out["expand_src"]),
                           _ptr(out["assist_dst"]), _ptr(dev_err), _stream(stream))
    _check("moe_dispatch", rc)
    return out


def moe_update_dispatch(x, expert_ids, table, n_ranks: int, local_experts: int,
                        quant_mode: int = 0, tile: int = 0, expert_scales=None, prune_thr=None,
                        token_mask=None, quant_scales=None, balanced_ids=None,
                        balanced_mask=None, out: Optional[dict] = None, dev_err=None,
                        stream=None) -> dict:
    """Expert mapping + dispatch in one launch; returns the dispatch outputs
    plus 'balanced_ids' / 'balanced_mask' (allocated unless passed in)."""
    Bs, H = x.shape
    K = expert_ids.shape[1]
    n_logical, F = table.shape
    if out is None:
        out = dispatch_buffers(Bs, H, K, n_ranks * local_experts, quant_mode, tile, x.device)
    if balanced_ids is None:
        balanced_ids = torch.empty((Bs, K), dtype=torch.int32, device=x.device)
    if balanced_mask is None:
        balanced_mask = torch.empty((Bs, K), dtype=torch.uint8, device=x.device)
    _dispatch_args(x, expert_ids, Bs, H, K, n_ranks * local_experts, quant_mode, tile,
                   quant_scales, out, dev_err)
    _arg(table, "table", _I32, n_logical * F)
    _arg(expert_scales, "expert_scales", _F32, Bs * K, required=False)
    _arg(prune_thr, "prune_thr", _F32, K, required=False)
    _arg(token_mask, "token_mask", _BYTE_TYPES, Bs, required=False)
    _arg(balanced_ids, "balanced_ids", _I32, Bs * K)
    _arg(balanced_mask, "balanced_mask", _BYTE_TYPES, Bs * K)
    rc = _lib.moe_update_dispatch(_ptr(x), _ptr(expert_ids), _ptr(expert_scales), _ptr(table),
                                  _ptr(prune_thr), _ptr(token_mask), Bs, H, K, n_logical, F,
                                  n_ranks, local_experts, quant_mode, tile, _ptr(quant_scales),
                                  scales_kind(quant_scales, H, n_ranks * local_experts),
                                  _ptr(balanced_ids),
                                  _ptr(balanced_mask), _ptr(out["expand_x"]),
                                  _ptr(out.get("expand_scales")), _ptr(out["expert_counts"]),
                                  _ptr(out["expert_offsets"]), _ptr(out["expand_src"]),
                                  _ptr(out["assist_dst"]), _ptr(dev_err), _stream(stream))
    _check("moe_update_dispatch", rc)
    out["balanced_ids"] = balanced_ids
    out["balanced_mask"] = balanced_mask
    return out


def moe_combine_add_rmsnorm(expert_out, assist_dst, expert_scales, residual_x, gamma,
                            eps: float = 1e-6, shared_x=None, shared_mode: int = SHARED_PAGE,
                            y=None, x_out=None, rstd=None, want_x: bool = True,
                            want_rstd: bool = True, dev_err=None, stream=None):
    Bs, H = residual_x.shape
    K = expert_scales.shape[1]
    dev = residual_x.device
    if y is None:
        y = torch.empty((Bs, H), dtype=torch.bfloat16, device=dev)
    if x_out is None and want_x:
        x_out = torch.empty((Bs, H), dtype=torch.bfloat16, device=dev)
    if rstd is None and want_rstd:
        rstd = torch.empty((Bs,), dtype=torch.float32, device=dev)
    _arg(expert_out, "expert_out", _BF16, Bs * K * H)
    _arg(assist_dst, "assist_dst", _I32, Bs * K)
    _arg(expert_scales, "expert_scales", _F32, Bs * K)
    _arg(shared_x, "shared_x", _BF16, Bs * H, required=False)
    _arg(residual_x, "residual_x", _BF16, Bs * H)
    _arg(gamma, "gamma", _BF16, H)
    _arg(y, "y", _BF16, Bs * H)
    _arg(x_out, "x_out", _BF16, Bs * H, required=False)
    _arg(rstd, "rstd", _F32, Bs, required=False)
    _arg(dev_err, "dev_err", _I32, 1, required=False)
    rc = _lib.moe_combine_add_rmsnorm(_ptr(expert_out), _ptr(assist_dst), _ptr(expert_scales),
                                      _ptr(shared_x), _ptr(residual_x), _ptr(gamma), eps, Bs, H,
                                      K, shared_mode, _ptr(y), _ptr(x_out), _ptr(rstd),
                                      _ptr(dev_err), _stream(stream))
    _check("moe_combine_add_rmsnorm", rc)
    return y, x_out, rstd


def pack_mx_weight_scales(w_sc: torch.Tensor) -> torch.Tensor:
    """Weight preparation for mxfp8 moe_expert_gemm, done once per weight set: the E8M0
    weight exponents u8 [E, N, H/32] (row-major, one per 32 elements of a column) ->
    the group-major u8 [E, ceil(H/512), N, 16] the library reads (group q holds blocks
    16q .. 16q+15 of every column; a partial last group is zero-padded)."""
    E, N, nb = w_sc.shape
    groups = -(-nb // 16)
    padded = torch.zeros((E, N, groups * 16), dtype=torch.uint8, device=w_sc.device)
    padded[:, :, :nb] = w_sc
    return padded.view(E, N, groups, 16).permute(0, 2, 1, 3).contiguous()


def moe_expert_gemm(expand_x, expand_scales, expert_offsets, weights, weight_scales,
                    quant_mode: int = QUANT_MXFP8, y=None, dev_err=None, stream=None):
    """Grouped GEMM of the expert computation -> y bf16 [rows, N] (rows outside every
    instance's range are not written).  mxfp8: expand_x u8 [rows, H] (E4M3),
    expand_scales u8 [rows, H/32] (E8M0; QUANT_MXFP8_GM: the dispatch's group-major
    [ceil(H/512), rows, 16] for a dispatch of rows = Bs*K), weights u8 [E, N, H],
    weight_scales u8 [E, ceil(H/512), N, 16] (pack_mx_weight_scales of the [E, N, H/32]
    exponents).  int8 (QUANT_INT8_TOKEN / QUANT_INT8_TILE): expand_x int8 [rows, H],
    expand_scales f32 [rows] / [rows, H/128], weights int8 [E, N, H], weight_scales f32
    [E, N].  expert_offsets int32 [E+1]."""
    rows, H = expand_x.shape
    E = expert_offsets.numel() - 1
    N = weights.shape[1]
    if y is None:
        y = torch.empty((rows, N), dtype=torch.bfloat16, device=expand_x.device)
    mx = quant_mode in _MX
    _arg(expand_x, "expand_x", _BYTE_TYPES[:2], rows * H)
    _arg(expand_scales, "expand_scales", (torch.uint8,) if mx else _F32,
         rows * (n_scale_entries(quant_mode, H) if mx else
                 H // 128 if quant_mode == QUANT_INT8_TILE else 1))
    _arg(expert_offsets, "expert_offsets", _I32, E + 1)
    _arg(weights, "weights", _BYTE_TYPES[:2], E * N * H)
    _arg(weight_scales, "weight_scales", (torch.uint8,) if mx else _F32,
         E * (-(-H // 512)) * N * 16 if mx else E * N)
    _arg(y, "y", _BF16, rows * N)
    _arg(dev_err, "dev_err", _I32, 1, required=False)
    rc = _lib.moe_expert_gemm(_ptr(expand_x), _ptr(expand_scales), _ptr(expert_offsets), E, rows,
                              _ptr(weights), _ptr(weight_scales), N, H, quant_mode, _ptr(y),
                              _ptr(dev_err), _stream(stream))
    _check("moe_expert_gemm", rc)
    return y


def moe_expert_swiglu(y1, expert_offsets, quant_mode: int = QUANT_MXFP8, act_codes=None,
                      act_scales=None, act=None, want_act: bool = False, dev_err=None,
                      stream=None):
    """Activation between the expert FFN's projections: y1 bf16 [rows, 2I] (gate | up)
    -> (act_codes u8 E4M3 [rows, I], act_scales u8 E8M0 [rows, I/32] or group-major
    [ceil(I/512), rows, 16] for QUANT_MXFP8_GM, act bf16 [rows, I] or None).  Rows
    outside [offsets[0], offsets[E]) are not written."""
    rows, I2 = y1.shape
    I = I2 // 2
    E = expert_offsets.numel() - 1
    dev = y1.device
    ns = n_scale_entries(quant_mode, I) if quant_mode in _MX else 0
    if act_codes is None:
        act_codes = torch.empty((rows, I), dtype=torch.uint8, device=dev)
    if act_scales is None and ns:
        shape = (ns // 16, rows, 16) if quant_mode == QUANT_MXFP8_GM else (rows, ns)
        act_scales = torch.empty(shape, dtype=torch.uint8, device=dev)
    if act is None and want_act:
        act = torch.empty((rows, I), dtype=torch.bfloat16, device=dev)
    _arg(y1, "y1", _BF16, rows * 2 * I)
    _arg(expert_offsets, "expert_offsets", _I32, E + 1)
    _arg(act_codes, "act_codes", _BYTE_TYPES[:2], rows * I)
    _arg(act_scales, "act_scales", (torch.uint8,), rows * ns, required=ns > 0)
    _arg(act, "act", _BF16, rows * I, required=False)
    _arg(dev_err, "dev_err", _I32, 1, required=False)
    rc = _lib.moe_expert_swiglu(_ptr(y1), _ptr(expert_offsets), E, rows, I, quant_mode,
                                _ptr(act_codes), _ptr(act_scales), _ptr(act), _ptr(dev_err),
                                _stream(stream))
    _check("moe_expert_swiglu", rc)
    return act_codes, act_scales, act


def raw():
    """The ctypes library handle (for tests of the C ABI itself)."""
    return _lib
