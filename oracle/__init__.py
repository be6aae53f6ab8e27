"""Python access to the plain-C CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library and
its Python binding never import it.

Arrays are numpy; bf16 data travels as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_ORACLE_LIB")  # a planted-mistake build (mutation tests)
        if path is None:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        L = C.CDLL(path)
        P = C.c_void_p
        i = C.c_int
        L.oracle_e4m3_encode.argtypes = [P, i, P]
        L.oracle_bf16_round.argtypes = [P, i, P]
        L.oracle_quant_int8.argtypes = [P, i, P, P]
        L.oracle_quant_mxfp8.argtypes = [P, i, P, P]
        L.oracle_update_expert.argtypes = [P, P, P, P, P, i, i, i, i, i, P, P, P]
        L.oracle_route.argtypes = [P, P, i, i, P, P, P, P, P]
        L.oracle_dispatch.argtypes = [P, P, P, i, i, i, i, i, i, i, P, P, P, P, P, P, P]
        L.oracle_dispatch_scaled.argtypes = [P, P, P, i, i, i, i, i, i, i, P, i, P, P, P, P, P,
                                             P, P]
        L.oracle_combine_add_rmsnorm.argtypes = [P, P, P, P, P, P, C.c_float, i, i, i, i,
                                                 P, P, P]
        L.oracle_e4m3_decode.argtypes = [P, i, P]
        L.oracle_set_threads.argtypes = [i]
        L.oracle_set_threads.restype = i
        L.oracle_expert_gemm_mx.argtypes = [P, P, P, i, i, P, P, i, i, P, P, P]
        L.oracle_expert_gemm_i8.argtypes = [P, P, i, P, i, i, P, P, i, i, P, P, P]
        L.oracle_swiglu_mx.argtypes = [P, P, i, i, i, P, P, P]
        for f in (L.oracle_update_expert, L.oracle_route, L.oracle_dispatch,
                  L.oracle_dispatch_scaled, L.oracle_combine_add_rmsnorm,
                  L.oracle_expert_gemm_mx, L.oracle_expert_gemm_i8, L.oracle_swiglu_mx):
            f.restype = C.c_int
        _lib = L
    return _lib


def set_threads(n: int) -> int:
    """Threads of the per-token loops (dispatch quantise-and-copy, combine);
    n <= 0 means every core.  Returns the count in effect."""
    return int(lib().oracle_set_threads(n))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def bf16_bits(t) -> np.ndarray:
    """bf16 torch tensor -> uint16 numpy bit patterns."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32).reshape(-1)
    out = np.empty(v.size, dtype=np.uint8)
    lib().oracle_e4m3_encode(_p(v), v.size, _p(out))
    return out


def bf16_round(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float64).reshape(-1)
    out = np.empty(v.size, dtype=np.uint16)
    lib().oracle_bf16_round(_p(v), v.size, _p(out))
    return out


def quant_int8(x_bits: np.ndarray):
    x = _c(x_bits, np.uint16).reshape(-1)
    q = np.empty(x.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    lib().oracle_quant_int8(_p(x), x.size, _p(q), _p(s))
    return q, float(s[0])


def quant_mxfp8(x_bits: np.ndarray):
    x = _c(x_bits, np.uint16).reshape(-1)
    q = np.empty(x.size, dtype=np.uint8)
    s = np.zeros(1, dtype=np.uint8)
    lib().oracle_quant_mxfp8(_p(x), x.size, _p(q), _p(s))
    return q, int(s[0])


def update_expert(ids, scores, table, thr, token_mask, n_instances: int):
    ids = _c(ids, np.int32)
    Bs, K = ids.shape
    table = _c(table, np.int32)
    n_logical, F = table.shape
    scores = _c(scores, np.float32)
    thr = _c(thr, np.float32)
    token_mask = _c(token_mask, np.uint8)
    out_ids = np.empty((Bs, K), dtype=np.int32)
    out_mask = np.empty((Bs, K), dtype=np.uint8)
    err = np.zeros(1, dtype=np.int32)
    rc = lib().oracle_update_expert(_p(ids), _p(scores), _p(table), _p(thr), _p(token_mask),
                                    Bs, K, n_logical, F, n_instances, _p(out_ids),
                                    _p(out_mask), _p(err))
    if rc:
        raise ValueError(f"oracle_update_expert rc={rc}")
    return out_ids, out_mask, int(err[0])


def route(ids, mask, E: int):
    ids = _c(ids, np.int32).reshape(-1)
    mask = _c(mask, np.uint8)
    mask = None if mask is None else mask.reshape(-1)
    N = ids.size
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    assist = np.empty(N, dtype=np.int32)
    src = np.empty(N, dtype=np.int32)
    err = np.zeros(1, dtype=np.int32)
    rc = lib().oracle_route(_p(ids), _p(mask), N, E, _p(counts), _p(offsets), _p(assist),
                            _p(src), _p(err))
    if rc:
        raise ValueError(f"oracle_route rc={rc}")
    return counts, offsets, assist, src, int(err[0])


def n_scales(quant_mode: int, H: int, tile: int) -> int:
    return {0: 0, 1: 0, 2: 1, 3: -(-H // tile) if tile > 0 else 0, 4: H // 32, 6: 0}[quant_mode]


SCALES_NONE, SCALES_ONE, SCALES_ROW, SCALES_EXPERT = 0, 1, 2, 3


def dispatch(x_bits, ids, mask, n_ranks: int, local_experts: int, quant_mode: int,
             tile: int = 0, qscales=None, qscales_kind: int = SCALES_NONE):
    """Returns dict(expand_x, scales, counts, offsets, src, assist, err).
    Rows past offsets[E] are zero (never written).  quant_mode 1 (static int8),
    6 (static E4M3, one coefficient) and the scales input (qscales_kind: 1 = [1],
    2 = [H], 3 = [E, H]) go through oracle_dispatch_scaled."""
    x = _c(x_bits, np.uint16)
    Bs, H = x.shape
    ids = _c(ids, np.int32)
    K = ids.shape[1]
    mask = _c(mask, np.uint8)
    N = Bs * K
    E = n_ranks * local_experts
    if quant_mode == 0:
        ex = np.zeros((N, H), dtype=np.uint16)
    elif quant_mode in (4, 6):
        ex = np.zeros((N, H), dtype=np.uint8)
    else:
        ex = np.zeros((N, H), dtype=np.int8)
    ns = n_scales(quant_mode, H, tile)
    if quant_mode == 4:
        sc = np.zeros((N, ns), dtype=np.uint8)
    elif quant_mode in (2, 3):
        sc = np.zeros((N, ns), dtype=np.float32)
    else:
        sc = None
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    src = np.empty(N, dtype=np.int32)
    assist = np.empty(N, dtype=np.int32)
    err = np.zeros(1, dtype=np.int32)
    if quant_mode in (1, 6) or qscales_kind != SCALES_NONE:
        qs = _c(qscales, np.float32)
        rc = lib().oracle_dispatch_scaled(_p(x), _p(ids), _p(mask), Bs, H, K, n_ranks,
                                          local_experts, quant_mode, tile, _p(qs), qscales_kind,
                                          _p(ex), _p(sc), _p(counts), _p(offsets), _p(src),
                                          _p(assist), _p(err))
    else:
        rc = lib().oracle_dispatch(_p(x), _p(ids), _p(mask), Bs, H, K, n_ranks, local_experts,
                                   quant_mode, tile, _p(ex), _p(sc), _p(counts), _p(offsets),
                                   _p(src), _p(assist), _p(err))
    if rc:
        raise ValueError(f"oracle_dispatch rc={rc}")
    return dict(expand_x=ex, scales=sc, counts=counts, offsets=offsets, src=src,
                assist=assist, err=int(err[0]))


def combine(expert_out_bits, assist, scales, shared_bits, residual_bits, gamma_bits,
            eps: float, shared_mode: int = 0):
    """Returns (y_bits, x_out_bits, rstd) with y/x_out as uint16 bf16 patterns."""
    eo = _c(expert_out_bits, np.uint16)
    res = _c(residual_bits, np.uint16)
    Bs, H = res.shape
    assist = _c(assist, np.int32).reshape(Bs, -1)
    K = assist.shape[1]
    scales = _c(scales, np.float32).reshape(Bs, K)
    sh = _c(shared_bits, np.uint16)
    gamma = _c(gamma_bits, np.uint16)
    y = np.empty((Bs, H), dtype=np.uint16)
    xo = np.empty((Bs, H), dtype=np.uint16)
    rstd = np.empty(Bs, dtype=np.float32)
    rc = lib().oracle_combine_add_rmsnorm(_p(eo), _p(assist), _p(scales), _p(sh), _p(res),
                                          _p(gamma), eps, Bs, H, K, shared_mode, _p(y),
                                          _p(xo), _p(rstd))
    if rc:
        raise ValueError(f"oracle_combine rc={rc}")
    return y, xo, rstd


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    c = _c(codes, np.uint8).reshape(-1)
    out = np.empty(c.size, dtype=np.float64)
    lib().oracle_e4m3_decode(_p(c), c.size, _p(out))
    return out


def expert_gemm_mx(a, a_sc, offsets, w, w_sc, y_init=None):
    """Expert computation on mxfp8 operands.  a u8 [rows, Kd], a_sc u8
    [rows, Kd/32], offsets int32 [E+1], w u8 [E, N, Kd], w_sc u8 [E, N, Kd/32].
    Returns (y_bits uint16 [rows, N], y64, abs64); rows outside the experts'
    ranges keep y_init (default zeros) and 0 in y64 / abs64."""
    a = _c(a, np.uint8)
    rows, Kd = a.shape
    a_sc = _c(a_sc, np.uint8)
    offsets = _c(offsets, np.int32)
    E = offsets.size - 1
    w = _c(w, np.uint8)
    N = w.shape[1]
    assert w.shape == (E, N, Kd) and a_sc.shape == (rows, Kd // 32)
    w_sc = _c(w_sc, np.uint8)
    assert w_sc.shape == (E, N, Kd // 32)
    y = np.zeros((rows, N), dtype=np.uint16) if y_init is None else _c(y_init, np.uint16).copy()
    y64 = np.zeros((rows, N), dtype=np.float64)
    abs64 = np.zeros((rows, N), dtype=np.float64)
    rc = lib().oracle_expert_gemm_mx(_p(a), _p(a_sc), _p(offsets), E, rows, _p(w), _p(w_sc), N,
                                     Kd, _p(y), _p(y64), _p(abs64))
    if rc:
        raise ValueError(f"oracle_expert_gemm_mx rc={rc}")
    return y, y64, abs64


def swiglu_mx(y1_bits, offsets, init=None):
    """Activation of the expert FFN between its projections: y1 bf16 bits [rows, 2I]
    (gate | up), offsets int32 [E+1].  Returns (act_bits uint16 [rows, I], codes u8
    [rows, I], scales u8 [rows, I/32]); rows outside [offsets[0], offsets[E]) keep
    `init` (a (act, codes, scales) triple) or zeros."""
    y1 = _c(y1_bits, np.uint16)
    rows, I2 = y1.shape
    I = I2 // 2
    offsets = _c(offsets, np.int32)
    E = offsets.size - 1
    if init is None:
        act = np.zeros((rows, I), dtype=np.uint16)
        codes = np.zeros((rows, I), dtype=np.uint8)
        sc = np.zeros((rows, I // 32), dtype=np.uint8)
    else:
        act, codes, sc = (_c(t, d).copy() for t, d in zip(init, (np.uint16, np.uint8, np.uint8)))
    rc = lib().oracle_swiglu_mx(_p(y1), _p(offsets), E, rows, I, _p(act), _p(codes), _p(sc))
    if rc:
        raise ValueError(f"oracle_swiglu_mx rc={rc}")
    return act, codes, sc


def expert_gemm_i8(a, a_sc, offsets, w, w_sc, y_init=None):
    """Expert computation on int8 operands.  a int8 [rows, Kd]; a_sc f32 [rows] (one scale
    per row) or [rows, Kd/128] (per tile of 128); offsets int32 [E+1]; w int8 [E, N, Kd];
    w_sc f32 [E, N].  Returns (y_bits, y64, abs64) as expert_gemm_mx."""
    a = _c(a, np.int8)
    rows, Kd = a.shape
    a_sc = _c(a_sc, np.float32)
    n_tiles = 1 if a_sc.ndim == 1 else a_sc.shape[1]
    assert a_sc.shape[0] == rows
    offsets = _c(offsets, np.int32)
    E = offsets.size - 1
    w = _c(w, np.int8)
    N = w.shape[1]
    assert w.shape == (E, N, Kd)
    w_sc = _c(w_sc, np.float32)
    assert w_sc.shape == (E, N)
    y = np.zeros((rows, N), dtype=np.uint16) if y_init is None else _c(y_init, np.uint16).copy()
    y64 = np.zeros((rows, N), dtype=np.float64)
    abs64 = np.zeros((rows, N), dtype=np.float64)
    rc = lib().oracle_expert_gemm_i8(_p(a), _p(a_sc), n_tiles, _p(offsets), E, rows, _p(w),
                                     _p(w_sc), N, Kd, _p(y), _p(y64), _p(abs64))
    if rc:
        raise ValueError(f"oracle_expert_gemm_i8 rc={rc}")
    return y, y64, abs64
