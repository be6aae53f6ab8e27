"""Pins for the oracle's expert computation on mxfp8 operands (CPU only).

The oracle multiplies the rows of each instance by that instance's weight
matrix after dequantising both operands per block of 32 along H (the mxfp8
layout of expandX / dynamicScales in "aclnnMoeDistributeDispatchV2", case 5;
the expert computation itself sits between dispatch and combine in the
calling sequence of "aclnnMoeUpdateExpert").  Each check below is something
other than the oracle itself:
  - the E4M3 decoder against torch's float8_e4m3fn conversion, and encode/decode round trips;
  - the grouped product against numpy float64 matmuls per instance on operands decoded by torch;
  - closed forms: one-hot weights pick single dequantised activations, an E8M0 step doubles
    exactly one block's contribution, and an activation scale step doubles a whole row;
  - structure: empty instances, rows past the last instance are left untouched, and
    malformed offsets are rejected.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_expert_amd import workloads as W


def torch_e4m3(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def dequant(codes: np.ndarray, sc: np.ndarray) -> np.ndarray:
    """codes [..., Kd] E4M3, sc [..., Kd/32] E8M0 -> float64 values (torch decoder)."""
    return torch_e4m3(codes) * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=-1)


def numpy_gemm(g: W.GemmCase) -> np.ndarray:
    out = np.zeros((g.rows, g.N))
    A = dequant(g.a, g.a_sc)
    for e in range(g.E):
        lo, hi = g.offsets[e], g.offsets[e + 1]
        out[lo:hi] = A[lo:hi] @ dequant(g.w[e], g.w_sc[e]).T
    return out


# ---------------------------------------------------------------- E4M3 decode

def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = torch_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got).sum() == 2  # 0x7F and 0xFF
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_e4m3_encode_decode_round_trip():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(oracle.e4m3_encode(vals.astype(np.float32)), codes)
    assert oracle.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0
    assert oracle.e4m3_decode(np.array([0x01], np.uint8))[0] == 2.0 ** -9


# ---------------------------------------------------------------- grouped product

@pytest.mark.parametrize("counts,N,Kd,tail", [
    ([0, 17, 21], 24, 96, 2),
    ([5], 7, 32, 0),
    ([3, 0, 0, 9, 1], 16, 160, 3),
])
def test_gemm_matches_numpy(counts, N, Kd, tail):
    g = W.make_gemm_case(11 + N, counts, N, Kd, tail=tail)
    y, y64, abs64 = oracle.expert_gemm_mx(g.a, g.a_sc, g.offsets, g.w, g.w_sc)
    ref = numpy_gemm(g)
    last = int(g.offsets[-1])
    assert np.all(np.abs(y64 - ref) <= 1e-12 * abs64 + 1e-300)
    assert np.array_equal(y[:last], oracle.bf16_round(ref[:last]).reshape(last, N))
    assert np.all(y[last:] == 0) and np.all(y64[last:] == 0)
    absref = np.zeros_like(ref)
    A = np.abs(dequant(g.a, g.a_sc))
    for e in range(g.E):
        lo, hi = g.offsets[e], g.offsets[e + 1]
        absref[lo:hi] = A[lo:hi] @ np.abs(dequant(g.w[e], g.w_sc[e])).T
    assert np.allclose(abs64, absref, rtol=1e-12, atol=0)


def test_gemm_one_hot_weights_select_activations():
    """W[e][n][k] = 1.0 at k = perm_e[n], else +0, unit scales: y[r][n] = A(r, perm_e[n])."""
    rng = np.random.default_rng(5)
    counts, N, Kd = [4, 6, 3], 40, 128
    g = W.make_gemm_case(6, counts, N, Kd, tail=1)
    perms = [rng.permutation(Kd)[:N] for _ in range(g.E)]
    w = np.zeros((g.E, N, Kd), dtype=np.uint8)
    for e in range(g.E):
        w[e, np.arange(N), perms[e]] = 0x38
    w_sc = np.full((g.E, N, Kd // 32), 127, dtype=np.uint8)
    y, y64, _ = oracle.expert_gemm_mx(g.a, g.a_sc, g.offsets, w, w_sc)
    A = dequant(g.a, g.a_sc)
    for e in range(g.E):
        for r in range(g.offsets[e], g.offsets[e + 1]):
            assert np.array_equal(y64[r], A[r, perms[e]])
            # an E4M3 value times a power of two has 4 significant bits: exact in bf16
            assert np.array_equal(y[r], oracle.bf16_round(A[r, perms[e]]))


def test_gemm_scale_steps():
    """Raising one weight block's E8M0 code by 1 adds exactly that block's partial sum to one
    output column; raising one row's activation codes by 1 doubles that row."""
    counts, N, Kd = [3, 4], 8, 128
    g = W.make_gemm_case(9, counts, N, Kd)
    _, base, _ = oracle.expert_gemm_mx(g.a, g.a_sc, g.offsets, g.w, g.w_sc)
    e, n, b = 1, 5, 2
    w_sc = g.w_sc.copy()
    w_sc[e, n, b] += 1
    _, step, _ = oracle.expert_gemm_mx(g.a, g.a_sc, g.offsets, g.w, w_sc)
    A = dequant(g.a, g.a_sc)
    Wd = dequant(g.w[e], g.w_sc[e])
    lo, hi = g.offsets[e], g.offsets[e + 1]
    part = A[lo:hi, 32 * b:32 * b + 32] @ Wd[n, 32 * b:32 * b + 32]
    delta = step - base
    assert np.allclose(delta[lo:hi, n], part, rtol=1e-12, atol=1e-300)
    mask = np.ones_like(delta, dtype=bool)
    mask[lo:hi, n] = False
    assert np.all(delta[mask] == 0)
    a_sc = g.a_sc.copy()
    a_sc[2] += 1
    _, dbl, _ = oracle.expert_gemm_mx(g.a, a_sc, g.offsets, g.w, g.w_sc)
    assert np.array_equal(dbl[2], 2 * base[2])
    assert np.array_equal(np.delete(dbl, 2, 0), np.delete(base, 2, 0))


def test_gemm_empty_untouched_and_bad_offsets():
    g = W.make_gemm_case(12, [0, 0], 16, 64, tail=5)
    init = np.full((g.rows, 16), 0x1234, dtype=np.uint16)
    y, _, _ = oracle.expert_gemm_mx(g.a, g.a_sc, g.offsets, g.w, g.w_sc, y_init=init)
    assert np.array_equal(y, init)
    g = W.make_gemm_case(13, [2, 3], 16, 64, tail=2)
    init = np.full((g.rows, 16), 0x1234, dtype=np.uint16)
    y, _, _ = oracle.expert_gemm_mx(g.a, g.a_sc, g.offsets, g.w, g.w_sc, y_init=init)
    assert np.all(y[5:] == 0x1234) and not np.any(np.all(y[:5] == 0x1234, axis=1))
    for bad in ([0, 3, 2], [-1, 2, 5], [0, 2, 8]):
        with pytest.raises(ValueError):
            oracle.expert_gemm_mx(g.a, g.a_sc, np.array(bad, np.int32), g.w, g.w_sc)


# ---------------------------------------------------------------- int8 operands

def numpy_gemm_i8(g) -> np.ndarray:
    """Per tile: exact int64 products summed, scaled in float64 (numpy einsum)."""
    out = np.zeros((g.rows, g.N))
    n_t = 1 if g.a_sc.ndim == 1 else g.a_sc.shape[1]
    tl = g.Kd // n_t
    a_sc = g.a_sc.reshape(g.rows, n_t).astype(np.float64)
    for e in range(g.E):
        lo, hi = g.offsets[e], g.offsets[e + 1]
        for t in range(n_t):
            isum = np.einsum("rk,nk->rn", g.a[lo:hi, t * tl:(t + 1) * tl].astype(np.int64),
                             g.w[e, :, t * tl:(t + 1) * tl].astype(np.int64))
            out[lo:hi] += a_sc[lo:hi, t:t + 1] * g.w_sc[e].astype(np.float64)[None, :] * isum
    return out


@pytest.mark.parametrize("per_tile", [False, True])
@pytest.mark.parametrize("counts,N,Kd,tail", [([0, 9, 21], 24, 256, 2), ([5], 8, 128, 0),
                                                ([3, 0, 7, 1], 16, 384, 3)])
def test_gemm_i8_matches_numpy(per_tile, counts, N, Kd, tail):
    g = W.make_gemm_case_i8(21 + N + Kd, counts, N, Kd, per_tile, tail=tail)
    y, y64, abs64 = oracle.expert_gemm_i8(g.a, g.a_sc, g.offsets, g.w, g.w_sc)
    ref = numpy_gemm_i8(g)
    last = int(g.offsets[-1])
    assert np.all(np.abs(y64 - ref) <= 1e-13 * abs64 + 1e-300)
    assert np.array_equal(y[:last], oracle.bf16_round(ref[:last]).reshape(last, N))
    assert np.all(y[last:] == 0)
    n_t = g.a_sc.reshape(g.rows, -1).shape[1]
    A = np.abs(g.a.astype(np.float64)) * np.repeat(g.a_sc.reshape(g.rows, n_t), Kd // n_t, axis=1)
    for e in range(g.E):
        lo, hi = g.offsets[e], g.offsets[e + 1]
        Wd = np.abs(g.w[e].astype(np.float64)) * g.w_sc[e].astype(np.float64)[:, None]
        assert np.allclose(abs64[lo:hi], A[lo:hi] @ Wd.T, rtol=1e-12, atol=0)


def test_gemm_i8_one_hot_and_scale_steps():
    """One-hot weights with unit scales return single dequantised activations; doubling one
    weight scale doubles one column; doubling one tile's scale adds exactly that tile's term."""
    rng = np.random.default_rng(8)
    g = W.make_gemm_case_i8(31, [4, 5], 32, 256, True)
    perms = [rng.permutation(g.Kd)[:g.N] for _ in range(g.E)]
    w = np.zeros_like(g.w)
    for e in range(g.E):
        w[e, np.arange(g.N), perms[e]] = 1
    w_sc = np.ones_like(g.w_sc)
    _, y64, _ = oracle.expert_gemm_i8(g.a, g.a_sc, g.offsets, w, w_sc)
    for e in range(g.E):
        for r in range(g.offsets[e], g.offsets[e + 1]):
            k = perms[e]
            assert np.array_equal(y64[r], g.a[r, k].astype(np.float64) *
                                  g.a_sc[r, k // 128].astype(np.float64))
    _, base, _ = oracle.expert_gemm_i8(g.a, g.a_sc, g.offsets, g.w, g.w_sc)
    w_sc2 = g.w_sc.copy()
    w_sc2[1, 7] *= 2
    _, dbl, _ = oracle.expert_gemm_i8(g.a, g.a_sc, g.offsets, g.w, w_sc2)
    lo, hi = g.offsets[1], g.offsets[2]
    assert np.array_equal(dbl[lo:hi, 7], 2 * base[lo:hi, 7])
    mask = np.ones_like(base, dtype=bool)
    mask[lo:hi, 7] = False
    assert np.array_equal(dbl[mask], base[mask])
    a_sc2 = g.a_sc.copy()
    a_sc2[2, 1] *= 2
    _, st, _ = oracle.expert_gemm_i8(g.a, a_sc2, g.offsets, g.w, g.w_sc)
    tile = (g.a[2, 128:256].astype(np.int64) @ g.w[0, :, 128:256].astype(np.int64).T)
    term = g.a_sc[2, 1].astype(np.float64) * g.w_sc[0].astype(np.float64) * tile
    assert np.allclose(st[2] - base[2], term, rtol=1e-12, atol=1e-300)


def test_gemm_i8_one_tile_equals_per_token():
    """Per-tile scales that are equal along a row give the per-token result."""
    g = W.make_gemm_case_i8(41, [6, 2], 16, 384, False)
    _, tok, _ = oracle.expert_gemm_i8(g.a, g.a_sc, g.offsets, g.w, g.w_sc)
    per_tile = np.repeat(g.a_sc[:, None], 3, axis=1)
    _, til, abs64 = oracle.expert_gemm_i8(g.a, per_tile, g.offsets, g.w, g.w_sc)
    assert np.all(np.abs(til - tok) <= 1e-15 * abs64)


def test_gemm_i8_rejects_bad_tiles():
    g = W.make_gemm_case_i8(51, [3], 8, 256, True)
    with pytest.raises(ValueError):
        oracle.expert_gemm_i8(g.a, np.ones((g.rows, 3), np.float32), g.offsets, g.w, g.w_sc)
