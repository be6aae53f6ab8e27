"""Pins for the oracle's dispatch (row placement, per-token / per-tile / mxfp8
rows and scales) and combine + add + RMSNorm (CPU only).

Dispatch rows are checked against the already-pinned per-segment quantisers
applied independently to each token, and against bit copies for quantMode 0.
The combine ("aclnnMoeDistributeCombineAddRmsNorm" formula) is checked against
closed forms: identity experts (the dispatch-then-combine round trip gives
sum(scales) * x), constant rows (exact scalar arithmetic), torch's rms_norm for
the K=1 special case, the unit-RMS invariant, both shared-expert weightings,
and dropped (pruned) entries.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle
from combine_expert_amd import workloads as W


def bits(t):
    return oracle.bf16_bits(t)


def f32(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("mode,tile", [(0, 0), (2, 0), (3, 128), (3, 96), (4, 0)])
def test_dispatch_rows_match_per_token_quantiser(mode, tile):
    wl = W.make_small(seed=31 + mode, Bs=37, H=1120, K=5, n_ranks=3, local_experts=4,
                      quant_mode=mode, tile=tile or 128, prune=True)
    tile = tile if mode == 3 else 0
    ids = wl.logical_ids.numpy()
    rng = np.random.default_rng(9)
    mask = (rng.random(ids.shape) < 0.8).astype(np.uint8)
    xb = bits(wl.x)
    d = oracle.dispatch(xb, ids, mask, wl.n_ranks, wl.local_experts, mode, tile)
    H, K = wl.H, wl.K
    total = int(d["offsets"][-1])
    assert total == int(mask.sum())
    for r in range(total):
        f = int(d["src"][r])
        i = f // K
        row = d["expand_x"][r]
        if mode == 0:
            np.testing.assert_array_equal(row, xb[i])
        elif mode == 2:
            q, s = oracle.quant_int8(xb[i])
            np.testing.assert_array_equal(row, q)
            assert d["scales"][r, 0] == np.float32(s)
        elif mode == 3:
            nt = -(-H // tile)
            assert d["scales"].shape[1] == nt
            for t in range(nt):
                q, s = oracle.quant_int8(xb[i, t * tile:(t + 1) * tile])
                np.testing.assert_array_equal(row[t * tile:(t + 1) * tile], q)
                assert d["scales"][r, t] == np.float32(s)
        else:
            for b in range(H // 32):
                q, s = oracle.quant_mxfp8(xb[i, b * 32:(b + 1) * 32])
                np.testing.assert_array_equal(row[b * 32:(b + 1) * 32], q)
                assert d["scales"][r, b] == s
    # rows past the total are never written
    assert not d["expand_x"][total:].any()


def test_dispatch_instance_major_layout():
    # row blocks run [rank][local expert][token]: instance v*L + l owns the
    # rows offsets[v*L + l] .. offsets[v*L + l + 1]
    wl = W.make("c2")
    d = oracle.dispatch(bits(wl.x), wl.logical_ids.numpy(), None, wl.n_ranks,
                        wl.local_experts, 0, 0)
    ids = wl.logical_ids.numpy().reshape(-1)
    L = wl.local_experts
    last = (-1, -1)
    for r in range(int(d["offsets"][-1])):
        f = int(d["src"][r])
        v, l = divmod(int(ids[f]), L)
        assert (v, l) >= last
        last = (v, l)


# ---------------------------------------------------------------- combine

def _rand_bf16(rng, shape, s=1.0):
    return bits(W.bf16(rng.normal(0, s, size=shape)))


def test_combine_identity_expert_round_trip():
    # Identity experts: Eout row r = x[src[r] // K], so the weighted sum over the
    # token's K rows is (sum_k s_k) * x_i.  With residual 0 and no shared
    # expert, x = (sum s) * x_i and y = rms_norm(x) * gamma.
    wl = W.make_small(seed=5, Bs=20, H=1024, K=4, n_ranks=2, local_experts=4, quant_mode=0,
                      shared=False)
    xb = bits(wl.x)
    ids = wl.logical_ids.numpy()
    d = oracle.dispatch(xb, ids, None, wl.n_ranks, wl.local_experts, 0, 0)
    scales = wl.scales.numpy() * 1.7
    zero = np.zeros((wl.Bs, wl.H), np.uint16)
    gamma = np.full(wl.H, 0x3F80, np.uint16)  # 1.0
    y, xo, rstd = oracle.combine(d["expand_x"], d["assist"], scales, None, zero, gamma, 1e-6)
    ssum = scales.astype(np.float64).sum(axis=1)
    xexp = ssum[:, None] * f32(xb).astype(np.float64)
    np.testing.assert_array_equal(xo, oracle.bf16_round(xexp).reshape(xo.shape))
    ms = (xexp ** 2).mean(axis=1)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(ms + 1e-6), rtol=1e-6)
    # unit RMS before gamma (gamma = 1): within bf16 rounding
    yv = f32(y).astype(np.float64)
    rms = np.sqrt((yv ** 2).mean(axis=1))
    np.testing.assert_allclose(rms, 1.0, atol=2e-3)


def test_combine_k1_reduces_to_torch_rms_norm():
    rng = np.random.default_rng(8)
    Bs, H = 16, 2048
    eo = _rand_bf16(rng, (Bs, H), 3.0)
    gamma = _rand_bf16(rng, (H,), 1.0)
    assist = np.arange(Bs, dtype=np.int32)[:, None]
    ones = np.ones((Bs, 1), np.float32)
    zero = np.zeros((Bs, H), np.uint16)
    y, xo, rstd = oracle.combine(eo, assist, ones, None, zero, gamma, 1e-6)
    xt = torch.from_numpy(f32(eo).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (H,), eps=1e-6) * torch.from_numpy(
        f32(gamma).astype(np.float64))
    ref_bits = oracle.bf16_round(ref.numpy()).reshape(Bs, H)
    # both in fp64; only a result within 1e-15 of a bf16 tie could differ
    assert (y != ref_bits).mean() < 1e-4
    np.testing.assert_array_equal(xo, eo)


def test_combine_constant_rows_exact():
    # Every row constant along H: Eout rows a_k, shared b, residual c.  Then
    # x = sum_k s_k a_k + w b + c (w = sum s_k or 1) and
    # y = x / sqrt(x^2 + eps) * g exactly, evaluated here in rationals.
    H, K = 64, 3
    a = [1.5, -2.0, 0.25]
    s = np.array([[0.5, 0.25, 2.0]], np.float32)
    b, c, g, eps = 0.75, -1.0, 1.25, 1e-6
    eo = np.stack([np.full(H, np.float32(v)) for v in a])
    eo_b = bits(torch.from_numpy(eo).to(torch.bfloat16))
    sh = bits(torch.full((1, H), b).to(torch.bfloat16))
    res = bits(torch.full((1, H), c).to(torch.bfloat16))
    gm = bits(torch.full((H,), g).to(torch.bfloat16))
    assist = np.array([[0, 1, 2]], np.int32)
    for mode in (0, 1):
        y, xo, rstd = oracle.combine(eo_b, assist, s, sh, res, gm, eps, shared_mode=mode)
        ws = sum(Fraction(float(v)) for v in s[0])
        w = ws if mode == 0 else Fraction(1)
        x = sum(Fraction(float(s[0, k])) * Fraction(a[k]) for k in range(K)) + w * Fraction(b) \
            + Fraction(c)
        xe = float(x)
        ye = xe / math.sqrt(xe * xe + float(np.float32(eps))) * g
        assert np.all(xo == oracle.bf16_round(np.array([xe]))[0])
        assert np.all(y == oracle.bf16_round(np.array([ye]))[0])
    # the two weightings differ here (sum s = 2.75): the shared term is not 1*b
    # (y of a constant row is +-g either way, so compare the pre-norm x)
    _, x0, _ = oracle.combine(eo_b, assist, s, sh, res, gm, eps, shared_mode=0)
    _, x1, _ = oracle.combine(eo_b, assist, s, sh, res, gm, eps, shared_mode=1)
    assert not np.array_equal(x0, x1)


def test_combine_pruned_entries_drop_out():
    rng = np.random.default_rng(4)
    Bs, H, K = 6, 1024, 4
    eo = _rand_bf16(rng, (Bs * K, H))
    sh = _rand_bf16(rng, (Bs, H))
    res = _rand_bf16(rng, (Bs, H))
    gm = _rand_bf16(rng, (H,), 0.1)
    s = rng.random((Bs, K)).astype(np.float32)
    assist = np.arange(Bs * K, dtype=np.int32).reshape(Bs, K)
    pr = assist.copy()
    pr[:, 1] = -1
    pr[2, :] = -1  # token 2: nothing dispatched -> x = residual (weight sum 0)
    y, xo, _ = oracle.combine(eo, pr, s, sh, res, gm, 1e-6, shared_mode=0)
    keep = [0, 2, 3]
    s2 = s[:, keep].copy()
    a2 = assist[:, keep].copy()
    s2[2] = 0.0
    y2, xo2, _ = oracle.combine(eo, a2, s2, sh, res, gm, 1e-6, shared_mode=0)
    np.testing.assert_array_equal(xo, xo2)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(xo[2], res[2])


def test_combine_scale_invariance_of_y():
    # RMSNorm is invariant to a positive scaling of x (up to eps): doubling
    # every weight with zero residual and no shared expert leaves y unchanged.
    rng = np.random.default_rng(6)
    Bs, H, K = 8, 1024, 3
    eo = _rand_bf16(rng, (Bs * K, H))
    gm = _rand_bf16(rng, (H,), 1.0)
    s = rng.random((Bs, K)).astype(np.float32) + 0.1
    assist = np.arange(Bs * K, dtype=np.int32).reshape(Bs, K)
    zero = np.zeros((Bs, H), np.uint16)
    y1, _, r1 = oracle.combine(eo, assist, s, None, zero, gm, 0.0)
    y2, _, r2 = oracle.combine(eo, assist, s * 2, None, zero, gm, 0.0)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_allclose(r1, 2 * r2, rtol=1e-6)


def test_combine_eps_inside_the_root():
    # RMS(x) = sqrt(mean(x^2) + eps).  With x = 0.75 everywhere and
    # eps = 0.4375: mean(x^2) + eps = 0.5625 + 0.4375 = 1, so rstd = 1 exactly
    # and y = bf16(0.75 * gamma).
    H = 1024
    rng = np.random.default_rng(21)
    gm = _rand_bf16(rng, (H,), 1.0)
    eo = np.zeros((1, H), np.uint16)
    res = bits(torch.full((1, H), 0.75).to(torch.bfloat16))
    y, xo, rstd = oracle.combine(eo, np.array([[0]], np.int32), np.ones((1, 1), np.float32),
                                 None, res, gm, 0.4375)
    assert rstd[0] == 1.0
    np.testing.assert_array_equal(y[0], oracle.bf16_round(0.75 * f32(gm).astype(np.float64)))
