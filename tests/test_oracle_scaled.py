"""Pins of the oracle's scales input and static quantisation (CPU only).

Dispatch page ("aclnnMoeDistributeDispatchV2"), 计算公式 case 2 (quantMode 1,
static: xFp32 = CastToFp32(X) * scales, quantOut = Cast(xFp32, int8)) and the
scales factor of cases 3-4; quantMode constraints for the shapes of the
scales input (one coefficient, one row shared by all experts, one row per
expert).

Pinned against:
- brute force: the static code of each element is the integer in
  [-128, 127] nearest to the fp32 product (numpy float32 multiply), ties to
  even, found by searching all 256 codes;
- hand-worked ties, saturation and NaN;
- special cases that reduce to the pinned unscaled quantisers: unit scales,
  and power-of-two scales (codes unchanged, scale output multiplied by the
  power exactly);
- consistency: one row for all experts equals that row repeated per expert;
  per-expert rows follow the instance each copy is sent to.
"""
import numpy as np
import pytest
import torch

import oracle

CODES = np.arange(-128, 128, dtype=np.float64)


def bf16_bits_of(a):
    return oracle.bf16_bits(torch.from_numpy(np.asarray(a, dtype=np.float32)).bfloat16())


def bf16_vals(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def brute_static(v):
    """Nearest of the 256 int8 codes to each fp32 value, ties to the even code."""
    v = np.asarray(v, dtype=np.float64).ravel()
    dist = np.abs(v[:, None] - CODES[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    even = (CODES.astype(np.int64) % 2 == 0)[None, :]
    pick = np.where(cand & even, 1, 0) + np.where(cand, 1, 0)  # prefer even among ties
    return CODES[pick.argmax(axis=1)].astype(np.int8)


def case(seed, Bs=13, H=96, K=3, R=2, L=3, scale=1.0):
    rng = np.random.default_rng(seed)
    E = R * L
    x = bf16_bits_of(rng.normal(0.0, scale, size=(Bs, H)))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(Bs)]).astype(np.int32)
    return rng, x, ids, E


def scale_of(kind, qs, e, H):
    if kind == 1:
        return np.full(H, qs[0], dtype=np.float32)
    if kind == 2:
        return qs.astype(np.float32)
    return qs[e].astype(np.float32)


@pytest.mark.parametrize("kind", [1, 2, 3])
def test_static_codes_brute_force(kind):
    rng, x, ids, E = case(71 + kind, scale=40.0)
    Bs, H = x.shape
    K = ids.shape[1]
    qs = {1: rng.uniform(0.5, 4.0, size=1), 2: rng.uniform(0.2, 4.0, size=H),
          3: rng.uniform(0.2, 4.0, size=(E, H))}[kind].astype(np.float32)
    o = oracle.dispatch(x, ids, None, 2, 3, 1, 0, qs, kind)
    assert o["scales"] is None
    xv = bf16_vals(x)
    for f in range(Bs * K):
        i, e, r = f // K, ids.flat[f], o["assist"][f]
        v = xv[i] * scale_of(kind, qs, e, H)  # numpy float32 product (IEEE)
        np.testing.assert_array_equal(o["expand_x"][r], brute_static(v))


def test_static_hand_worked():
    vals = [0.5, 1.5, 2.5, -0.5, -2.5, 126.5, 127.5, -127.5, 129.0, -300.0, 3.25, -3.75]
    want = [0, 2, 2, 0, -2, 126, 127, -128, 127, -128, 3, -4]
    x = bf16_bits_of([vals + [0.0] * (32 - len(vals))])
    assert np.array_equal(bf16_vals(x)[0, :len(vals)], np.float32(vals))  # exact in bf16
    o = oracle.dispatch(x, np.array([[0]], np.int32), None, 1, 1, 1, 0,
                        np.array([1.0], np.float32), 1)
    assert o["expand_x"][0, :len(vals)].tolist() == want
    nan = np.full((1, 32), 0x7FC0, dtype=np.uint16)
    o = oracle.dispatch(nan, np.array([[0]], np.int32), None, 1, 1, 1, 0,
                        np.array([1.0], np.float32), 1)
    assert not o["expand_x"][0].any()


def test_static_integers_pass_through():
    # integer-valued inputs in [-128, 127] with scale 1 are their own codes
    x = bf16_bits_of(np.arange(-128, 128, dtype=np.float32).reshape(2, 128))
    ids = np.array([[0], [1]], np.int32)
    o = oracle.dispatch(x, ids, None, 1, 2, 1, 0, np.ones(128, np.float32), 2)
    got = np.concatenate([o["expand_x"][o["assist"][0]], o["expand_x"][o["assist"][1]]])
    np.testing.assert_array_equal(got, np.arange(-128, 128).astype(np.int8))


@pytest.mark.parametrize("mode,tile", [(2, 0), (3, 32), (3, 40)])
@pytest.mark.parametrize("kind", [1, 2, 3])
def test_unit_scales_reduce_to_unscaled(mode, tile, kind):
    rng, x, ids, E = case(90 + kind + mode)
    H = x.shape[1]
    qs = {1: np.ones(1), 2: np.ones(H), 3: np.ones((E, H))}[kind].astype(np.float32)
    a = oracle.dispatch(x, ids, None, 2, 3, mode, tile, qs, kind)
    b = oracle.dispatch(x, ids, None, 2, 3, mode, tile)
    for key in ("expand_x", "scales", "assist", "offsets", "src"):
        np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("mode,tile", [(2, 0), (3, 32)])
def test_power_of_two_expert_rows(mode, tile):
    """Row e = 2^p(e): codes equal the unscaled ones, the scale sent is the
    unscaled scale times 2^p(e) exactly."""
    rng, x, ids, E = case(120 + mode)
    H = x.shape[1]
    K = ids.shape[1]
    p = np.array([(e % 5) - 2 for e in range(E)])
    qs = np.repeat(np.ldexp(1.0, p)[:, None], H, axis=1).astype(np.float32)
    a = oracle.dispatch(x, ids, None, 2, 3, mode, tile, qs, 3)
    b = oracle.dispatch(x, ids, None, 2, 3, mode, tile)
    np.testing.assert_array_equal(a["expand_x"], b["expand_x"])
    for f in range(ids.size):
        r = a["assist"][f]
        np.testing.assert_array_equal(a["scales"][r],
                                      np.ldexp(b["scales"][r], p[ids.flat[f]]).astype(np.float32))


@pytest.mark.parametrize("mode,tile", [(1, 0), (2, 0), (3, 32)])
def test_row_equals_repeated_expert_rows(mode, tile):
    rng, x, ids, E = case(140 + mode)
    H = x.shape[1]
    row = rng.uniform(0.25, 3.0, size=H).astype(np.float32)
    a = oracle.dispatch(x, ids, None, 2, 3, mode, tile, row, 2)
    b = oracle.dispatch(x, ids, None, 2, 3, mode, tile, np.tile(row, (E, 1)), 3)
    np.testing.assert_array_equal(a["expand_x"], b["expand_x"])
    if mode != 1:
        np.testing.assert_array_equal(a["scales"], b["scales"])


def test_dynamic_smoothing_brute_force():
    """Per-token dynamic int8 on xFp32 = x * row(e): max over the copy, IEEE
    float32 127 / max, codes by searching the codes in [-127, 127]."""
    rng, x, ids, E = case(160)
    Bs, H = x.shape
    K = ids.shape[1]
    qs = rng.uniform(0.1, 5.0, size=(E, H)).astype(np.float32)
    o = oracle.dispatch(x, ids, None, 2, 3, 2, 0, qs, 3)
    xv = bf16_vals(x)
    for f in range(Bs * K):
        i, e, r = f // K, ids.flat[f], o["assist"][f]
        v = xv[i] * qs[e]
        d = np.float32(127.0) / np.abs(v).max()
        codes = brute_static(v * d)
        assert np.abs(codes.astype(int)).max() <= 127
        np.testing.assert_array_equal(o["expand_x"][r], codes)
        assert o["scales"][r, 0] == np.float32(1.0) / d


def test_rejects_static_without_scales():
    rng, x, ids, E = case(170)
    with pytest.raises(ValueError):
        oracle.dispatch(x, ids, None, 2, 3, 1, 0)


# ---- static quantisation, second output type (read as OCP E4M3), one coefficient

def e4m3_table():
    """Value of each of the 256 E4M3 codes from the format definition (sign bit,
    4 exponent bits with bias 7, 3 mantissa bits, exponent 0 subnormal with step
    2^-9, S.1111.111 NaN); NaN codes as nan."""
    c = np.arange(256)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c >= 128, -mag, mag)


E4M3 = e4m3_table()


def brute_e4m3(v):
    """Nearest finite E4M3 code to each value after saturation to +-448, ties to the
    even code (even mantissa); zeros and values that round to zero keep their sign;
    NaN -> 0x7F."""
    v = np.asarray(v, dtype=np.float64).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    pos = np.arange(128)[~np.isnan(E4M3[:128])]
    for j, x in enumerate(v):
        if x != x:
            out[j] = 0x7F
            continue
        a = min(abs(x), 448.0)
        dist = np.abs(E4M3[pos] - a)
        cand = pos[dist == dist.min()]
        c = cand[0] if cand.size == 1 else cand[cand % 2 == 0][0]
        out[j] = c | (0x80 if np.signbit(x) else 0)
    return out


def test_e4m3_table_against_torch():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(np.isnan(codes), np.isnan(E4M3))
    ok = ~np.isnan(E4M3)
    np.testing.assert_array_equal(codes[ok].astype(np.float64), E4M3[ok])


def test_static_e4m3_brute_force():
    rng, x, ids, E = case(181, scale=60.0)
    Bs, H = x.shape
    K = ids.shape[1]
    qs = np.array([rng.uniform(0.5, 9.0)], np.float32)
    o = oracle.dispatch(x, ids, None, 2, 3, 6, 0, qs, 1)
    assert o["scales"] is None and o["expand_x"].dtype == np.uint8
    xv = bf16_vals(x)
    for f in range(Bs * K):
        i, r = f // K, o["assist"][f]
        v = xv[i] * qs[0]  # numpy float32 product (IEEE)
        np.testing.assert_array_equal(o["expand_x"][r], brute_e4m3(v))


def test_static_e4m3_against_torch():
    """Small, tiny and large products: the clamped fp32 product through torch's
    float8_e4m3fn conversion (round to nearest even)."""
    rng = np.random.default_rng(182)
    H = 512
    mag = np.exp2(rng.uniform(-14, 11, size=(6, H)))
    x = bf16_bits_of(mag * rng.choice([-1.0, 1.0], size=mag.shape))
    ids = np.arange(6, dtype=np.int32).reshape(6, 1) % 4
    for s in (1.0, 0.3, 7.0):
        qs = np.array([s], np.float32)
        o = oracle.dispatch(x, ids, None, 2, 2, 6, 0, qs, 1)
        v = np.clip(bf16_vals(x) * np.float32(s), -448.0, 448.0).astype(np.float32)
        want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = np.stack([o["expand_x"][o["assist"][f]] for f in range(6)])
        np.testing.assert_array_equal(got, want)


def test_static_e4m3_hand_worked():
    vals = [1.0, 1.0625, 1.1875, 3.0, 300.0, -300.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10,
            -np.inf, np.inf, 0.0, -0.0, 448.0, 464.0, 480.0, -2.0 ** -11]
    want1 = [0x38, 0x38, 0x3A, 0x44, 0x79, 0xF9, 0x01, 0x00, 0x02, 0xFE, 0x7E, 0x00, 0x80,
             0x7E, 0x7E, 0x7E, 0x80]
    # times 2: 600 and 928 saturate; 1.0625 * 2 = 2.125 ties to 2.0; 2^-8 and 3 * 2^-9
    # are still subnormal (the smallest normal is 2^-6)
    want2 = [0x40, 0x40, 0x42, 0x4C, 0x7E, 0xFE, 0x02, 0x01, 0x03, 0xFE, 0x7E, 0x00, 0x80,
             0x7E, 0x7E, 0x7E, 0x80]
    n = len(vals)
    x = bf16_bits_of([vals + [0.0] * (32 - n)])
    assert np.array_equal(bf16_vals(x)[0, :n], np.float32(vals))  # exact in bf16
    for s, want in ((1.0, want1), (2.0, want2)):
        o = oracle.dispatch(x, np.array([[0]], np.int32), None, 1, 1, 6, 0,
                            np.array([s], np.float32), 1)
        assert o["expand_x"][0, :n].tolist() == want, s
    # NaN inputs of either sign, and an infinity times a zero coefficient: 0x7F
    nan = np.array([[0x7FC0, 0xFFC0, 0x7F80, 0xFF80] + [0] * 28], dtype=np.uint16)
    o = oracle.dispatch(nan, np.array([[0]], np.int32), None, 1, 1, 6, 0,
                        np.array([1.0], np.float32), 1)
    assert o["expand_x"][0, :4].tolist() == [0x7F, 0x7F, 0x7E, 0xFE]
    o = oracle.dispatch(nan, np.array([[0]], np.int32), None, 1, 1, 6, 0,
                        np.array([0.0], np.float32), 1)
    assert o["expand_x"][0, :4].tolist() == [0x7F, 0x7F, 0x7F, 0x7F]
    assert o["expand_x"][0, 4:].tolist() == [0] * 28


@pytest.mark.parametrize("kind", [0, 2, 3])
def test_static_e4m3_takes_one_coefficient_only(kind):
    rng, x, ids, E = case(183)
    H = x.shape[1]
    qs = {0: None, 2: np.ones(H, np.float32), 3: np.ones((E, H), np.float32)}[kind]
    with pytest.raises(ValueError):
        oracle.dispatch(x, ids, None, 2, 3, 6, 0, qs, kind)
