"""Pins for the oracle's number formats and quantisers (CPU only).

Each oracle routine is checked against something other than itself:
  - e4m3: a brute-force nearest-code search over all 256 codes decoded from
    the OCP E4M3 format definition, and torch's float8_e4m3fn cast after
    clamping to +-448;
  - bf16 rounding of doubles: exact rational nearest-neighbour search;
  - int8 per-segment quantiser (dispatch formula cases 3 and 4 of
    "aclnnMoeDistributeDispatchV2"): numpy IEEE float32 arithmetic with
    brute-force round-half-even, and reconstruction / extremum invariants;
  - mxfp8 block quantiser (case 5): the E8M0 exponent from frexp, the codes
    from the brute-force e4m3 search, and the block-maximum invariant.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- e4m3

def e4m3_decode(code: int) -> float:
    """OCP E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; S.1111.111 is NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


MAGS = np.array([e4m3_decode(c) for c in range(0x7F)])  # finite non-negative codes 0..126


def e4m3_brute(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0x00)
    d = np.abs(a[:, None] - MAGS[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # ties -> the even code (at most two candidates tie)
    codes = np.where(cand & (np.arange(0x7F)[None, :] % 2 == 0), np.arange(0x7F)[None, :], 999)
    pick = codes.min(axis=1)
    only = np.argmax(cand, axis=1)
    n_cand = cand.sum(axis=1)
    code = np.where(n_cand > 1, pick, only)
    code = np.where(a >= 448.0, 0x7E, code)  # saturate
    return (code | sign).astype(np.uint8)


def all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_e4m3_decode_table_sanity():
    assert e4m3_decode(0x7E) == 448.0
    assert e4m3_decode(0x08) == 2.0 ** -6
    assert e4m3_decode(0x01) == 2.0 ** -9
    assert e4m3_decode(0x38) == 1.0
    assert np.all(np.diff(MAGS) > 0)  # codes increase with magnitude


def test_e4m3_all_bf16_inputs_vs_brute_force():
    v = all_bf16_values()
    got = oracle.e4m3_encode(v)
    for lo in range(0, v.size, 8192):
        sl = slice(lo, lo + 8192)
        np.testing.assert_array_equal(got[sl], e4m3_brute(v[sl]))


def test_e4m3_midpoints_and_neighbours():
    mids = (MAGS[:-1] + MAGS[1:]) / 2.0
    pts = np.concatenate([mids, MAGS, [448.0, 464.0, 479.0, 480.0, 1e30]]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    v = np.concatenate([pts, up, dn])
    v = np.concatenate([v, -v]).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(v), e4m3_brute(v))


def test_e4m3_random_fp32_vs_brute_force_and_torch():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.uniform(-600, 600, 20000),
        rng.standard_normal(20000) * 2.0 ** rng.integers(-14, 9, 20000),
    ]).astype(np.float32)
    got = oracle.e4m3_encode(v)
    np.testing.assert_array_equal(got, e4m3_brute(v))
    clamped = torch.from_numpy(np.clip(v, -448.0, 448.0))
    ref = clamped.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)


def test_e4m3_signed_zero_and_nan():
    got = oracle.e4m3_encode(np.array([0.0, -0.0, -1e-30, np.nan], dtype=np.float32))
    assert list(got[:3]) == [0x00, 0x80, 0x80]
    assert got[3] & 0x7F == 0x7F


# ---------------------------------------------------------------- bf16 rounding

def bf16_val(b: int) -> Fraction:
    f = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def bf16_brute(v: float) -> int:
    """Nearest bf16 by exact rational comparison over the neighbours of the
    fp32-truncated pattern; ties to the even pattern."""
    t = np.array([v], dtype=np.float64).astype(np.float32).view(np.uint32)[0] >> 16
    best = None
    for b in (int(t) - 2, int(t) - 1, int(t), int(t) + 1, int(t) + 2):
        b &= 0xFFFF
        fb = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
        if not np.isfinite(fb) or (np.signbit(fb) != np.signbit(v) and fb != 0):
            continue
        dist = abs(Fraction(v) - Fraction(float(fb)))
        key = (dist, b & 1)
        if best is None or key < best[0]:
            best = (key, b)
    return best[1]


def test_bf16_round_vs_exact_search():
    rng = np.random.default_rng(12)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-5, 5, 3000),
                        rng.standard_normal(300) * 1e-39])  # bf16 subnormal range
    got = oracle.bf16_round(v)
    for x, g in zip(v, got):
        assert g == bf16_brute(float(x)), (x, hex(g))


def test_bf16_round_exact_ties():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0 (0x3F80)
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: even -> 1+2^-6 (0x3F82)
    got = oracle.bf16_round(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]))
    assert list(got) == [0x3F80, 0x3F82, 0xBF80]
    # a value just above the tie must not be double-rounded down
    got = oracle.bf16_round(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))
    assert got[0] == 0x3F81
    # overflow to infinity and max finite
    big = float((2 - 2.0 ** -8) * 2.0 ** 127)
    got = oracle.bf16_round(np.array([big, float((2 - 2.0 ** -7) * 2.0 ** 127)]))
    assert list(got) == [0x7F80, 0x7F7F]


# ---------------------------------------------------------------- int8

def bf16_bits_of(x32: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits(torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16))


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def rne_brute(v: np.ndarray) -> np.ndarray:
    lo = np.floor(v)
    hi = lo + 1
    dl = v - lo
    dh = hi - v
    pick = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    return np.clip(pick, -127, 127).astype(np.int8)


@pytest.mark.parametrize("n,scale", [(1024, 1.0), (128, 1.0), (96, 1e-3), (7168, 40.0),
                                     (4096, 1e-38)])
def test_int8_segment_vs_numpy_float32(n, scale):
    rng = np.random.default_rng(n)
    for trial in range(20):
        xb = bf16_bits_of(rng.standard_normal(n) * scale)
        q, s = oracle.quant_int8(xb)
        x = bits_to_f32(xb)
        m = np.max(np.abs(x))
        d = np.float32(127.0) / np.float32(m)
        v = x * d  # IEEE float32 products
        np.testing.assert_array_equal(q, rne_brute(v.astype(np.float64)))
        np.testing.assert_array_equal(q, np.clip(np.rint(v), -127, 127).astype(np.int8))
        assert np.float32(s) == np.float32(1.0) / d


def test_int8_invariants():
    rng = np.random.default_rng(5)
    for trial in range(50):
        n = int(rng.integers(1, 300))
        x32 = rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3)
        if trial % 2:
            x32[rng.integers(n)] = -np.abs(x32).max() * 3  # negative extremum
        xb = bf16_bits_of(x32)
        x = bits_to_f32(xb).astype(np.float64)
        q, s = oracle.quant_int8(xb)
        j = int(np.argmax(np.abs(x)))
        assert abs(int(q[j])) == 127 and np.sign(q[j]) == np.sign(x[j])
        # reconstruction within half a step, plus the fp32 rounding of d = 127/m
        # and of the product x*d (each below 2^-17 of a step for |x*d| <= 127)
        assert np.all(np.abs(x - q.astype(np.float64) * s) <= s * (0.5 + 2.0 ** -15))
        assert np.all(np.sign(q) * np.sign(x) >= 0)
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(q[order].astype(np.int32)) >= 0)  # monotone


def test_int8_zero_segment_and_worked_values():
    q, s = oracle.quant_int8(np.zeros(64, dtype=np.uint16))
    assert s == 0.0 and not q.any()
    # maximum a tiny subnormal: 127 / m overflows to +inf in fp32, so nonzero
    # elements saturate, zeros (0 * inf) stay 0 and the scale 1/inf is 0
    xb = np.array([0x0001, 0x8003, 0x0000, 0x8000, 0x0002], np.uint16)
    assert np.isinf(np.float32(127.0) / bits_to_f32(xb[1:2])[0].__abs__())
    q, s = oracle.quant_int8(xb)
    assert list(q) == [127, -127, 0, 0, 127] and s == 0.0
    # x = [1, -2, 0.5, 4]: m = 4, d = 127/4 = 31.75 (exact);
    # x*d = [31.75, -63.5, 15.875, 127] -> [32, -64 (tie to even), 16, 127]
    q, s = oracle.quant_int8(bf16_bits_of(np.array([1.0, -2.0, 0.5, 4.0])))
    assert list(q) == [32, -64, 16, 127]
    assert np.float32(s) == np.float32(1.0) / np.float32(31.75)


# ---------------------------------------------------------------- mxfp8

def test_mxfp8_block_vs_frexp_and_brute_force():
    rng = np.random.default_rng(13)
    for trial in range(400):
        sc = 10.0 ** rng.uniform(-30, 30) if trial % 3 else 10.0 ** rng.uniform(-41, -37)
        x32 = rng.standard_normal(32) * sc
        if trial % 7 == 0:
            x32[rng.integers(32)] = 0.0
        xb = bf16_bits_of(x32)
        x = bits_to_f32(xb).astype(np.float64)
        codes, sbyte = oracle.quant_mxfp8(xb)
        m = np.max(np.abs(x))
        _, ex = np.frexp(m)           # m = f * 2^ex, f in [0.5, 1)
        se = int(np.clip(ex - 1 - 8, -127, 127)) if m > 0 else -127
        assert sbyte == se + 127
        np.testing.assert_array_equal(codes, e4m3_brute(x * 2.0 ** -se))
        if se > -127:
            top = max(abs(e4m3_decode(int(c))) for c in codes)
            assert 256.0 <= top <= 448.0


def test_mxfp8_zero_block_and_worked_values():
    codes, sbyte = oracle.quant_mxfp8(np.zeros(32, dtype=np.uint16))
    assert sbyte == 0 and not codes.any()
    # max |x| = 3: floor(log2 3) = 1, sharedExp = 1 - 8 = -7, byte 120;
    # 3 * 2^7 = 384 = 1.5 * 2^8 -> code 0x7C; 1 * 2^7 = 2^7 -> 0x70;
    # -0.5 * 2^7 = -64 = -2^6 -> 0x80 | 0x68
    x = np.zeros(32)
    x[:3] = [3.0, 1.0, -0.5]
    codes, sbyte = oracle.quant_mxfp8(bf16_bits_of(x))
    assert sbyte == 120
    assert list(codes[:3]) == [0x7C, 0x70, 0xE8]
    assert not codes[3:].any()


# ---------------------------------------------------------------- non-finite inputs
# The pages do not say how an infinity or a NaN in x is coded.  The reading
# taken: a maximum skips NaN; an infinite maximum gives sharedExp =
# floor(log2 inf) clamped to 127, or the int8 multiplier 127 / inf = 0 with
# scale 1 / 0 = inf; E4M3 codes a NaN as its sign with every other bit set
# and an infinity as +-448 (saturation); int8 codes NaN (and inf * 0) as 0.

def test_mxfp8_nonfinite_worked_values():
    # a block holding +-inf: sharedExp 127 (byte 254), every finite value
    # scaled by 2^-127: 1 -> 2^-127 and -2 -> -2^-126 code +0 / -0;
    # 2^117 -> 2^-10, half the smallest subnormal step, ties to even 0;
    # 2^118 -> 2^-9 = code 1; the largest finite bf16 (2 - 2^-7) * 2^127 ->
    # 1.9921875, which rounds to 2.0 = 0x40; NaN keeps its sign, inf saturates
    x = np.zeros(32, dtype=np.uint16)
    x[:9] = [0x7F80, 0x3F80, 0xC000, 0x7FC0, 0xFFC0, 0x7A00, 0x7A80, 0xFF80, 0x7F7F]
    codes, sbyte = oracle.quant_mxfp8(x)
    assert sbyte == 254
    assert list(codes[:9]) == [0x7E, 0x00, 0x80, 0x7F, 0xFF, 0x00, 0x01, 0xFE, 0x40]
    assert not codes[9:].any()
    # a NaN does not set the maximum: max |x| = 3 as in the finite block
    x = np.zeros(32, dtype=np.uint16)
    x[:4] = [0x7FC0, 0x4040, 0x3F00, 0xFFFF]  # NaN, 3, 0.5, -NaN
    codes, sbyte = oracle.quant_mxfp8(x)
    assert sbyte == 120
    assert list(codes[:4]) == [0x7F, 0x7C, 0x68, 0xFF]
    assert not codes[4:].any()
    # a block of NaN only: maximum 0, sharedExp -127 (byte 0)
    codes, sbyte = oracle.quant_mxfp8(np.full(32, 0x7FC1, dtype=np.uint16))
    assert sbyte == 0 and np.all(codes == 0x7F)


def test_int8_nonfinite_worked_values():
    # [inf, 5, NaN, -3]: m = inf, d = 127 / inf = 0: 5 * 0 = 0, inf * 0 = NaN -> 0
    q, s = oracle.quant_int8(np.array([0x7F80, 0x40A0, 0x7FC0, 0xC040], np.uint16))
    assert list(q) == [0, 0, 0, 0] and s == float("inf")
    # [NaN, 4, -2]: m = 4, d = 31.75: [NaN -> 0, 127, -63.5 -> -64]
    q, s = oracle.quant_int8(np.array([0x7FC0, 0x4080, 0xC000], np.uint16))
    assert list(q) == [0, 127, -64]
    assert np.float32(s) == np.float32(1.0) / np.float32(31.75)
    # NaN only: maximum 0, codes 0, scale 0
    q, s = oracle.quant_int8(np.full(8, 0xFFC0, dtype=np.uint16))
    assert not q.any() and s == 0.0
