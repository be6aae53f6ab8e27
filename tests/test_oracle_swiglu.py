"""Pins of the oracle's activation between the expert FFN's two projections
(CPU only).

The pages name the expert computation in the fixed calling sequence
("aclnnMoeUpdateExpert") and fix its operand formats (dispatch page, 计算公式
case 5) but do not define it; the reading is the gated FFN of a
DeepSeek-V3-shaped layer: act = bf16(silu(gate) * up) on the first
projection's [gate | up] row, then the case-5 mxfp8 quantiser on act.

Pinned against:
- torch.nn.functional.silu in float64 times up, rounded once to bf16 by the
  pinned double -> bf16 rounding;
- closed forms: a zero gate or up gives a signed zero, a large positive gate
  gives bf16(gate * up) (the product is exact in fp64), a very negative gate
  gives -0 for a positive up;
- the codes and E8M0 bytes against a brute-force search over the 256 E4M3 codes
  decoded from the format, with the block exponent from frexp;
- rows outside [offsets[0], offsets[E]) untouched; bad offsets rejected.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_scaled import brute_e4m3


def bf16_bits_of(a):
    return oracle.bf16_bits(torch.from_numpy(np.asarray(a, dtype=np.float32)).bfloat16())


def vals(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def y1_case(seed, rows, I, gate_scale=3.0, up_scale=2.0):
    rng = np.random.default_rng(seed)
    g = rng.normal(0.0, gate_scale, size=(rows, I))
    u = rng.normal(0.0, up_scale, size=(rows, I))
    return bf16_bits_of(np.concatenate([g, u], axis=1))


def silu_ref(y1_bits):
    I = y1_bits.shape[1] // 2
    g = torch.from_numpy(vals(y1_bits[:, :I]))
    u = vals(y1_bits[:, I:])
    a = torch.nn.functional.silu(g).numpy() * u
    return oracle.bf16_round(a).reshape(a.shape)


def test_act_against_torch_silu():
    y1 = y1_case(401, 24, 256)
    off = np.array([0, 5, 5, 24], np.int32)
    act, codes, sc = oracle.swiglu_mx(y1, off)
    np.testing.assert_array_equal(act, silu_ref(y1))


def test_act_closed_forms():
    I = 64
    g = np.zeros((4, I))
    u = np.ones((4, I))
    g[1] = 0.0; u[1] = -3.0                       # zero gate: 0 * -3 = -0
    g[2] = np.linspace(64.0, 512.0, I)            # silu(g) = g to far below a bf16 ulp
    u[2] = np.linspace(-7.0, 9.0, I)
    g[3] = -128.0                                 # silu(-128) * 1 underflows bf16: -0
    u[0] = 0.0                                    # zero up: +0 * 0 = +0
    y1 = bf16_bits_of(np.concatenate([g, u], axis=1))
    act, _, _ = oracle.swiglu_mx(y1, np.array([0, 4], np.int32))
    assert (act[0] == 0x0000).all()
    assert (act[1] == 0x8000).all()
    gu = vals(y1[2, :I]) * vals(y1[2, I:])        # exact in fp64
    np.testing.assert_array_equal(act[2], oracle.bf16_round(gu))
    assert (act[3] == 0x8000).all()


def test_codes_brute_force():
    y1 = y1_case(402, 9, 320, gate_scale=6.0, up_scale=0.5)
    act, codes, sc = oracle.swiglu_mx(y1, np.array([0, 9], np.int32))
    a = vals(act)
    for r in range(a.shape[0]):
        for b in range(a.shape[1] // 32):
            blk = a[r, 32 * b:32 * b + 32]
            m = np.abs(blk).max()
            se = -127 if m == 0 else max(-127, np.frexp(m)[1] - 1 - 8)
            assert sc[r, b] == se + 127
            np.testing.assert_array_equal(codes[r, 32 * b:32 * b + 32],
                                          brute_e4m3(np.ldexp(blk, -se)))


def test_rows_outside_untouched_and_bad_offsets():
    y1 = y1_case(403, 12, 64)
    init = (np.full((12, 64), 0x1234, np.uint16), np.full((12, 64), 0x5A, np.uint8),
            np.full((12, 2), 0xA5, np.uint8))
    act, codes, sc = oracle.swiglu_mx(y1, np.array([2, 6, 9], np.int32), init=init)
    for t, v in zip((act, codes, sc), (0x1234, 0x5A, 0xA5)):
        assert (t[:2] == v).all() and (t[9:] == v).all()
        assert not (t[2:9] == v).all()
    for off in ([0, 13], [-1, 4], [5, 3]):
        with pytest.raises(ValueError):
            oracle.swiglu_mx(y1, np.array(off, np.int32))
