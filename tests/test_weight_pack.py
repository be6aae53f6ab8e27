"""The mxfp8 weight-scale preparation (host only): pack_mx_weight_scales turns the
row-major E8M0 exponents [E, N, H/32] into the group-major [E, ceil(H/512), N, 16]
layout the expert GEMM reads, with S(e, n, b) = packed[e][b // 16][n][b % 16] and a
zero pad after the last block of a partial group."""
import numpy as np
import torch

from combine_expert_amd import moe


def check(E, N, nb, seed):
    rng = np.random.default_rng(seed)
    w_sc = rng.integers(1, 255, size=(E, N, nb), dtype=np.uint8)
    packed = moe.pack_mx_weight_scales(torch.from_numpy(w_sc))
    groups = -(-nb // 16)
    assert packed.shape == (E, groups, N, 16) and packed.dtype == torch.uint8
    assert packed.is_contiguous()
    p = packed.numpy()
    for e in range(E):
        for n in range(N):
            for b in range(nb):
                assert p[e, b // 16, n, b % 16] == w_sc[e, n, b]
    pad = groups * 16 - nb
    if pad:
        assert np.all(p[:, groups - 1, :, 16 - pad:] == 0)


def test_pack_whole_groups():
    check(2, 5, 32, 1)          # H = 1024: two whole groups


def test_pack_partial_last_group():
    check(3, 4, 20, 2)          # H = 640: one group and 4 of 16 blocks of the next
    check(1, 7, 4, 3)           # H = 128: a single partial group
