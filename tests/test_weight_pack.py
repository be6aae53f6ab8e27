"""The group-major mxfp8 exponent layouts (host only): pack_mx_weight_scales turns
the row-major E8M0 weight exponents [E, N, H/32] into the group-major
[E, ceil(H/512), N, 16] layout the expert GEMM reads, with S(e, n, b) =
packed[e][b // 16][n][b % 16] and a zero pad after the last block of a partial group;
the dispatch's group-major activation exponents (quant mode 5) follow the same order
per row."""
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


def test_group_major_activation_buffers_and_test_permutation():
    """The dispatch's group-major exponent buffer (quant mode 5) from the binding, and the
    host-side permutations the GPU tests compare it with: exponent b of row r at
    [b // 16][r][b % 16], a pad after the last block of a partial group, and the two
    permutations inverse to each other on the blocks."""
    from tests.gpu_common import gm_to_row_major, row_major_to_gm
    for H in (1024, 1056, 2080, 7168, 8192):
        nb, G = H // 32, -(-H // 512)
        assert moe.n_scale_entries(moe.QUANT_MXFP8_GM, H) == G * 16
        out = moe.dispatch_buffers(3, H, 2, 4, moe.QUANT_MXFP8_GM, device="cpu")
        assert tuple(out["expand_scales"].shape) == (G, 6, 16)
        assert out["expand_scales"].dtype == torch.uint8
        rng = np.random.default_rng(H)
        sc = rng.integers(0, 255, size=(6, nb), dtype=np.uint8)
        gm = row_major_to_gm(sc, H)
        assert gm.shape == (G, 6, 16)
        for r in range(6):
            for b in range(nb):
                assert gm[b // 16, r, b % 16] == sc[r, b]
        assert np.all(gm[G - 1, :, nb - 16 * (G - 1):] == 0xFF)
        np.testing.assert_array_equal(gm_to_row_major(gm, 6, H), sc)
