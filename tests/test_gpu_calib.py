"""The measurement kernels on the GPU move the bytes they are declared to
move: the scatter shape writes the high byte of each element of token i's
row to each of its rows, the gather shape writes a + b + the token's rows
(as 32-bit word sums) and then that plus gamma with one word mixed by the
block's reduction, the stream writes its output range and nothing past it.
"""
import numpy as np
import pytest
import torch

from tests.gpu_common import say

pytestmark = pytest.mark.gpu


def _assist(Bs, K, rows, seed):
    rng = np.random.default_rng(seed)
    a = rng.permutation(Bs * K).astype(np.int32)
    a[a >= rows] = -1
    return a


@pytest.mark.parametrize("Bs,H,K", [(16, 1024, 4), (33, 7168, 8), (8, 8192, 16), (5, 1056, 3)])
def test_scatter_shape(Bs, H, K):
    from combine_expert_amd import calib
    say(f"[calib] scatter shape Bs={Bs} H={H} K={K}")
    rows = Bs * K - 3
    x = torch.randn(Bs, H).bfloat16()
    a = _assist(Bs, K, rows, Bs)
    out = torch.full((rows + 4, H), 0xAB, dtype=torch.uint8, device="cuda")
    calib.scatter_shape(x.cuda(), torch.from_numpy(a).cuda(), rows, out)
    got = out.cpu().numpy()
    hi = (x.view(torch.int16).numpy().astype(np.uint16) >> 8).astype(np.uint8)
    for f, r in enumerate(a):
        if r >= 0:
            np.testing.assert_array_equal(got[r], hi[f // K])
    assert np.all(got[rows:] == 0xAB)


@pytest.mark.parametrize("Bs,H,K,with_b", [(16, 1024, 4, True), (9, 7168, 8, True),
                                            (4, 8192, 16, True), (5, 8192, 16, False)])
def test_gather_shape(Bs, H, K, with_b):
    from combine_expert_amd import calib
    say(f"[calib] gather shape Bs={Bs} H={H} K={K} second row={with_b}")
    rows_n = Bs * K - 2
    rng = np.random.default_rng(H + K)
    r = torch.from_numpy(rng.integers(0, 1 << 15, (rows_n, H), dtype=np.int16)).view(torch.bfloat16)
    a = torch.from_numpy(rng.integers(0, 1 << 15, (Bs, H), dtype=np.int16)).view(torch.bfloat16)
    b = torch.from_numpy(rng.integers(0, 1 << 15, (Bs, H), dtype=np.int16)).view(torch.bfloat16)
    g = torch.from_numpy(rng.integers(0, 1 << 15, (H,), dtype=np.int16)).view(torch.bfloat16)
    asg = _assist(Bs, K, rows_n, K)
    o1 = torch.empty(Bs, H, dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty(Bs, H, dtype=torch.bfloat16, device="cuda")
    calib.gather_shape(r.cuda(), torch.from_numpy(asg).cuda(), a.cuda(),
                       b.cuda() if with_b else None, g.cuda(), rows_n, o1, o2)
    w = lambda t: t.view(torch.int16).numpy().view(np.uint32).reshape(t.shape[0] if t.dim() > 1 else 1, -1).astype(np.uint64)
    rw, aw, bw = w(r), w(a), w(b)
    exp1 = (aw + bw) if with_b else aw.copy()  # without b its reads return zeros
    for f, rr in enumerate(asg):
        if rr >= 0:
            exp1[f // K] += rw[rr]
    exp1 = (exp1 & 0xFFFFFFFF).astype(np.uint32)
    np.testing.assert_array_equal(o1.cpu().view(torch.int16).numpy().view(np.uint32).reshape(Bs, -1), exp1)
    # out2 = out1 + gamma (word sums), one word per 4 mixed with the block's value
    got2 = o2.cpu().view(torch.int16).numpy().view(np.uint32).reshape(Bs, -1).astype(np.uint64)
    exp2 = (exp1.astype(np.uint64) + w(g)) & 0xFFFFFFFF
    mask = np.ones_like(exp2, dtype=bool)
    mask[:, 0::4] = False  # the word each lane mixes
    np.testing.assert_array_equal(got2[mask], exp2[mask])


def test_stream_writes_its_range_only():
    from combine_expert_amd import calib
    say("[calib] stream")
    src = torch.randint(0, 255, (3 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.full((2 << 20,), 0x5A, dtype=torch.uint8, device="cuda")
    calib.stream(src, 3 << 20, dst, (1 << 20) + 4096)
    torch.cuda.synchronize()
    tail = dst[(1 << 20) + 4096:].cpu().numpy()
    assert np.all(tail == 0x5A)
