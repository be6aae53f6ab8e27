"""GPU parity of the expert computation (grouped mxfp8 GEMM) against the oracle.

Tolerance, derived from the arithmetic of the instruction the kernel uses
(v_mfma_scale_f32_16x16x128_f8f6f4; measured with one-wave probes on single
products, since the ISA does not spell it out):
  - each product of two E4M3 values and two E8M0 scales is exact;
  - products are summed in groups of 8 consecutive K; within a group each
    product is truncated toward zero to a multiple of 2^-13 times the leading
    power of two of the group's largest product (1 + 2^-13 survives, 1 + 2^-14
    does not, 1 - 1.75 * 2^-13 gives 1 - 2^-13), so a group loses less than
    7 * 2^-13 of its largest product;
  - group sums are accumulated in fp32 with round to nearest even (1 + 2^-23
    from another block survives), at most about Kd/8 additions;
  - the fp32 result is rounded once to bf16 (half an ulp, 2^-9 relative).
With abs64 the sum of the products' magnitudes, the test allows
|gpu - exact| <= 2^-8 |exact| + (7 * 2^-13 + Kd * 2^-26) * abs64,
twice the bf16 and fp32 terms and the full worst case of the truncation term.
Rows outside every instance's range must keep their poison bytes.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_expert_amd import workloads as W

from gpu_common import M, say

pytestmark = pytest.mark.gpu
POISON16 = 0xFFFF  # a bf16 NaN pattern: any row written by mistake shows
# Share of sampled outputs that must equal the oracle's bf16 bit for bit.  Measured on
# MI355X: 0.966-0.973 on every sampled case (Kd from 512 to 16384, the bench shape, 1024
# instances, 4M rows, both tilings); a structural mistake (a wrong block, chunk, scale or
# row) leaves almost none equal, and an accuracy loss in the accumulation far fewer.
BIT_EQUAL_MIN = 0.9


def run_gpu(g: W.GemmCase, offsets=None, dev_err=None):
    m = M()
    off = g.offsets if offsets is None else offsets
    y = torch.full((g.rows, g.N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    m.moe_expert_gemm(torch.from_numpy(g.a).cuda(), torch.from_numpy(g.a_sc).cuda(),
                      torch.from_numpy(np.ascontiguousarray(off, np.int32)).cuda(),
                      torch.from_numpy(g.w).cuda(),
                      m.pack_mx_weight_scales(torch.from_numpy(g.w_sc).cuda()), y=y,
                      dev_err=dev_err)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def f32(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_close(y_bits, y64, abs64, Kd, where=""):
    got = f32(y_bits)
    tol = 2.0 ** -8 * np.abs(y64) + (7 * 2.0 ** -13 + Kd * 2.0 ** -26) * abs64
    err = np.abs(got - y64)
    bad = ~(err <= tol)
    assert not bad.any(), (f"{where}: {bad.sum()} of {bad.size} outside tolerance; worst "
                           f"{np.max(err / np.maximum(tol, 1e-300)):.3g}x at "
                           f"{np.unravel_index(np.argmax(err - tol), err.shape)}")


CASES = [
    # (counts per instance, N, Kd, tail rows)
    ([0, 17, 130, 1, 255], 256, 256, 5),      # ragged tiles, an empty instance, spare rows
    ([128], 128, 128, 0),                     # exactly one tile
    ([1, 129, 64], 384, 384, 0),
    ([3, 0, 0, 7, 0, 200, 0, 1], 128, 512, 2),
    ([5, 260, 0, 131], 256, 1536, 1),         # three scale groups: an odd count of groups
    (list(np.random.default_rng(77).integers(0, 21, 64)), 128, 128, 3),  # many small instances
    ([300, 41], 256, 1024, 0),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_gemm_parity_small(ci):
    counts, N, Kd, tail = CASES[ci]
    say(f"[gemm] case {ci}: counts={list(map(int, counts))[:12]} N={N} Kd={Kd} tail={tail}")
    g = W.make_gemm_case(500 + ci, counts, N, Kd, tail=tail)
    y = run_gpu(g)
    ref, y64, abs64 = oracle.expert_gemm_mx(g.a, g.a_sc, g.offsets, g.w, g.w_sc)
    last = int(g.offsets[-1])
    assert_close(y[:last], y64[:last], abs64[:last], Kd, f"case {ci}")
    assert np.all(y[last:] == POISON16)
    # most outputs are the oracle's bf16 bit for bit (measured: about 97%); a structural
    # mistake (a wrong block, chunk or scale) leaves far fewer
    assert np.mean(y[:last] == ref[:last]) > BIT_EQUAL_MIN if last else True


def test_gemm_all_instances_empty():
    say("[gemm] all instances empty")
    g = W.make_gemm_case(600, [0, 0, 0], 128, 128, tail=10)
    y = run_gpu(g)
    assert np.all(y == POISON16)


def test_gemm_malformed_offsets_flagged_in_bounds():
    """Offsets that decrease or leave [0, rows] raise the error bit; every range is clamped
    into the buffer, so nothing outside y is written (the guard rows after it stay poisoned)."""
    say("[gemm] malformed offsets")
    m = M()
    g = W.make_gemm_case(601, [50, 10, 40], 128, 128)
    for off in ([0, 50, 20, 100], [-5, 10, 60, 100], [0, 30, 60, 140]):
        dev_err = torch.zeros(1, dtype=torch.int32, device="cuda")
        guard = torch.full((g.rows + 64, g.N), -1, dtype=torch.int16, device="cuda")
        y = guard[:g.rows].view(torch.bfloat16)
        m.moe_expert_gemm(torch.from_numpy(g.a).cuda(), torch.from_numpy(g.a_sc).cuda(),
                          torch.tensor(off, dtype=torch.int32, device="cuda"),
                          torch.from_numpy(g.w).cuda(),
                          m.pack_mx_weight_scales(torch.from_numpy(g.w_sc).cuda()), y=y,
                          dev_err=dev_err)
        torch.cuda.synchronize()
        assert int(dev_err.item()) & m.ERR_OFFSETS, off
        assert torch.all(guard[g.rows:] == -1), off


def test_gemm_full_size_sampled():
    """The bench shape (8 instances, 4096 rows, Kd = 7168, N = 4096) in the bench's launch:
    sampled rows (first, last and a middle row of every instance) and 256 sampled columns
    spread over all column tiles are checked against the oracle on that sub-problem."""
    g = W.make_g3()
    say(f"[gemm] full size: counts={g.counts.tolist()} N={g.N} Kd={g.Kd}")
    y = run_gpu(g)
    rng = np.random.default_rng(9)
    rows, inst = [], []
    for e in range(g.E):
        lo, hi = int(g.offsets[e]), int(g.offsets[e + 1])
        for r in sorted({lo, (lo + hi) // 2, hi - 1} if hi > lo else set()):
            rows.append(r)
            inst.append(e)
    rows = np.array(rows)
    cols = np.sort(rng.choice(g.N, 256, replace=False))
    sub_counts = np.bincount(np.array(inst), minlength=g.E)
    sub_off = np.zeros(g.E + 1, np.int32)
    sub_off[1:] = np.cumsum(sub_counts)
    ref, y64, abs64 = oracle.expert_gemm_mx(g.a[rows], g.a_sc[rows], sub_off,
                                            np.ascontiguousarray(g.w[:, cols]),
                                            np.ascontiguousarray(g.w_sc[:, cols]))
    got = y[rows][:, cols]
    assert_close(got, y64, abs64, g.Kd, "g3 sample")
    equal = float(np.mean(got == ref))
    say(f"[gemm] g3 sample: {equal:.3f} of sampled outputs bit-equal to the oracle")
    assert equal > BIT_EQUAL_MIN, equal
    assert not np.any(y[:int(g.offsets[-1])] == POISON16)




def check_sampled(g, y, cols=None, extra_rows=(), where=""):
    """The first, middle and last row of every instance (plus extra_rows) and the given
    columns (all by default) against the oracle on that sub-problem: within the tolerance,
    and mostly equal to the oracle's bf16 bit for bit."""
    rows, inst = [], []
    for e in range(g.E):
        lo, hi = int(g.offsets[e]), int(g.offsets[e + 1])
        pick = {lo, (lo + hi) // 2, hi - 1} if hi > lo else set()
        pick |= {r for r in extra_rows if lo <= r < hi}
        for r in sorted(pick):
            rows.append(r)
            inst.append(e)
    rows = np.array(rows)
    cols = np.arange(g.N) if cols is None else np.asarray(cols)
    sub_off = np.zeros(g.E + 1, np.int32)
    sub_off[1:] = np.cumsum(np.bincount(np.array(inst), minlength=g.E))
    ref, y64, abs64 = oracle.expert_gemm_mx(g.a[rows], g.a_sc[rows], sub_off,
                                            np.ascontiguousarray(g.w[:, cols]),
                                            np.ascontiguousarray(g.w_sc[:, cols]))
    got = y[rows][:, cols]
    assert_close(got, y64, abs64, g.Kd, where)
    equal = float(np.mean(got == ref))
    say(f"[gemm] {where}: {equal:.3f} of sampled outputs bit-equal to the oracle")
    assert equal > BIT_EQUAL_MIN, (where, equal)


def test_gemm_max_instances():
    """1024 instances (the limit), most with 0-3 rows: the instance prefix and the binary
    search over it at full length."""
    counts = np.random.default_rng(7101).integers(0, 4, 1024)
    g = W.make_gemm_case(7102, counts, 128, 128, tail=5)
    say(f"[gemm] 1024 instances, {int(g.offsets[-1])} rows")
    y = run_gpu(g)
    check_sampled(g, y, where="1024 instances")
    assert np.all(y[int(g.offsets[-1]):] == POISON16)


def test_gemm_max_k_and_max_n():
    """K = 16384 (the limit: 128 K steps, 32 scale groups) and, separately, N = 16384 (64
    column tiles; 256 sampled columns checked)."""
    g = W.make_gemm_case(7103, [200, 77, 129], 256, 16384)
    say("[gemm] K = 16384")
    check_sampled(g, run_gpu(g), where="K=16384")
    g = W.make_gemm_case(7104, [130, 3], 16384, 128)
    say("[gemm] N = 16384")
    cols = np.sort(np.random.default_rng(7105).choice(g.N, 256, replace=False))
    check_sampled(g, run_gpu(g), cols=cols, where="N=16384")


def test_gemm_max_rows():
    """4194304 rows (the limit; 32768 row tiles counted in 16 bits on the device, 128
    rounds of the grid), split into two instances at a row that is not a tile boundary;
    sampled rows checked."""
    g = W.make_gemm_case(7106, [4194304 - 1000, 1000], 128, 128)
    say("[gemm] 4194304 rows")
    y = run_gpu(g)
    extra = np.random.default_rng(7107).integers(0, g.rows, 64)
    check_sampled(g, y, extra_rows=extra, where="4M rows")



def test_gemm_wide_tiling():
    """Shapes whole rounds of 256 x 256 tiles fill (one and three rounds on 256 CUs), where
    the launch takes the wide tiling: sampled rows and columns against the oracle."""
    for seed, counts, N, Kd in ((7201, [4096], 4096, 512), (7202, [4096, 8192], 4096, 512)):
        g = W.make_gemm_case(seed, counts, N, Kd)
        say(f"[gemm] wide tiling: counts={counts} N={N} Kd={Kd}")
        y = run_gpu(g)
        cols = np.sort(np.random.default_rng(seed).choice(g.N, 256, replace=False))
        extra = np.random.default_rng(seed + 1).integers(0, g.rows, 48)
        check_sampled(g, y, cols=cols, extra_rows=extra, where=f"wide {counts}")


def mx_tiling(counts, rows, N, cus=256):
    """The mxfp8 launch's choice (with grouped scales) restated on the host: 'narrow' or
    ('wide', split of the last round's tiles), from the row tiles of both tilings and the
    cost model the kernel applies."""
    def cost(tiles, G, round_cost, quarter, half):
        r, tail = divmod(tiles, G)
        split = 1 if tail == 0 else (4 if G // tail >= 4 else (2 if G // tail >= 2 else 1))
        last = 0.0 if tail == 0 else (quarter if split == 4 else half if split == 2 else 1.0)
        return np.float32(round_cost) * np.float32(r + last), split
    col_tiles = -(-N // 256)
    m_narrow = sum(-(-c // 128) for c in counts)
    m_wide = sum(-(-c // 256) for c in counts)
    G = min((-(-rows // 128) + len(counts)) * col_tiles, cus)
    cw, split = cost(m_wide * col_tiles, G, 1.9, 0.5, 0.6)
    cn, _ = cost(m_narrow * col_tiles, G, 1.0, 0.5, 0.67)
    return ("wide", split) if cw < cn else ("narrow", None)


WIDE_RAGGED = [
    # (seed, counts per instance, N, Kd, spare rows, the branch the launch takes)
    (7211, [6176], 2048, 512, 40, ("wide", 1)),                  # a ragged last row tile
    (7212, [3000, 1500, 2600, 700], 2048, 512, 17, ("wide", 1)),  # boundaries inside tiles
    (7213, [36928], 1024, 512, 8, ("wide", 2)),                  # last round in half tiles
    (7214, [20000, 16928], 1024, 512, 3, ("wide", 2)),
    (7215, [51264], 1024, 512, 64, ("wide", 4)),                 # last round in quarter tiles
]


@pytest.mark.parametrize("case", WIDE_RAGGED, ids=[f"w{c[0]}" for c in WIDE_RAGGED])
def test_gemm_wide_tiling_ragged_and_split(case):
    """Shapes on which the launch takes the 256 x 256 tiling with a ragged last row tile,
    instance boundaries inside the walk, and a last round cut into half or quarter pieces:
    rows at every instance's ends and around each 256-row tile boundary near them, plus
    random rows, all columns, against the oracle; spare rows past the last instance stay
    untouched."""
    seed, counts, N, Kd, tail, branch = case
    g = W.make_gemm_case(seed, counts, N, Kd, tail=tail)
    assert mx_tiling(counts, g.rows, N) == branch
    say(f"[gemm] wide tiling {branch}: counts={counts} N={N} Kd={Kd} spare={tail}")
    y = run_gpu(g)
    extra = set(np.random.default_rng(seed + 1).integers(0, g.rows - tail, 48).tolist())
    for e in range(g.E):
        lo, hi = int(g.offsets[e]), int(g.offsets[e + 1])
        last_tile = lo + (hi - lo - 1) // 256 * 256  # first row of the instance's last tile
        extra |= {lo + 1, last_tile - 1, last_tile, last_tile + 1, hi - 2}
    check_sampled(g, y, extra_rows=sorted(extra), where=f"wide {counts}")
    assert np.all(y[g.rows - tail:] == POISON16), "spare rows were written"


# ---------------------------------------------------------------- int8 operands

def run_gpu_i8(g, quant_mode):
    m = M()
    y = torch.full((g.rows, g.N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    m.moe_expert_gemm(torch.from_numpy(g.a).cuda(), torch.from_numpy(g.a_sc).cuda(),
                      torch.from_numpy(g.offsets).cuda(), torch.from_numpy(g.w).cuda(),
                      torch.from_numpy(g.w_sc).cuda(), quant_mode=quant_mode, y=y)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_close_i8(y_bits, y64, abs64, Kd, per_tile, where=""):
    """int8: the integer sums are exact; per token the fp32 conversion and two multiplies
    add at most about 3 * 2^-24 relative; per tile each step's fused multiply-add rounds once
    (Kd/128 of them) and the column scale once more.  Plus half a bf16 ulp."""
    got = f32(y_bits)
    extra = (Kd // 128 + 2) * 2.0 ** -23 if per_tile else 2.0 ** -21
    tol = 2.0 ** -8 * np.abs(y64) + extra * abs64
    err = np.abs(got - y64)
    bad = ~(err <= tol)
    assert not bad.any(), f"{where}: {bad.sum()} of {bad.size} outside tolerance"


I8_CASES = [
    ([0, 17, 130, 1, 255], 256, 256, 5),
    ([128], 128, 128, 0),
    ([1, 129, 64], 384, 384, 0),
    ([3, 0, 0, 7, 0, 200, 0, 1], 128, 512, 2),
    ([300, 41], 256, 1024, 0),
    ([5, 260, 0, 131], 256, 1536, 1),
]


@pytest.mark.parametrize("per_tile", [False, True])
@pytest.mark.parametrize("ci", range(len(I8_CASES)))
def test_gemm_i8_parity_small(ci, per_tile):
    counts, N, Kd, tail = I8_CASES[ci]
    mode = M().QUANT_INT8_TILE if per_tile else M().QUANT_INT8_TOKEN
    say(f"[gemm i8] case {ci} per_tile={per_tile}: counts={counts[:8]} N={N} Kd={Kd}")
    g = W.make_gemm_case_i8(700 + ci, counts, N, Kd, per_tile, tail=tail)
    y = run_gpu_i8(g, mode)
    ref, y64, abs64 = oracle.expert_gemm_i8(g.a, g.a_sc, g.offsets, g.w, g.w_sc)
    last = int(g.offsets[-1])
    assert_close_i8(y[:last], y64[:last], abs64[:last], Kd, per_tile, f"case {ci}")
    assert np.all(y[last:] == POISON16)
    assert np.mean(y[:last] == ref[:last]) > 0.9


@pytest.mark.parametrize("per_tile", [False, True])
def test_gemm_i8_full_size_sampled(per_tile):
    """8 instances, 4096 rows, Kd = 7168, N = 4096, int8; sampled rows and columns."""
    mode = M().QUANT_INT8_TILE if per_tile else M().QUANT_INT8_TOKEN
    rng0 = np.random.default_rng(3100)
    counts = W.zipf_counts(rng0, 4096, 8, 1.2)
    g = W.make_gemm_case_i8(3200 + per_tile, counts, 4096, 7168, per_tile)
    say(f"[gemm i8] full size per_tile={per_tile}")
    y = run_gpu_i8(g, mode)
    rows = []
    for e in range(g.E):
        lo, hi = int(g.offsets[e]), int(g.offsets[e + 1])
        rows += sorted({lo, (lo + hi) // 2, hi - 1}) if hi > lo else []
    rows = np.array(rows)
    cols = np.sort(np.random.default_rng(10).choice(g.N, 256, replace=False))
    inst = np.searchsorted(g.offsets[1:], rows, side="right")
    sub_off = np.zeros(g.E + 1, np.int32)
    sub_off[1:] = np.cumsum(np.bincount(inst, minlength=g.E))
    _, y64, abs64 = oracle.expert_gemm_i8(g.a[rows], g.a_sc[rows], sub_off,
                                          np.ascontiguousarray(g.w[:, cols]),
                                          np.ascontiguousarray(g.w_sc[:, cols]))
    assert_close_i8(y[rows][:, cols], y64, abs64, g.Kd, per_tile, "full size")



@pytest.mark.parametrize("per_tile", [False, True])
def test_gemm_i8_limits(per_tile):
    """int8 at the size limits: K = 16384 (grouped tile scales when per tile) and 1024
    instances of 0-3 rows; sampled rows (first, middle, last of each instance) and columns
    against the oracle."""
    mode = M().QUANT_INT8_TILE if per_tile else M().QUANT_INT8_TOKEN
    cases = ((7301 + per_tile, [200, 77, 129], 256, 16384),
             (7303 + per_tile, list(np.random.default_rng(7305).integers(0, 4, 1024)), 128, 128))
    for seed, counts, N, Kd in cases:
        g = W.make_gemm_case_i8(seed, counts, N, Kd, per_tile)
        say(f"[gemm i8] limits per_tile={per_tile} E={g.E} N={N} Kd={Kd}")
        y = run_gpu_i8(g, mode)
        rows = []
        for e in range(g.E):
            lo, hi = int(g.offsets[e]), int(g.offsets[e + 1])
            rows += sorted({lo, (lo + hi) // 2, hi - 1}) if hi > lo else []
        rows = np.array(rows)
        inst = np.searchsorted(g.offsets[1:], rows, side="right")
        sub_off = np.zeros(g.E + 1, np.int32)
        sub_off[1:] = np.cumsum(np.bincount(inst, minlength=g.E))
        _, y64, abs64 = oracle.expert_gemm_i8(g.a[rows], g.a_sc[rows], sub_off, g.w, g.w_sc)
        assert_close_i8(y[rows], y64, abs64, g.Kd, per_tile, f"limits E={g.E} Kd={Kd}")

def test_gemm_i8_on_dispatch_output():
    """Dispatch (per-token int8, c2 shapes but 128 tokens) then the expert GEMM on its rows,
    against the oracle's dispatch and GEMM (the two dispatch outputs are equal bit for bit)."""
    m = M()
    wl = W.make_small(seed=77, Bs=128, H=1024, K=4, n_ranks=2, local_experts=4,
                      quant_mode=W.QUANT_INT8_TOKEN)
    say("[gemm i8] on dispatch output")
    d = m.moe_dispatch(wl.x.cuda(), wl.logical_ids.cuda(), wl.n_ranks, wl.local_experts,
                       wl.quant_mode)
    od = oracle.dispatch(oracle.bf16_bits(wl.x), wl.logical_ids.numpy(), None, wl.n_ranks,
                         wl.local_experts, wl.quant_mode)
    total = int(od["offsets"][-1])
    assert np.array_equal(d["expand_x"].cpu().numpy()[:total], od["expand_x"][:total])
    rng = np.random.default_rng(5)
    w = rng.integers(-127, 128, size=(wl.E, 256, wl.H), dtype=np.int8)
    w_sc = rng.uniform(0.0002, 0.002, size=(wl.E, 256)).astype(np.float32)
    y = m.moe_expert_gemm(d["expand_x"], d["expand_scales"].reshape(-1), d["expert_offsets"],
                          torch.from_numpy(w).cuda(), torch.from_numpy(w_sc).cuda(),
                          quant_mode=m.QUANT_INT8_TOKEN)
    torch.cuda.synchronize()
    _, y64, abs64 = oracle.expert_gemm_i8(od["expand_x"], od["scales"].reshape(-1),
                                          od["offsets"], w, w_sc)
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert_close_i8(yb[:total], y64[:total], abs64[:total], wl.H, False, "dispatch chain")


# ---------------------------------------------------------------- determinism, graphs

def test_gemm_deterministic_and_graph_replays():
    """Two launches give the same bits; a captured HIP graph of the GEMM (mxfp8 and int8 per
    tile, the split last round included) reproduces the eager output on every replay, with
    the output poisoned before each replay and unrelated eager work between replays."""
    m = M()
    say("[gemm] determinism and graph replays")
    g = W.make_gemm_case(800, [300, 41, 0, 129], 512, 1024, tail=3)
    gi = W.make_gemm_case_i8(801, [300, 41, 0, 129], 512, 1024, True, tail=3)
    bufs = []
    for case, mode in ((g, m.QUANT_MXFP8), (gi, m.QUANT_INT8_TILE)):
        t = [torch.from_numpy(np.ascontiguousarray(v)).cuda()
             for v in (case.a, case.a_sc, case.offsets, case.w, case.w_sc)]
        if mode == m.QUANT_MXFP8:
            t[4] = m.pack_mx_weight_scales(t[4])
        y = torch.empty((case.rows, case.N), dtype=torch.bfloat16, device="cuda")
        bufs.append((t, y, mode))

    def launch_all():
        for t, y, mode in bufs:
            m.moe_expert_gemm(*t, quant_mode=mode, y=y)

    launch_all()
    torch.cuda.synchronize()
    first = [y.clone() for _, y, _ in bufs]
    launch_all()
    torch.cuda.synchronize()
    for (_, y, _), f in zip(bufs, first):
        assert torch.equal(y.view(torch.int16), f.view(torch.int16))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch_all()
    other = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for _, y, _ in bufs:
            y.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (_, y, _), f in zip(bufs, first):
            last = y.shape[0] - 3
            assert torch.equal(y[:last].view(torch.int16), f[:last].view(torch.int16)), rep
        other.mul_(1.0001).add_(0.5)
        launch_all()
        torch.cuda.synchronize()
