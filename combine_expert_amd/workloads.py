"""Seeded synthetic inputs for MoE dispatch / combine.

This module only draws inputs: token activations, top-K routing, routing
scores, replica mapping tables, expert-output stand-ins, shared-expert
outputs, residuals and RMSNorm weights.  It holds none of the method's
arithmetic (no mapping, histogram, scan, permutation, quantisation or
combine); both the GPU library tests and the CPU oracle tests draw from it.

Shapes follow the Ascend operator pages' problem statement
("aclnnMoeDistributeDispatchV2" / "aclnnMoeDistributeCombineAddRmsNorm",
shape constraints: H in [1024, 8192], 0 < Bs <= 512, 0 < K <= 16;
"aclnnMoeUpdateExpert": at most 1024 deployed instances, mapping table
column 0 = replica count, columns 1.. = instance ids).

Five workloads are defined (c1..c5) plus a replica-mix variant of c4 (c4b):

  c1  Bs=8,   H=1024, E=8   (1 rank x 8),  K=2,  no quantisation, no shared expert,
      expert = identity + per-expert bf16 bias ~N(0, 0.1)
  c2  Bs=512, H=4096, E=64  (8 x 8),       K=8,  per-token int8, 1 shared expert,
      x ~N(0,1) with 0.1% of elements scaled by 10
  c3  Bs=512, H=7168, E=256 (32 x 8),      K=8,  mxfp8, 1 shared expert,
      Zipf(1.2) expert popularity over a seeded permutation of expert ids
  c4  Bs=512, H=8192, 512 logical -> 1024 instances (64 x 16), K=16,
      per-tile int8 (tile 128), scores = softmax over all 512 logits N(0, 1.5),
      top-16, prune score < 0.02, replica = token index mod replica count
  c4b as c4 but a seeded half of the experts have 2 replicas, the rest 1
      (768 instances on 64 x 12)
  c5  16 layers of c3 shapes with per-token int8, fresh Zipf routing per layer

Expert-computation (grouped GEMM) operands, the step between dispatch and
combine:

  g3  one expert-parallel rank's share of a c3-shaped layer: 8 local
      instances, Kd = H = 7168, N = 4096 output columns (a gate and an up
      projection of width 2048 side by side), 4096 rows (the average number
      of rows a rank receives: 32 ranks x 512 tokens x 8 / 32) split over the
      8 instances by a multinomial draw from a Zipf(1.2) law over a seeded
      permutation.  Operands are mxfp8: random finite E4M3 codes with the
      exponent field uniform in [6, 15] (magnitudes 2^-1 .. 448, like the
      codes of a block whose maximum is scaled to the top binade) and E8M0
      block scales uniform in a narrow band (activations 2^-9 .. 2^-5,
      weights 2^-17 .. 2^-13).

N(mu, s) means mean mu and standard deviation s.  bf16 values are fp32 draws
rounded to nearest even.  Seeds: 1000 * config number (+ layer for c5).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

QUANT_NONE = 0
QUANT_INT8_TOKEN = 2
QUANT_INT8_TILE = 3
QUANT_MXFP8 = 4

SHARED_PAGE = 0  # shared term weighted by the sum of the token's active scales
SHARED_ADD = 1   # shared term added with weight 1


def bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 numpy array -> bf16 torch tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _softmax(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=-1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=-1, keepdims=True)


def uniform_distinct_ids(rng, Bs: int, E: int, K: int) -> np.ndarray:
    """K distinct expert ids per token, uniformly at random."""
    return np.argsort(rng.random((Bs, E)), axis=1, kind="stable")[:, :K].astype(np.int32)


def zipf_distinct_ids(rng, Bs: int, E: int, K: int, s: float) -> np.ndarray:
    """K distinct ids per token, drawn without replacement from a Zipf(s)
    popularity law over a seeded permutation of the ids (Gumbel top-K)."""
    perm = rng.permutation(E)
    p = np.empty(E)
    p[perm] = (np.arange(E) + 1.0) ** (-s)
    p /= p.sum()
    keys = np.log(p)[None, :] + rng.gumbel(size=(Bs, E))
    return np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)


def softmax_scales(rng, Bs: int, K: int) -> np.ndarray:
    """Routing weights: softmax over the K chosen experts of N(0,1) logits."""
    return _softmax(rng.normal(0.0, 1.0, size=(Bs, K))).astype(np.float32)


def identity_table(n: int) -> np.ndarray:
    """Mapping table where logical expert e has one instance, e itself."""
    t = np.empty((n, 2), dtype=np.int32)
    t[:, 0] = 1
    t[:, 1] = np.arange(n, dtype=np.int32)
    return t


@dataclass
class Workload:
    name: str
    Bs: int
    H: int
    K: int
    n_ranks: int
    local_experts: int
    n_logical: int
    quant_mode: int
    tile: int
    x: torch.Tensor                    # bf16 [Bs, H]
    logical_ids: torch.Tensor          # int32 [Bs, K]
    scales: torch.Tensor               # f32 [Bs, K]
    table: torch.Tensor                # int32 [n_logical, F]
    prune_thr: Optional[torch.Tensor]  # f32 [K] or None
    token_mask: Optional[torch.Tensor] # u8 [Bs] or None
    residual: torch.Tensor             # bf16 [Bs, H]
    gamma: torch.Tensor                # bf16 [H]
    eps: float
    shared: Optional[torch.Tensor]     # bf16 [Bs, H] or None
    shared_mode: int = SHARED_PAGE
    expert_out: Optional[torch.Tensor] = None  # bf16 [Bs*K, H] (None: made by expert_bias)
    expert_bias: Optional[torch.Tensor] = None # bf16 [E, H] (identity + bias expert)
    extra: dict = field(default_factory=dict)

    @property
    def E(self) -> int:
        return self.n_ranks * self.local_experts

    @property
    def F(self) -> int:
        return int(self.table.shape[1])


def _combine_side(rng, Bs, H):
    residual = bf16(rng.normal(0.0, 1.0, size=(Bs, H)))
    gamma = bf16(rng.normal(1.0, 0.1, size=(H,)))
    return residual, gamma


def make_c1(seed: int = 1000) -> Workload:
    rng = np.random.default_rng(seed)
    Bs, H, E, K = 8, 1024, 8, 2
    x = bf16(rng.normal(0.0, 1.0, size=(Bs, H)))
    ids = uniform_distinct_ids(rng, Bs, E, K)
    scales = softmax_scales(rng, Bs, K)
    bias = bf16(rng.normal(0.0, 0.1, size=(E, H)))
    residual, gamma = _combine_side(rng, Bs, H)
    return Workload("c1", Bs, H, K, 1, E, E, QUANT_NONE, 0, x, torch.from_numpy(ids),
                    torch.from_numpy(scales), torch.from_numpy(identity_table(E)), None, None,
                    residual, gamma, 1e-6, None, expert_bias=bias)


def make_c2(seed: int = 2000) -> Workload:
    rng = np.random.default_rng(seed)
    Bs, H, R, L, K = 512, 4096, 8, 8, 8
    xf = rng.normal(0.0, 1.0, size=(Bs, H)).astype(np.float32)
    n_out = int(round(0.001 * Bs * H))
    hot = rng.choice(Bs * H, size=n_out, replace=False)
    xf.reshape(-1)[hot] *= 10.0
    x = bf16(xf)
    ids = uniform_distinct_ids(rng, Bs, R * L, K)
    scales = softmax_scales(rng, Bs, K)
    eout = bf16(rng.normal(0.0, 1.0, size=(Bs * K, H)))
    shared = bf16(rng.normal(0.0, 1.0, size=(Bs, H)))
    residual, gamma = _combine_side(rng, Bs, H)
    return Workload("c2", Bs, H, K, R, L, R * L, QUANT_INT8_TOKEN, 0, x, torch.from_numpy(ids),
                    torch.from_numpy(scales), torch.from_numpy(identity_table(R * L)), None,
                    None, residual, gamma, 1e-6, shared, expert_out=eout)


def make_c3(seed: int = 3000, quant_mode: int = QUANT_MXFP8, with_expert_out: bool = True,
            name: str = "c3") -> Workload:
    rng = np.random.default_rng(seed)
    Bs, H, R, L, K = 512, 7168, 32, 8, 8
    x = bf16(rng.normal(0.0, 1.0, size=(Bs, H)))
    ids = zipf_distinct_ids(rng, Bs, R * L, K, 1.2)
    scales = softmax_scales(rng, Bs, K)
    eout = bf16(rng.normal(0.0, 1.0, size=(Bs * K, H))) if with_expert_out else None
    shared = bf16(rng.normal(0.0, 1.0, size=(Bs, H)))
    residual, gamma = _combine_side(rng, Bs, H)
    return Workload(name, Bs, H, K, R, L, R * L, quant_mode, 0, x, torch.from_numpy(ids),
                    torch.from_numpy(scales), torch.from_numpy(identity_table(R * L)), None,
                    None, residual, gamma, 1e-6, shared, expert_out=eout)


def _c4_table(rng, n_logical: int, two_replicas: np.ndarray, n_slots: int) -> np.ndarray:
    """Place each logical expert's replicas on distinct seeded-random instance slots."""
    slots = rng.permutation(n_slots).astype(np.int32)  # unused slots stay empty
    table = np.full((n_logical, 3), -1, dtype=np.int32)
    pos = 0
    for e in range(n_logical):
        n = 2 if two_replicas[e] else 1
        table[e, 0] = n
        table[e, 1:1 + n] = slots[pos:pos + n]
        pos += n
    assert pos <= n_slots
    return table


def make_c4(seed: int = 4000, variant: str = "c4") -> Workload:
    rng = np.random.default_rng(seed)
    Bs, H, K, n_logical = 512, 8192, 16, 512
    x = bf16(rng.normal(0.0, 1.0, size=(Bs, H)))
    probs = _softmax(rng.normal(0.0, 1.5, size=(Bs, n_logical)))
    ids = np.argsort(-probs, axis=1, kind="stable")[:, :K].astype(np.int32)
    scores = np.take_along_axis(probs, ids.astype(np.int64), axis=1).astype(np.float32)
    if variant == "c4":
        two = np.ones(n_logical, dtype=bool)
        R, L = 64, 16
    else:
        two = np.zeros(n_logical, dtype=bool)
        two[rng.choice(n_logical, size=n_logical // 2, replace=False)] = True
        R, L = 64, 12
    table = _c4_table(rng, n_logical, two, R * L)
    eout = bf16(rng.normal(0.0, 1.0, size=(Bs * K, H)))
    residual, gamma = _combine_side(rng, Bs, H)
    thr = np.full((K,), 0.02, dtype=np.float32)
    return Workload(variant, Bs, H, K, R, L, n_logical, QUANT_INT8_TILE, 128, x,
                    torch.from_numpy(ids), torch.from_numpy(scores), torch.from_numpy(table),
                    torch.from_numpy(thr), None, residual, gamma, 1e-6, None,
                    expert_out=eout)


def make_c5_layers(n_layers: int = 16, base_seed: int = 5000, with_expert_out: bool = True):
    """Per-layer inputs of the c5 stack.  Layer 0 carries x and residual; later
    layers take x_{l+1} = y_l and residual_{l+1} = x_out_l from the run itself."""
    return [make_c3(seed=base_seed + l, quant_mode=QUANT_INT8_TOKEN,
                    with_expert_out=with_expert_out, name=f"c5.l{l}") for l in range(n_layers)]


def make(name: str) -> Workload:
    return {"c1": make_c1, "c2": make_c2, "c3": make_c3, "c4": make_c4,
            "c4b": lambda: make_c4(variant="c4b")}[name]()


def make_small(seed: int, Bs: int, H: int, K: int, n_ranks: int, local_experts: int,
               quant_mode: int, tile: int = 128, prune: bool = False, shared: bool = True,
               token_mask_prefix: Optional[int] = None, replicas: bool = False,
               x_scale: float = 1.0) -> Workload:
    """A small seeded case for parity tests: several tiles and a ragged tail."""
    rng = np.random.default_rng(seed)
    E = n_ranks * local_experts
    n_logical = E // 2 if replicas else E
    K = min(K, n_logical)
    x = bf16(rng.normal(0.0, x_scale, size=(Bs, H)))
    ids = uniform_distinct_ids(rng, Bs, n_logical, K)
    scales = softmax_scales(rng, Bs, K)
    if replicas:
        table = _c4_table(rng, n_logical, np.ones(n_logical, dtype=bool), E)
    else:
        table = identity_table(E)
    thr = torch.full((K,), 0.9 / K, dtype=torch.float32) if prune else None
    tmask = None
    if token_mask_prefix is not None:
        m = np.zeros(Bs, dtype=np.uint8)
        m[:token_mask_prefix] = 1
        tmask = torch.from_numpy(m)
    eout = bf16(rng.normal(0.0, 1.0, size=(Bs * K, H)))
    sh = bf16(rng.normal(0.0, 1.0, size=(Bs, H))) if shared else None
    residual, gamma = _combine_side(rng, Bs, H)
    return Workload(f"small{seed}", Bs, H, K, n_ranks, local_experts, n_logical, quant_mode,
                    tile if quant_mode == QUANT_INT8_TILE else 0, x, torch.from_numpy(ids),
                    torch.from_numpy(scales), torch.from_numpy(table), thr, tmask, residual,
                    gamma, 1e-6, sh, expert_out=eout)


def identity_bias_expert(expand_x: torch.Tensor, offsets: torch.Tensor,
                         bias: torch.Tensor) -> torch.Tensor:
    """Stand-in expert FFN for c1: row r of instance e returns bf16(x_row + bias[e]).

    Rows past offsets[E] are filled with zeros.  This is the step between
    dispatch and combine, outside both; it only reads the dispatch output.
    """
    rows, H = expand_x.shape
    E = bias.shape[0]
    off = offsets.to(torch.int64).cpu()
    out = torch.zeros((rows, H), dtype=torch.bfloat16)
    total = int(off[E])
    if total == 0:
        return out
    r = torch.arange(total)
    inst = torch.searchsorted(off[1:E + 1], r, right=True)
    out[:total] = (expand_x[:total].float().cpu() + bias[inst].float()).to(torch.bfloat16)
    return out


def make_quant_scales(seed: int, kind: int, E: int, H: int, lo: float = 0.25,
                      hi: float = 4.0) -> Optional[torch.Tensor]:
    """Seeded scales input of the dispatch: kind 1 -> f32 [1], 2 -> [H] (one
    row shared by the experts), 3 -> [E, H] (one row per instance); values
    uniform in [lo, hi).  kind 0 -> None."""
    if kind == 0:
        return None
    rng = np.random.default_rng(seed)
    shape = {1: (1,), 2: (H,), 3: (E, H)}[kind]
    return torch.from_numpy(rng.uniform(lo, hi, size=shape).astype(np.float32))


def e4m3_codes(rng, shape, ef_lo: int = 6, ef_hi: int = 15) -> np.ndarray:
    """Random finite OCP E4M3 codes: uniform sign bit, exponent field uniform
    in [ef_lo, ef_hi], mantissa field uniform (the NaN pattern S.1111.111 is
    replaced by S.1111.110)."""
    u8 = np.uint8
    sign = rng.integers(0, 2, size=shape, dtype=u8) << u8(7)
    ef = rng.integers(ef_lo, ef_hi + 1, size=shape, dtype=u8)
    m = rng.integers(0, 8, size=shape, dtype=u8)
    m[(ef == 15) & (m == 7)] = 6
    return sign | (ef << u8(3)) | m


def e8m0_codes(rng, shape, lo: int, hi: int) -> np.ndarray:
    """Random E8M0 scale codes uniform in [lo, hi] (2^(lo-127) .. 2^(hi-127))."""
    return rng.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def zipf_counts(rng, total: int, E: int, s: float) -> np.ndarray:
    """Rows per instance: a multinomial draw of `total` rows over a Zipf(s)
    law on a seeded permutation of the E instances."""
    perm = rng.permutation(E)
    p = np.empty(E)
    p[perm] = (np.arange(E) + 1.0) ** (-s)
    return rng.multinomial(total, p / p.sum()).astype(np.int32)


@dataclass
class GemmCase:
    name: str
    E: int
    N: int
    Kd: int
    rows: int                # capacity of a / y; rows past offsets[E] are not part of any instance
    offsets: np.ndarray      # int32 [E+1], offsets[0] = 0, non-decreasing
    a: np.ndarray            # u8 E4M3 [rows, Kd]
    a_sc: np.ndarray         # u8 E8M0 [rows, Kd/32]
    w: np.ndarray            # u8 E4M3 [E, N, Kd]
    w_sc: np.ndarray         # u8 E8M0 [E, N, Kd/32]

    @property
    def counts(self) -> np.ndarray:
        return np.diff(self.offsets).astype(np.int32)


def make_gemm_case(seed: int, counts, N: int, Kd: int, tail: int = 0,
                   name: str = "gemm") -> GemmCase:
    """mxfp8 grouped-GEMM operands for the given rows per instance, plus
    `tail` spare rows past the last instance."""
    rng = np.random.default_rng(seed)
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.size
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    rows = int(offsets[-1]) + tail
    a = e4m3_codes(rng, (rows, Kd))
    a_sc = e8m0_codes(rng, (rows, Kd // 32), 118, 122)
    w = e4m3_codes(rng, (E, N, Kd))
    w_sc = e8m0_codes(rng, (E, N, Kd // 32), 110, 114)
    return GemmCase(name, E, N, Kd, rows, offsets, a, a_sc, w, w_sc)


@dataclass
class GemmCaseI8:
    name: str
    E: int
    N: int
    Kd: int
    rows: int
    offsets: np.ndarray      # int32 [E+1]
    a: np.ndarray            # int8 [rows, Kd]
    a_sc: np.ndarray         # f32 [rows] (per token) or [rows, Kd/128] (per tile)
    w: np.ndarray            # int8 [E, N, Kd]
    w_sc: np.ndarray         # f32 [E, N] (one per output column)

    @property
    def counts(self) -> np.ndarray:
        return np.diff(self.offsets).astype(np.int32)


def make_gemm_case_i8(seed: int, counts, N: int, Kd: int, per_tile: bool, tail: int = 0,
                      name: str = "gemm_i8") -> GemmCaseI8:
    """int8 grouped-GEMM operands: codes uniform in [-127, 127] (the range the dynamic
    quantisers produce), activation scales uniform in [0.002, 0.05] per row or per tile of
    128 (1/127 of a row maximum of about 0.25 .. 6), weight scales uniform in
    [0.0002, 0.002] per output column."""
    rng = np.random.default_rng(seed)
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.size
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    rows = int(offsets[-1]) + tail
    a = rng.integers(-127, 128, size=(rows, Kd), dtype=np.int8)
    a_sc = rng.uniform(0.002, 0.05, size=(rows, Kd // 128) if per_tile else (rows,))
    w = rng.integers(-127, 128, size=(E, N, Kd), dtype=np.int8)
    w_sc = rng.uniform(0.0002, 0.002, size=(E, N))
    return GemmCaseI8(name, E, N, Kd, rows, offsets, a, a_sc.astype(np.float32), w,
                      w_sc.astype(np.float32))


def make_g3(seed: int = 3100) -> GemmCase:
    rng = np.random.default_rng(seed)
    counts = zipf_counts(rng, 4096, 8, 1.2)
    return make_gemm_case(seed + 1, counts, 4096, 7168, name="g3")
