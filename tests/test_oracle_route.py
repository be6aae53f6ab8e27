"""Pins for the oracle's routing (histogram, exclusive scan, stable rank) and
expert mapping / pruning (CPU only).

Routing is checked against an O(N^2) brute-force rank (the number of active
entries that come before an entry in (instance, flat index) order), against
numpy's bincount / cumsum / stable argsort, and against invariants
(counts sum to Bs*K minus pruned entries; src and assist are inverse; every
row block holds its own instance in ascending flat index).

Mapping ("aclnnMoeUpdateExpert") is checked against special cases that
reduce to a plain gather (identity table, one replica per expert), the
round-robin balance of replicas, pruning limits and the mask rules of
"aclnnMoeDistributeDispatchV2" (1-D mask true-then-false, 2-D mask prunes
per entry).
"""
import numpy as np
import pytest

import oracle
from combine_expert_amd import workloads as W


def brute_route(ids, mask, E):
    ids = np.asarray(ids).reshape(-1)
    N = ids.size
    act = [bool(mask is None or np.asarray(mask).reshape(-1)[f]) and 0 <= ids[f] < E
           for f in range(N)]
    counts = [sum(1 for f in range(N) if act[f] and ids[f] == e) for e in range(E)]
    assist = []
    for f in range(N):
        if not act[f]:
            assist.append(-1)
            continue
        assist.append(sum(1 for g in range(N)
                          if act[g] and (ids[g], g) < (ids[f], f)))
    return np.array(counts), np.array(assist)


def check_invariants(ids, mask, E, counts, offsets, assist, src):
    ids = np.asarray(ids).reshape(-1)
    N = ids.size
    act = np.ones(N, bool) if mask is None else np.asarray(mask).reshape(-1).astype(bool)
    act &= (ids >= 0) & (ids < E)
    total = int(offsets[E])
    assert counts.sum() == N - (~act).sum() == total
    assert offsets[0] == 0 and np.all(np.diff(offsets) == counts)
    assert np.all(src[total:] == -1)
    assert np.all(assist[~act] == -1)
    f_act = np.nonzero(act)[0]
    assert np.all(src[assist[f_act]] == f_act)
    for e in range(E):
        blk = src[offsets[e]:offsets[e + 1]]
        assert np.all(ids[blk] == e)
        assert np.all(np.diff(blk) > 0)


@pytest.mark.parametrize("seed", range(12))
def test_route_vs_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    Bs = int(rng.integers(1, 9))
    K = int(rng.integers(1, 5))
    E = int(rng.integers(1, 9))
    ids = rng.integers(0, E, size=(Bs, K)).astype(np.int32)  # duplicates allowed
    mask = (rng.random((Bs, K)) < 0.7).astype(np.uint8) if seed % 2 else None
    counts, offsets, assist, src, err = oracle.route(ids, mask, E)
    bc, ba = brute_route(ids, mask, E)
    np.testing.assert_array_equal(counts, bc)
    np.testing.assert_array_equal(assist, ba)
    assert err == 0
    check_invariants(ids, mask, E, counts, offsets, assist, src)


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_route_vs_numpy_library(name):
    wl = W.make(name)
    ids = wl.logical_ids.numpy()
    E = wl.E
    counts, offsets, assist, src, err = oracle.route(ids, None, E)
    flat = ids.reshape(-1)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    order = np.argsort(flat, kind="stable")
    np.testing.assert_array_equal(src, order)
    check_invariants(ids, None, E, counts, offsets, assist, src)


def test_route_with_pruning_vs_stable_argsort():
    rng = np.random.default_rng(77)
    Bs, K, E = 300, 16, 1024
    ids = rng.integers(0, E, size=(Bs, K)).astype(np.int32)
    mask = (rng.random((Bs, K)) < 0.35).astype(np.uint8)
    counts, offsets, assist, src, err = oracle.route(ids, mask, E)
    key = np.where(mask.reshape(-1) != 0, ids.reshape(-1), E)
    order = np.argsort(key, kind="stable")
    total = int(mask.sum())
    np.testing.assert_array_equal(src[:total], order[:total])
    check_invariants(ids, mask, E, counts, offsets, assist, src)


def test_route_edge_cases():
    # everything pruned
    ids = np.zeros((4, 2), np.int32)
    counts, offsets, assist, src, err = oracle.route(ids, np.zeros((4, 2), np.uint8), 3)
    assert not counts.any() and not offsets.any()
    assert np.all(assist == -1) and np.all(src == -1)
    # one expert takes everything, in flat order
    counts, offsets, assist, src, err = oracle.route(ids, None, 1)
    assert list(counts) == [8] and list(src) == list(range(8)) and list(assist) == list(range(8))
    # an active id out of range is flagged and dropped; an inactive one is not flagged
    ids = np.array([[0, 5], [1, -1]], np.int32)
    counts, offsets, assist, src, err = oracle.route(ids, None, 2)
    assert err == 1 and list(assist) == [0, -1, 1, -1]
    counts, offsets, assist, src, err = oracle.route(ids, np.array([[1, 0], [1, 0]], np.uint8), 2)
    assert err == 0 and list(assist) == [0, -1, 1, -1]


def test_route_worked_example():
    # Bs=3, K=2, E=3; ids [[2,0],[0,2],[1,0]]; mask drops (1,1).
    # counts: e0 -> f=1,2,5 (3); e1 -> f=4 (1); e2 -> f=0 (f=3 pruned) (1)
    # offsets [0,3,4,5]; rows: 0:f1 1:f2 2:f5 3:f4 4:f0
    ids = np.array([[2, 0], [0, 2], [1, 0]], np.int32)
    mask = np.array([[1, 1], [1, 0], [1, 1]], np.uint8)
    counts, offsets, assist, src, err = oracle.route(ids, mask, 3)
    assert list(counts) == [3, 1, 1]
    assert list(offsets) == [0, 3, 4, 5]
    assert list(assist) == [4, 0, 1, -1, 3, 2]
    assert list(src) == [1, 2, 5, 4, 0, -1]


# ---------------------------------------------------------------- mapping / pruning

def test_update_identity_table_is_identity():
    wl = W.make("c3")
    ids = wl.logical_ids.numpy()
    out, m, err = oracle.update_expert(ids, None, wl.table.numpy(), None, None, wl.E)
    np.testing.assert_array_equal(out, ids)
    assert m.all() and err == 0


def test_update_single_replica_is_gather():
    rng = np.random.default_rng(3)
    n_log, n_inst = 40, 64
    inst = rng.permutation(n_inst)[:n_log].astype(np.int32)
    table = np.stack([np.ones(n_log, np.int32), inst], axis=1)
    ids = rng.integers(0, n_log, size=(50, 6)).astype(np.int32)
    out, m, err = oracle.update_expert(ids, None, table, None, None, n_inst)
    np.testing.assert_array_equal(out, inst[ids])
    assert m.all() and err == 0


def test_update_replicas_round_robin_balance():
    # every token picks logical expert 0, which has 3 replicas {7, 2, 9}:
    # token i uses replica i mod 3, so each replica gets Bs/3 tokens and
    # tokens i, i+3, i+6 ... share a replica.
    table = np.array([[3, 7, 2, 9], [1, 0, -1, -1]], np.int32)
    Bs = 30
    ids = np.zeros((Bs, 1), np.int32)
    out, m, err = oracle.update_expert(ids, None, table, None, None, 10)
    assert err == 0
    assert np.array_equal(np.bincount(out[:, 0], minlength=10)[[7, 2, 9]], [10, 10, 10])
    assert np.all(out[:-3, 0] == out[3:, 0])
    assert len({int(out[0, 0]), int(out[1, 0]), int(out[2, 0])}) == 3
    assert out[0, 0] == 7  # the first token takes the first listed instance


def test_update_c4_replicas_and_pruning():
    wl = W.make("c4")
    ids, sc, table, thr = (wl.logical_ids.numpy(), wl.scales.numpy(), wl.table.numpy(),
                           wl.prune_thr.numpy())
    out, m, err = oracle.update_expert(ids, sc, table, thr, None, wl.E)
    assert err == 0
    # every chosen instance is one of the logical expert's replicas
    for i in range(0, wl.Bs, 17):
        for k in range(wl.K):
            e = ids[i, k]
            assert out[i, k] in table[e, 1:1 + table[e, 0]]
    # pruning limits: threshold 0 keeps all, +inf prunes all
    _, m0, _ = oracle.update_expert(ids, sc, table, np.zeros(wl.K, np.float32), None, wl.E)
    _, mi, _ = oracle.update_expert(ids, sc, table, np.full(wl.K, np.inf, np.float32), None,
                                    wl.E)
    assert m0.all() and not mi.any()
    # monotone in the threshold, and the kept set is exactly score >= thr
    assert np.all(m <= m0)
    kept_scores = sc[m.astype(bool)]
    assert kept_scores.min() >= 0.02 and sc[~m.astype(bool)].max() < 0.02
    frac = 1.0 - m.mean()
    assert 0.5 < frac < 0.8  # the c4 workload prunes about two thirds of its entries


def test_update_nan_score_is_kept_and_token_mask():
    table = W.identity_table(4)
    ids = np.array([[0, 1], [2, 3], [1, 0]], np.int32)
    sc = np.array([[np.nan, 0.01], [0.5, 0.5], [0.5, 0.5]], np.float32)
    thr = np.array([0.1, 0.1], np.float32)
    out, m, err = oracle.update_expert(ids, sc, table, thr, None, 4)
    assert m.tolist() == [[1, 0], [1, 1], [1, 1]]
    # a score equal to the threshold is not below it: kept
    at = np.array([[0.1, 0.1], [0.5, np.nextafter(np.float32(0.1), np.float32(0))],
                   [0.5, 0.5]], np.float32)
    _, m, _ = oracle.update_expert(ids, at, table, thr, None, 4)
    assert m.tolist() == [[1, 1], [1, 0], [1, 1]]
    tm = np.array([1, 1, 0], np.uint8)
    out, m, err = oracle.update_expert(ids, sc, table, thr, tm, 4)
    assert m.tolist() == [[1, 0], [1, 1], [0, 0]] and err == 0
    # {true, false, true} is not a legal 1-D mask: flagged, still applied
    tm = np.array([1, 0, 1], np.uint8)
    out, m, err = oracle.update_expert(ids, None, table, None, tm, 4)
    assert err == 4 and m.tolist() == [[1, 1], [0, 0], [1, 1]]


def test_update_error_bits():
    table = np.array([[1, 0, -1], [0, 1, -1], [2, 1, 5]], np.int32)
    # id 3 out of range (bit 1); expert 1 has count 0 (bit 2); expert 2 replica
    # for odd tokens is instance 5 >= 4 (bit 2)
    ids = np.array([[3], [1], [2], [2]], np.int32)
    out, m, err = oracle.update_expert(ids, None, table, None, None, 4)
    assert err == 3
    assert out[:, 0].tolist() == [-1, -1, 1, -1]
    assert m[:, 0].tolist() == [0, 0, 1, 0]
    # the same failures on entries that are pruned anyway raise nothing
    out, m, err = oracle.update_expert(ids, None, table, None, np.zeros(4, np.uint8), 4)
    assert err == 0 and not m.any()
