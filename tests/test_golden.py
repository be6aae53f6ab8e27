"""Checks driven by the values the operator pages print (tests/golden/).

The pages print no worked numerical example of the operators' outputs, only
ranges, a mask-legality example and the quantisation mode list; those are
kept in tests/golden/page_constraints.json with their citations.
"""
import json
import os

import numpy as np

import oracle
from combine_expert_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constraints.json")


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_illegal_1d_mask_example_is_flagged():
    g = load()["dispatch_mask"]
    tm = np.array(g["illegal_example"], dtype=np.uint8)
    Bs = tm.size
    ids = np.zeros((Bs, 1), np.int32)
    _, m, err = oracle.update_expert(ids, None, W.identity_table(1), None, tm, 1)
    assert err & 4
    # a legal prefix mask of the same length raises nothing
    _, m, err = oracle.update_expert(ids, None, W.identity_table(1), None,
                                     np.array([1, 1, 0], np.uint8), 1)
    assert err == 0 and m[:, 0].tolist() == [1, 1, 0]


def test_workloads_respect_page_shapes():
    g = load()
    cs, us = g["combine_shapes"], g["update_expert_shapes"]
    for name in ("c1", "c2", "c3", "c4", "c4b"):
        wl = W.make(name)
        assert cs["H"]["min"] <= wl.H <= cs["H"]["max"]
        assert 0 < wl.Bs <= cs["Bs"]["max"]
        assert 0 < wl.K <= cs["K"]["max"] and wl.K <= wl.n_logical
        assert 0 < wl.n_logical <= us["moeExpertNum"]["max"]
        assert wl.E <= us["total_instances_max"]
        assert us["F"]["min"] <= wl.F <= wl.n_logical + 1
        t = wl.table.numpy()
        assert np.all(t[:, 0] > 0) and np.all(t[:, 0] <= wl.F - 1)
