"""Pins for oracle.plan_ref: a brute-force per-expert scan, and the invariants
that the route plan packs pairs by expert without changing the token-to-expert
mapping ("Optimization progress report", Optimization 14)."""

import numpy as np
import pytest

from oracle.moe import plan_ref
from synth import WORKLOADS, make_routing


def brute_plan(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    order = []
    offsets = [0]
    for e in range(E):
        for p, v in enumerate(flat):
            if v == e:
                order.append(p)
        offsets.append(len(order))
    return offsets, order


def check_invariants(ids, E, r):
    flat = np.asarray(ids).reshape(-1)
    P = flat.size
    off, sp, pr = r["expert_offsets"], r["sorted_pairs"], r["pair_rows"]
    n = int(off[-1])
    valid = (flat >= 0) & (flat < E)
    assert n == valid.sum() == P - r["dropped"]
    assert np.all(np.diff(off) >= 0) and off[0] == 0
    assert np.array_equal(np.diff(off), np.bincount(flat[valid], minlength=E))
    assert sorted(sp[:n].tolist()) == sorted(np.nonzero(valid)[0].tolist())   # a permutation of the valid pairs
    assert np.all(sp[n:] == -1)
    assert np.array_equal(pr[sp[:n]], np.arange(n))                           # inverse
    assert np.all(pr[~valid] == -1)
    e_along = flat[sp[:n]]
    assert np.all(np.diff(e_along) >= 0)                                     # grouped by expert
    for e in range(E):                                                       # stable in p
        seg = sp[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(flat[seg] == e)                                        # mapping unchanged


@pytest.mark.parametrize("T,K,E,seed", [(1, 1, 1, 0), (7, 8, 384, 1), (64, 2, 8, 2), (300, 4, 5, 3),
                                        (33, 8, 40, 4)])
def test_plan_matches_bruteforce(T, K, E, seed):
    ids = np.random.default_rng(seed).integers(0, E, (T, K))
    r = plan_ref(ids, E)
    off, order = brute_plan(ids, E)
    assert r["expert_offsets"].tolist() == off
    assert r["sorted_pairs"][:off[-1]].tolist() == order
    check_invariants(ids, E, r)


def test_plan_drops_invalid_ids():
    ids = np.array([[0, 5], [-1, 2], [2, 2], [7, 1]])
    r = plan_ref(ids, 3)
    assert r["dropped"] == 3
    assert r["expert_offsets"].tolist() == [0, 1, 2, 5]
    assert r["sorted_pairs"].tolist() == [0, 7, 3, 4, 5, -1, -1, -1]
    check_invariants(ids, 3, r)


def test_plan_empty():
    r = plan_ref(np.zeros((0, 8), dtype=np.int32), 16)
    assert r["expert_offsets"].tolist() == [0] * 17 and r["sorted_pairs"].size == 0


@pytest.mark.parametrize("name", ["tiny", "decode7", "decode256"])
def test_plan_on_workloads(name):
    w = WORKLOADS[name]
    ids, _ = make_routing(w)
    check_invariants(ids, w.E, plan_ref(ids, w.E))
