"""Pins of the oracle's grouping of routing slots by expert.

The pages print no worked example of the grouping, so it is pinned by a
hand-derived case (tests/golden), by invariants that any stable, padded
grouping must satisfy, and by NumPy's stable argsort as an independent sort.
"""

import json
import os

import numpy as np
import pytest

from oracle import group_slots

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_derived_example():
    g = json.load(open(os.path.join(GOLDEN, "grouping_n3_k2_e3_pad4.json")))
    r = group_slots(np.array(g["idx"]), g["num_experts"], pad=g["pad"])
    for key in ("counts", "offsets", "perm_slot", "perm_tok", "inv", "units"):
        assert r[key].tolist() == g[key], key


def _random_idx(rng, n, k, e, skew):
    p = rng.dirichlet(np.full(e, skew))
    return np.stack([rng.choice(e, size=k, replace=False, p=p) for _ in range(n)])


@pytest.mark.parametrize("n,k,e,skew", [(1, 1, 1, 1.0), (5, 2, 8, 1.0), (17, 4, 16, 0.2),
                                        (64, 8, 128, 0.05), (200, 8, 32, 5.0), (33, 16, 16, 1.0)])
def test_invariants(n, k, e, skew):
    rng = np.random.default_rng(n * 1000 + k * 10 + e)
    idx = _random_idx(rng, n, k, e, skew)
    r = group_slots(idx, e, pad=16)
    flat = idx.reshape(-1)
    counts, off, ps, pt, inv = r["counts"], r["offsets"], r["perm_slot"], r["perm_tok"], r["inv"]
    assert counts.sum() == n * k
    assert np.array_equal(counts, np.bincount(flat, minlength=e))
    assert off[0] == 0 and np.all(off % 16 == 0)
    width = np.diff(off)
    assert np.all(width >= counts) and np.all(width < counts + 16)
    assert np.all(width[counts == 0] == 0)
    real = ps >= 0
    # every slot exactly once, inv is the inverse map, tokens match slots
    assert sorted(ps[real].tolist()) == list(range(n * k))
    assert np.array_equal(inv[ps[real]], np.nonzero(real)[0])
    assert np.array_equal(pt[real], ps[real] // k)
    assert np.all(pt[~real] == -1)
    for ex in range(e):
        rows = np.arange(off[ex], off[ex + 1])
        # real rows first, then padding; all of this expert; slots ascending
        assert np.all(real[rows[:counts[ex]]]) and not np.any(real[rows[counts[ex]:]])
        s = ps[rows[:counts[ex]]]
        assert np.all(flat[s] == ex)
        assert np.all(np.diff(s) > 0)
        # a token routes to an expert at most once, so tokens are ascending too
        assert np.all(np.diff(pt[rows[:counts[ex]]]) > 0)
    assert np.array_equal(r["units"], np.nonzero(counts)[0])


def test_matches_stable_argsort():
    rng = np.random.default_rng(5)
    idx = _random_idx(rng, 300, 8, 64, 0.3)
    r = group_slots(idx, 64, pad=16)
    order = np.argsort(idx.reshape(-1), kind="stable")
    ps = r["perm_slot"]
    assert np.array_equal(ps[ps >= 0], order)


@pytest.mark.parametrize("lo,hi", [(0, 1), (3, 11), (8, 16), (0, 16)])
def test_share_grouping_is_the_full_one_restricted(lo, hi):
    # a share's grouping keeps, expert by expert, exactly the slots (in the
    # same order) that the full grouping puts under that expert
    rng = np.random.default_rng(lo * 100 + hi)
    n, k, e = 37, 4, 16
    idx = _random_idx(rng, n, k, e, 0.5)
    full = group_slots(idx, e, pad=16)
    part = group_slots(idx, e, pad=16, expert_range=(lo, hi))
    flat = idx.reshape(-1)
    local = (flat >= lo) & (flat < hi)
    assert np.array_equal(part["counts"], full["counts"][lo:hi])
    assert np.array_equal(part["units"], full["units"][(full["units"] >= lo)
                                                       & (full["units"] < hi)] - lo)
    assert (part["inv"][~local] == -1).all()
    for el in range(hi - lo):
        seg_p = part["perm_slot"][part["offsets"][el]:part["offsets"][el + 1]]
        seg_f = full["perm_slot"][full["offsets"][lo + el]:full["offsets"][lo + el + 1]]
        assert np.array_equal(seg_p, seg_f)
        assert part["offsets"][el] % 16 == 0
    s = np.nonzero(local)[0]
    assert np.array_equal(part["perm_slot"][part["inv"][s]], s)
    assert np.array_equal(part["perm_tok"][part["inv"][s]], s // k)
