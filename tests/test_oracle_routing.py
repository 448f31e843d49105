"""Pins for the oracle's router projection and top-k routing.

Checked against brute force over every k-subset, closed forms (two-expert
softmax, sigmoid), hand-worked examples and invariants: unique indices,
descending order, weights summing to the routed scaling factor, every selected
score above every unselected one.
"""

import itertools
import math

import numpy as np
import pytest

from oracle import route, router_logits, selection_scores


def _rng(s):
    return np.random.default_rng(s)


def test_router_one_hot_picks_columns():
    wr = _rng(0).standard_normal((5, 7))
    x = np.eye(7)[[2, 6]]
    np.testing.assert_array_equal(router_logits(x, wr), wr[:, [2, 6]].T)


def test_router_matches_loop():
    g = _rng(1)
    x = g.standard_normal((3, 9))
    wr = g.standard_normal((4, 9))
    z = router_logits(x, wr)
    for t in range(3):
        for e in range(4):
            assert math.isclose(z[t, e], sum(x[t, h] * wr[e, h] for h in range(9)),
                                rel_tol=1e-13, abs_tol=1e-13)


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("E,k", [(6, 1), (6, 3), (8, 4), (7, 7)])
def test_topk_set_is_best_subset_brute_force(scoring, E, k):
    g = _rng(E * 10 + k)
    z = g.standard_normal((5, E))
    bias = g.standard_normal(E) * 0.3 if scoring == "sigmoid" else None
    idx, _ = route(z, k, scoring, bias)
    s = selection_scores(z, scoring, bias)
    for t in range(5):
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(s[t, list(c)]))
        assert sorted(idx[t].tolist()) == sorted(best)
        # descending score order
        assert all(s[t, idx[t, j]] > s[t, idx[t, j + 1]] for j in range(k - 1))


def test_lowest_index_wins_ties():
    z = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    idx, _ = route(z, 2, "softmax", renorm=False)
    assert idx.tolist() == [[1, 2]]
    idx, _ = route(z, 4, "softmax", renorm=False)
    assert idx.tolist() == [[1, 2, 4, 3]]


def test_softmax_two_experts_closed_form():
    z = np.array([[0.3, -1.1]])
    idx, w = route(z, 1, "softmax", renorm=False)
    assert idx.tolist() == [[0]]
    assert math.isclose(w[0, 0], 1.0 / (1.0 + math.exp(-1.4)), rel_tol=1e-14)


def test_softmax_renorm_hand_worked():
    # z = ln(1..4): softmax p = (0.1, 0.2, 0.3, 0.4); top-2 = experts 3, 2;
    # renormalised weights 4/7 and 3/7; without renorm 0.4 and 0.3.
    z = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))
    idx, w = route(z, 2, "softmax", renorm=True)
    assert idx.tolist() == [[3, 2]]
    np.testing.assert_allclose(w[0], [4 / 7, 3 / 7], rtol=1e-14)
    idx, w = route(z, 2, "softmax", renorm=False)
    np.testing.assert_allclose(w[0], [0.4, 0.3], rtol=1e-14)
    # the routed scaling factor multiplies after renormalisation
    idx, w = route(z, 2, "softmax", renorm=True, rsf=2.5)
    np.testing.assert_allclose(w[0], [2.5 * 4 / 7, 2.5 * 3 / 7], rtol=1e-14)


def test_softmax_shift_invariant():
    z = _rng(4).standard_normal((3, 16))
    i0, w0 = route(z, 4, "softmax", renorm=False)
    i1, w1 = route(z + 7.25, 4, "softmax", renorm=False)
    assert np.array_equal(i0, i1)
    np.testing.assert_allclose(w0, w1, rtol=1e-13)


def test_sigmoid_bias_selects_but_does_not_weigh():
    z = np.array([[2.0, 1.0, 0.0, -1.0]])
    bias = np.array([0.0, 0.0, 0.0, 5.0])       # drags expert 3 into the top 2
    idx, w = route(z, 2, "sigmoid", bias, renorm=False, rsf=1.0)
    assert idx.tolist() == [[3, 0]]
    sig = lambda v: 1.0 / (1.0 + math.exp(-v))
    np.testing.assert_allclose(w[0], [sig(-1.0), sig(2.0)], rtol=1e-14)
    idx, w = route(z, 2, "sigmoid", bias, renorm=True, rsf=2.5)
    tot = sig(-1.0) + sig(2.0)
    np.testing.assert_allclose(w[0], [2.5 * sig(-1.0) / tot, 2.5 * sig(2.0) / tot],
                               rtol=1e-14)


def test_sigmoid_spot_values():
    s = selection_scores(np.array([[0.0, 40.0, -40.0]]), "sigmoid")
    assert s[0, 0] == 0.5
    assert math.isclose(s[0, 1], 1.0, rel_tol=1e-15)
    assert s[0, 2] < 1e-17


@pytest.mark.parametrize("scoring,rsf", [("softmax", 1.0), ("sigmoid", 2.5)])
def test_invariants(scoring, rsf):
    g = _rng(7)
    E, k = 64, 8
    z = g.standard_normal((16, E))
    bias = g.standard_normal(E) * 0.1 if scoring == "sigmoid" else None
    idx, w = route(z, k, scoring, bias, renorm=True, rsf=rsf)
    s = selection_scores(z, scoring, bias)
    for t in range(16):
        assert len(set(idx[t].tolist())) == k
        np.testing.assert_allclose(w[t].sum(), rsf, rtol=1e-12)
        mask = np.ones(E, bool)
        mask[idx[t]] = False
        assert s[t, idx[t]].min() > s[t, mask].max()
        assert (w[t] > 0).all()


def test_no_renorm_softmax_weights_are_probabilities():
    z = _rng(9).standard_normal((2, 10))
    idx, w = route(z, 10, "softmax", renorm=False)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-13)
