"""Pins of the oracle's routing variants: the softmax+bias arm, hash routing
and zero experts ("forward_batched.rs": router_bias_one, the hash-routing
branch, the router width num_experts + zero_expert_num).

The pages print no values for these, so each is pinned by a closed form
worked by hand, by brute force over subsets, or by reduction to an already
pinned case (plain top-k routing; a layer whose extra experts have zero
down weights).
"""

import itertools
import math

import numpy as np
import pytest

import synth
from oracle import (moe_forward, route, route_hash, routing_weights, selection_scores,
                    softmax_rows)


def test_softmax_bias_closed_form():
    # z = [0, ln 2, 0]: p = [1/4, 1/2, 1/4]; b = [0.3, 0, 0.2] gives scores
    # [0.55, 0.5, 0.45]: the bias moves the choice from expert 1 to expert 0,
    # whose weight stays the unbiased p = 1/4 (times rsf, no renorm)
    z = np.array([[0.0, math.log(2.0), 0.0]])
    b = np.array([0.3, 0.0, 0.2])
    s = selection_scores(z, "softmax", b)
    np.testing.assert_allclose(s, [[0.55, 0.5, 0.45]], rtol=0, atol=1e-15)
    idx, w = route(z, 1, "softmax", b, renorm=False, rsf=2.0)
    assert idx.tolist() == [[0]] and abs(w[0, 0] - 0.5) < 1e-15
    idx0, _ = route(z, 1, "softmax", None, renorm=False)
    assert idx0.tolist() == [[1]]
    # top-2 with renorm: experts 0 and 1, weights 1/4 and 1/2 renormalised
    idx, w = route(z, 2, "softmax", b, renorm=True, rsf=1.0)
    assert idx.tolist() == [[0, 1]]
    np.testing.assert_allclose(w, [[1 / 3, 2 / 3]], rtol=1e-15)


def test_softmax_bias_zero_bias_is_plain_softmax():
    rng = np.random.default_rng(5)
    z = rng.normal(size=(20, 24))
    a = route(z, 5, "softmax", np.zeros(24), True, 1.5)
    b = route(z, 5, "softmax", None, True, 1.5)
    assert np.array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1], b[1], rtol=1e-15)


def test_softmax_bias_selection_is_best_subset():
    # the chosen set is the k-subset with the largest sum of p + b (scores
    # distinct), found here by enumerating every subset
    rng = np.random.default_rng(6)
    for _ in range(20):
        z = rng.normal(size=(1, 7))
        b = rng.normal(scale=0.1, size=7)
        p = softmax_rows(z)[0]
        best = max(itertools.combinations(range(7), 3), key=lambda c: sum(p[i] + b[i] for i in c))
        idx, _ = route(z, 3, "softmax", b)
        assert sorted(idx[0].tolist()) == sorted(best)


def test_hash_closed_form():
    # two tokens, table rows [2, 0] and [1, 3]; softmax over all 4 logits
    z = np.array([[0.0, 0.0, math.log(3.0), 0.0],
                  [math.log(2.0), 0.0, 0.0, math.log(2.0)]])
    table = np.array([[0, 1], [2, 0], [1, 3]])
    idx, w = route_hash(z, table, [1, 2], 2, "softmax", renorm=False, rsf=1.0)
    assert idx.tolist() == [[2, 0], [1, 3]]
    np.testing.assert_allclose(w, [[3 / 6, 1 / 6], [1 / 6, 2 / 6]], rtol=1e-15)
    # sigmoid: the chosen logits' sigmoid, renormalised, times rsf
    idx, w = route_hash(z[:1], table, [1], 2, "sigmoid", renorm=True, rsf=2.0)
    s2, s0 = 1 / (1 + 1 / 3), 0.5
    np.testing.assert_allclose(w, [[2 * s2 / (s2 + s0), 2 * s0 / (s2 + s0)]], rtol=1e-15)


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_hash_with_the_topk_table_is_topk(scoring):
    # a table that lists each token's own top-k experts reproduces top-k
    # routing exactly (bias-free, so both rules weigh the same experts alike)
    rng = np.random.default_rng(7)
    z = rng.normal(size=(9, 32))
    idx, w = route(z, 6, scoring, None, True, 1.7)
    table = idx.copy()
    hidx, hw = route_hash(z, table, np.arange(9), 6, scoring, True, 1.7)
    assert np.array_equal(hidx, idx)
    np.testing.assert_allclose(hw, w, rtol=1e-15)


def _zero_expert_layer(Z):
    cfg = synth.reduced("tiny_bf16", E=6, k=3, Z=Z, bias_std=0.05, name=f"z{Z}")
    return synth.as_numpy(synth.make_layer(cfg))


def test_zero_experts_equal_experts_with_zero_down():
    # a zero expert is exactly an expert whose down projection is zero: give
    # the same router (E + Z rows) real experts E..E+Z-1 with zero down
    # weights and compare the whole layer
    npl = _zero_expert_layer(3)
    cfg = npl["cfg"]
    E, Z = cfg["E"], cfg["Z"]
    x = synth.make_tokens(synth.make_layer(cfg), 11, 3).view(__import__("torch").int16).numpy()
    x = x.view(np.uint16)
    ref = moe_forward(cfg, npl, x)
    assert (ref["idx"] >= E).any(), "no token chose a zero expert"
    wide = {k: dict(v) for k, v in npl["experts"].items()}
    for name in ("gate", "up", "down"):
        p = wide[name]
        extra = np.zeros((Z,) + p["data"].shape[1:], dtype=p["data"].dtype)
        if name != "down":
            extra = p["data"][:Z]  # any values: the zero down cancels them
        p["data"] = np.concatenate([p["data"], extra])
        p["count"] = E + Z
    cfg2 = dict(cfg, E=E + Z, Z=0)
    npl2 = dict(npl, experts=wide)
    ref2 = moe_forward(cfg2, npl2, x)
    assert np.array_equal(ref["idx"], ref2["idx"])
    np.testing.assert_allclose(ref["y"], ref2["y"], rtol=1e-12, atol=1e-15)


def test_zero_experts_count_in_renormalisation():
    # weights of a token's slots sum to rsf with renorm, zero slots included
    npl = _zero_expert_layer(2)
    cfg = npl["cfg"]
    x = synth.make_tokens(synth.make_layer(cfg), 8, 4).view(__import__("torch").int16).numpy()
    ref = moe_forward(cfg, npl, x.view(np.uint16))
    np.testing.assert_allclose(ref["w"].sum(axis=1), cfg["rsf"], rtol=1e-12)
    z = ref["z"]
    assert z.shape[1] == cfg["E"] + cfg["Z"]
    for t in range(8):
        np.testing.assert_allclose(
            ref["w"][t], routing_weights(z[t], ref["idx"][t], cfg["scoring"], True, cfg["rsf"]),
            rtol=1e-15)


# ---- NVFP4 router ------------------------------------------------------------

@pytest.mark.parametrize("mult", [1.0, 0.5])
def test_nvfp4_router_equals_bf16_router_of_its_values(mult):
    # with a power-of-two tensor scale every dequantised router weight (an
    # E2M1 value times an E4M3 scale: at most 6 significant bits) is a BF16
    # value, so a BF16 router holding those values must route and compute
    # exactly alike
    import torch
    from oracle import dequant
    cfg = synth.reduced("deepseek_v3_nvfp4", H=256, I=64, E=16, k=4, I_s=64, Z=2,
                        router_fmt="nvfp4", name="nvfp4_router_pin")
    npl = synth.as_numpy(synth.make_layer(cfg))
    q = npl["router"]["weight_q"]
    # the nearest power of two to the quantiser's own tensor scale
    ts0 = float(q["tensor_scale"][0])
    q["tensor_scale"] = np.full_like(q["tensor_scale"], mult * 2.0 ** round(math.log2(ts0)))
    w = dequant(q, 0)
    wb = torch.from_numpy(w).to(torch.bfloat16)
    assert np.array_equal(wb.double().numpy(), w), "values not BF16-exact"
    bf = dict(npl)
    bf["router"] = dict(npl["router"], weight=wb.view(torch.int16).numpy().view(np.uint16),
                        weight_q=None)
    x = synth.make_tokens(synth.make_layer(cfg), 6, 9).view(torch.int16).numpy().view(np.uint16)
    a = moe_forward(cfg, npl, x)
    b = moe_forward(cfg, bf, x)
    assert np.array_equal(a["z"], b["z"])
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["y"], b["y"])
