"""Pins for the oracle's expert and whole-layer arithmetic.

Closed forms (one-by-one SwiGLU, silu against SciPy's expit), special cases
(dense MoE with E = k, a single expert, zero routed down weights, zero gate),
invariants (token independence, expert relabelling, linearity in the down
weights) and a pure-Python brute-force layer on tiny shapes that decodes the
weights through torch's own dtype conversions.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import dequant, moe_forward, silu, swiglu_expert


def test_silu_matches_scipy_expit():
    v = np.linspace(-30, 30, 2001)
    np.testing.assert_allclose(silu(v), v * scipy.special.expit(v), rtol=1e-14, atol=1e-300)
    assert silu(0.0) == 0.0


def test_swiglu_one_by_one_closed_form():
    a, b, c, v = 0.7, -1.3, 2.2, 0.9
    _, _, act, d = swiglu_expert(np.array([[a]]), np.array([[b]]), np.array([[c]]),
                                 np.array([v]))
    g = a * v
    want = c * (g / (1.0 + math.exp(-g))) * (b * v)
    assert math.isclose(d[0], want, rel_tol=1e-15)
    assert math.isclose(act[0], want / c, rel_tol=1e-15)


def test_zero_gate_gives_zero_activation():
    g = np.random.default_rng(0)
    x = g.standard_normal(6)
    _, _, act, d = swiglu_expert(np.zeros((3, 6)), g.standard_normal((3, 6)),
                                 g.standard_normal((4, 3)), x)
    assert not act.any() and not d.any()


def _layer(cfg_over, base="tiny_bf16"):
    cfg = synth.reduced(base, **cfg_over)
    layer = synth.make_layer(cfg)
    return layer, synth.as_numpy(layer)


def _bf16_bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def test_token_independence():
    layer, npl = _layer(dict(H=64, I=32, E=6, k=2, I_s=16))
    x = synth.make_tokens(layer, 5, 1)
    full = moe_forward(npl["cfg"], npl, _bf16_bits(x))
    for t in range(5):
        one = moe_forward(npl["cfg"], npl, _bf16_bits(x[t:t + 1]))
        # the same arithmetic per token; BLAS may order the sums differently
        # for one token than for a batch, so equal up to FP64 rounding
        np.testing.assert_allclose(one["y"][0], full["y"][t], rtol=1e-12, atol=1e-18)
        np.testing.assert_array_equal(one["idx"][0], full["idx"][t])


def test_expert_relabelling_is_equivariant():
    layer, npl = _layer(dict(H=64, I=32, E=6, k=3, I_s=0))
    x = _bf16_bits(synth.make_tokens(layer, 4, 2))
    ref = moe_forward(npl["cfg"], npl, x)
    perm = np.array([4, 0, 5, 2, 1, 3])          # new expert i = old perm[i]
    p2 = dict(npl)
    p2["router"] = {"weight": npl["router"]["weight"][perm], "bias": None}
    p2["experts"] = {k: dict(v, data=v["data"][perm]) for k, v in npl["experts"].items()}
    out = moe_forward(npl["cfg"], p2, x)
    np.testing.assert_allclose(out["y"], ref["y"], rtol=1e-13, atol=1e-15)
    assert np.array_equal(perm[out["idx"]], ref["idx"])


def test_dense_moe_equals_probability_mixture():
    # E = k with renormalisation: every expert is used with its full-softmax
    # probability, so y = sum_e p_e d_e.
    layer, npl = _layer(dict(H=32, I=16, E=4, k=4, I_s=0))
    x = _bf16_bits(synth.make_tokens(layer, 3, 3))
    out = moe_forward(npl["cfg"], npl, x)
    xf = x.astype(np.uint32) << 16
    xf = xf.view(np.float32).astype(np.float64)
    wr = (npl["router"]["weight"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ex = npl["experts"]
    for t in range(3):
        z = wr @ xf[t]
        p = np.exp(z - z.max())
        p /= p.sum()
        y = np.zeros(32)
        for e in range(4):
            _, _, _, d = swiglu_expert(dequant(ex["gate"], e), dequant(ex["up"], e),
                                       dequant(ex["down"], e), xf[t])
            y += p[e] * d
        np.testing.assert_allclose(out["y"][t], y, rtol=1e-12, atol=1e-15)


def test_single_expert_layer_is_that_expert():
    layer, npl = _layer(dict(H=32, I=16, E=1, k=1, I_s=0))
    x = _bf16_bits(synth.make_tokens(layer, 2, 4))
    out = moe_forward(npl["cfg"], npl, x)
    assert np.array_equal(out["w"], np.ones((2, 1)))
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ex = npl["experts"]
    for t in range(2):
        _, _, _, d = swiglu_expert(dequant(ex["gate"], 0), dequant(ex["up"], 0),
                                   dequant(ex["down"], 0), xf[t])
        # equal up to FP64 rounding (one token against a batched product)
        np.testing.assert_allclose(out["y"][t], d, rtol=1e-12, atol=1e-18)


def test_zero_routed_down_leaves_shared_expert():
    layer, npl = _layer(dict(H=64, I=32, E=6, k=2, I_s=16))
    x = _bf16_bits(synth.make_tokens(layer, 3, 5))
    npl["experts"]["down"] = dict(npl["experts"]["down"],
                                  data=np.zeros_like(npl["experts"]["down"]["data"]))
    out = moe_forward(npl["cfg"], npl, x)
    np.testing.assert_array_equal(out["y"], out["shared"])


def test_linear_in_down_weights():
    # Scaling every routed down matrix by 2 (exact in BF16) doubles the
    # routed part of the output.
    layer, npl = _layer(dict(H=64, I=32, E=6, k=2, I_s=0))
    x = _bf16_bits(synth.make_tokens(layer, 3, 6))
    ref = moe_forward(npl["cfg"], npl, x)
    d = layer["experts"]["down"]["data"] * 2
    npl["experts"]["down"] = dict(npl["experts"]["down"], data=_bf16_bits(d))
    out = moe_forward(npl["cfg"], npl, x)
    np.testing.assert_allclose(out["y"], 2 * ref["y"], rtol=1e-14, atol=1e-300)


def test_squared_terms_single_expert_closed_form():
    # one expert, k = 1, weight 1: y_sq[r] = sum_i (Wd[r, i] a_i)^2, which is
    # never below y[r]^2 / I (Cauchy-Schwarz) nor above (sum_i |Wd a|)^2
    layer, npl = _layer(dict(H=32, I=16, E=1, k=1, I_s=0))
    x = _bf16_bits(synth.make_tokens(layer, 2, 12))
    out = moe_forward(npl["cfg"], npl, x)
    ex = npl["experts"]
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wd = dequant(ex["down"], 0)
    for t in range(2):
        _, _, a, d = swiglu_expert(dequant(ex["gate"], 0), dequant(ex["up"], 0), wd, xf[t])
        terms = wd * a[None, :]
        np.testing.assert_allclose(out["y_sq"][t], (terms ** 2).sum(axis=1), rtol=1e-12)
        assert np.all(out["y_sq"][t] * 16 >= d ** 2 * (1 - 1e-12))
        assert np.all(out["y_sq"][t] <= np.abs(terms).sum(axis=1) ** 2 * (1 + 1e-12))


def test_squared_terms_scale_with_the_weights():
    # doubling every routed down matrix (exact in BF16) quadruples y_sq
    layer, npl = _layer(dict(H=64, I=32, E=6, k=2, I_s=0))
    x = _bf16_bits(synth.make_tokens(layer, 3, 13))
    ref = moe_forward(npl["cfg"], npl, x)
    d = layer["experts"]["down"]["data"] * 2
    npl["experts"]["down"] = dict(npl["experts"]["down"], data=_bf16_bits(d))
    out = moe_forward(npl["cfg"], npl, x)
    np.testing.assert_allclose(out["y_sq"], 4 * ref["y_sq"], rtol=1e-14, atol=1e-300)


def test_rows_subset_matches_full():
    layer, npl = _layer(dict(H=64, I=32, E=6, k=2, I_s=16, routed_fmt="nvfp4"))
    x = _bf16_bits(synth.make_tokens(layer, 2, 7))
    full = moe_forward(npl["cfg"], npl, x)
    rows = np.array([63, 0, 17, 5])
    sub = moe_forward(npl["cfg"], npl, x, rows=rows)
    np.testing.assert_allclose(sub["y"], full["y"][:, rows], rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(sub["y_sq"], full["y_sq"][:, rows], rtol=1e-12, atol=1e-300)


# ---- brute force --------------------------------------------------------

def _tdq(p, e):
    """Dense weights through torch's dtype conversions only."""
    fmt = p["format"]
    if fmt == "bf16":
        return p["data"][e].double().tolist()
    if fmt == "fp8_rowscale":
        v = p["data"][e].view(torch.float8_e4m3fn).double()
        return (v * p["scales"][e].double()[:, None]).tolist()
    packed = p["data"][e]
    rows, half = packed.shape
    out = []
    e2m1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for r in range(rows):
        row = []
        for b in range(half):
            for nib in (int(packed[r, b]) & 15, int(packed[r, b]) >> 4):
                v = e2m1[nib & 7] * (-1.0 if nib & 8 else 1.0)
                col = len(row)
                if fmt == "mxfp4":
                    s = p["scales"][e, r, col // 32:col // 32 + 1].view(torch.float8_e8m0fnu)
                    row.append(v * float(s.double()))
                else:
                    s = p["scales"][e, r, col // 16:col // 16 + 1].view(torch.float8_e4m3fn)
                    row.append(v * float(s.double()) * float(p["tensor_scale"][e]))
        out.append(row)
    return out


def _brute_layer(layer, x):
    cfg = layer["cfg"]
    H, E, k = cfg["H"], cfg["E"], cfg["k"]
    wr = layer["router"]["weight"].double().tolist()
    bias = layer["router"]["bias"]
    xs = x.double().tolist()
    ys, sqs = [], []
    for xt in xs:
        z = [sum(wr[e][h] * xt[h] for h in range(H)) for e in range(E)]
        if cfg["scoring"] == "softmax":
            s = z
        else:
            s = [1 / (1 + math.exp(-v)) + float(bias[e]) for e, v in enumerate(z)]
        sel = sorted(range(E), key=lambda e: (-s[e], e))[:k]
        if cfg["scoring"] == "softmax":
            m = max(z)
            den = sum(math.exp(v - m) for v in z)
            w = [math.exp(z[e] - m) / den for e in sel]
        else:
            w = [1 / (1 + math.exp(-z[e])) for e in sel]
        if cfg["renorm"]:
            tot = sum(w)
            w = [v / tot for v in w]
        w = [v * cfg["rsf"] for v in w]
        y = [0.0] * H
        sq = [0.0] * H

        def ffn(wg, wu, wd, scale):
            # every term scale * wd[r][i] * a[i] of the output, listed
            inter = len(wg)
            g = [sum(wg[i][h] * xt[h] for h in range(H)) for i in range(inter)]
            u = [sum(wu[i][h] * xt[h] for h in range(H)) for i in range(inter)]
            a = [g[i] / (1 + math.exp(-g[i])) * u[i] for i in range(inter)]
            return [[scale * wd[r][i] * a[i] for i in range(inter)] for r in range(H)]

        ex = layer["experts"]
        terms = [ffn(_tdq(ex["gate"], e), _tdq(ex["up"], e), _tdq(ex["down"], e), we)
                 for e, we in zip(sel, w)]
        if layer["shared"] is not None:
            sh = layer["shared"]
            terms.append(ffn(_tdq(sh["gate"], 0), _tdq(sh["up"], 0), _tdq(sh["down"], 0), 1.0))
        for tr in terms:
            for r in range(H):
                y[r] += sum(tr[r])
                sq[r] += sum(v * v for v in tr[r])
        ys.append(y)
        sqs.append(sq)
    return np.array(ys), np.array(sqs)


@pytest.mark.parametrize("fmt,shared_fmt,scoring", [
    ("bf16", "bf16", "softmax"),
    ("mxfp4", None, "softmax"),
    ("nvfp4", "bf16", "sigmoid"),
    ("fp8_rowscale", "fp8_rowscale", "softmax"),
])
def test_layer_matches_pure_python_brute_force(fmt, shared_fmt, scoring):
    over = dict(H=32, I=32, E=5, k=2, I_s=32 if shared_fmt else 0, routed_fmt=fmt,
                shared_fmt=shared_fmt, scoring=scoring,
                bias_std=0.1 if scoring == "sigmoid" else None,
                rsf=2.5 if scoring == "sigmoid" else 1.0)
    layer, npl = _layer(over)
    x = synth.make_tokens(layer, 2, 8)
    got = moe_forward(npl["cfg"], npl, _bf16_bits(x))
    want, want_sq = _brute_layer(layer, x)
    np.testing.assert_allclose(got["y"], want, rtol=1e-11, atol=1e-13)
    # the sum of the squared terms of each output element
    np.testing.assert_allclose(got["y_sq"], want_sq, rtol=1e-11, atol=1e-300)


# ---- shared-expert gate and expert-parallel shares ----------------------

def test_shared_gate_weight_closed_form():
    from oracle import shared_gate_weight
    x = np.array([[0.5, -1.0, 2.0], [0.0, 0.0, 0.0]])
    w = np.array([1.0, 0.25, -0.125])
    g = shared_gate_weight(x, w)
    dots = [0.5 * 1.0 + (-1.0) * 0.25 + 2.0 * (-0.125), 0.0]
    for t in range(2):
        assert math.isclose(g[t], 1.0 / (1.0 + math.exp(-dots[t])), rel_tol=1e-15)
    assert np.array_equal(shared_gate_weight(x, None), np.ones(2))


def _gated_layer(cfg_over):
    cfg = synth.reduced("tiny_bf16", shared_gate=True, **cfg_over)
    layer = synth.make_layer(cfg)
    assert layer["router"]["shared_gate"] is not None
    return layer, synth.as_numpy(layer)


def test_zero_gate_vector_halves_the_shared_expert():
    # sigmoid(0) = 1/2 exactly: y = routed + s / 2
    layer, npl = _gated_layer(dict(H=64, I=32, E=6, k=2, I_s=16))
    x = _bf16_bits(synth.make_tokens(layer, 3, 8))
    npl["router"]["shared_gate"] = np.zeros_like(npl["router"]["shared_gate"])
    gated = moe_forward(npl["cfg"], npl, x)
    plain = dict(npl, router=dict(npl["router"], shared_gate=None))
    ref = moe_forward(npl["cfg"], plain, x)
    assert np.array_equal(gated["gamma"], np.full(3, 0.5))
    np.testing.assert_allclose(gated["y"], ref["y"] - 0.5 * ref["shared"], rtol=1e-12, atol=1e-15)


def test_gated_shared_squared_terms():
    # with zero routed down weights only the shared expert's terms remain;
    # a zero gate vector weights them by sigmoid(0) = 1/2, so y_sq by 1/4
    layer, npl = _gated_layer(dict(H=64, I=32, E=6, k=2, I_s=16))
    x = _bf16_bits(synth.make_tokens(layer, 3, 14))
    npl["experts"]["down"] = dict(npl["experts"]["down"],
                                  data=np.zeros_like(npl["experts"]["down"]["data"]))
    npl["router"]["shared_gate"] = np.zeros_like(npl["router"]["shared_gate"])
    gated = moe_forward(npl["cfg"], npl, x)
    plain = moe_forward(npl["cfg"], dict(npl, router=dict(npl["router"], shared_gate=None)), x)
    assert plain["y_sq"].min() > 0
    np.testing.assert_allclose(gated["y_sq"], 0.25 * plain["y_sq"], rtol=1e-14, atol=1e-300)


def test_gate_brute_force_per_token():
    layer, npl = _gated_layer(dict(H=32, I=16, E=4, k=2, I_s=8))
    xt = synth.make_tokens(layer, 2, 9)
    x = _bf16_bits(xt)
    out = moe_forward(npl["cfg"], npl, x)
    wsg = layer["router"]["shared_gate"].double().tolist()
    for t, row in enumerate(xt.double().tolist()):
        dot = sum(a * b for a, b in zip(row, wsg))
        assert math.isclose(out["gamma"][t], 1.0 / (1.0 + math.exp(-dot)), rel_tol=1e-13)


def _share(npl, lo, hi):
    """The layer as an expert-parallel share holding experts lo..hi-1."""
    ex = {}
    for name, p in npl["experts"].items():
        q = dict(p, data=p["data"][lo:hi], count=hi - lo)
        if p.get("scales") is not None:
            q["scales"] = p["scales"][lo:hi]
        if p.get("tensor_scale") is not None:
            q["tensor_scale"] = p["tensor_scale"][lo:hi]
        ex[name] = q
    return dict(npl, experts=ex)


@pytest.mark.parametrize("bounds", [(0, 3, 6), (0, 1, 4, 6), (0, 6)])
def test_expert_shares_sum_to_the_layer(bounds):
    # the shares' routed partials plus the gated shared expert, added once,
    # give the whole layer
    for gated in (False, True):
        layer, npl = _gated_layer(dict(H=64, I=32, E=6, k=3, I_s=16, routed_fmt="mxfp4"))
        if not gated:
            npl["router"]["shared_gate"] = None
        x = _bf16_bits(synth.make_tokens(layer, 4, 10))
        full = moe_forward(npl["cfg"], npl, x)
        parts = [moe_forward(npl["cfg"], _share(npl, lo, hi), x, expert_range=(lo, hi))
                 for lo, hi in zip(bounds[:-1], bounds[1:])]
        for p in parts:
            assert p["shared"] is None and np.array_equal(p["idx"], full["idx"])
        total = sum(p["y"] for p in parts) + full["gamma"][:, None] * full["shared"]
        np.testing.assert_allclose(total, full["y"], rtol=1e-12, atol=1e-15)


def test_share_without_selected_experts_is_zero():
    layer, npl = _gated_layer(dict(H=64, I=32, E=6, k=1, I_s=16))
    x = _bf16_bits(synth.make_tokens(layer, 2, 11))
    full = moe_forward(npl["cfg"], npl, x)
    used = set(full["idx"].reshape(-1).tolist())
    free = [e for e in range(6) if e not in used]
    if free:
        e = free[0]
        part = moe_forward(npl["cfg"], _share(npl, e, e + 1), x, expert_range=(e, e + 1))
        assert not part["y"].any()
