"""Parity of the expert-parallel share entry point (moe_forward_ep_partial)
against the FP64 oracle, through the C ABI, on both paths.

A layer's experts are split into G index ranges. Each share is checked on
its own against the oracle's share (routing over all experts, only the
share's experts computed, FP32 output), and the sum of the G shares plus
the shared expert's term, added once, against the oracle's whole layer.
Bar: routing bit-exact / within 1e-5 as for moe_forward, the share's
grouping bit-exact on the grouped path, every element within the element-wise
bound of parity_util (FP32 partials: the activations' BF16 hand-off only),
per-token relative L2 within 1e-2, and exact zeros for tokens none of whose
experts is in the share.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import bf16_to_f64, moe_forward
from parity_util import (OUT_RTOL, W_RTOL, assert_elementwise, bits, check_grouping,
                         device_error, rel_l2_per_token, tie_free_filter)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _split(E, G):
    # uneven on purpose when G does not divide E
    b = np.linspace(0, E, G + 1).round().astype(int)
    return [(int(lo), int(hi)) for lo, hi in zip(b[:-1], b[1:])]


def _run_shares(cfg_or_name, n, seed, ranges, carrier=None, accum=None, path="auto",
                label=""):
    """Run every share of ``ranges`` (share ``carrier`` adds the shared
    expert) and check each against the oracle, then their sum."""
    from mixture_experts_layer_35_amd import Layer
    print(f"[share] {label}", flush=True)
    layer = synth.make_layer(cfg_or_name, device=DEV)
    npl = synth.as_numpy(layer)
    cfg = npl["cfg"]
    x = synth.make_tokens(layer, n, seed, accept=tie_free_filter(npl))
    xb = bits(x)
    full = moe_forward(cfg, npl, xb)
    L = Layer(layer, n, accum=accum, path=path)
    grouped = L.num_launches(n) > 1
    total = np.zeros((n, cfg["H"]), np.float64)
    has_shared = full["shared"] is not None
    for g, (lo, hi) in enumerate(ranges):
        with_shared = has_shared and carrier == g
        idx = torch.full((n, cfg["k"]), 0xFFFF, dtype=torch.int32, device=DEV)
        w = torch.full((n, cfg["k"]), float("nan"), dtype=torch.float32, device=DEV)
        out = torch.full((n, cfg["H"]), float("nan"), dtype=torch.float32, device=DEV)
        L.forward_share(x, lo, hi, with_shared=with_shared, out=out, idx=idx, weights=w)
        torch.cuda.synchronize()
        assert device_error(L) == 0, "a workgroup wait expired"
        # the routing is the whole layer's, whichever share runs
        assert np.array_equal(idx.cpu().numpy().astype(np.int64), full["idx"]), (label, g)
        np.testing.assert_allclose(w.cpu().numpy(), full["w"], rtol=W_RTOL, atol=0)
        if grouped:
            check_grouping(L, n, full["idx"], cfg["E"], expert_range=(lo, hi))
        got = out.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), f"{label}: share {g} left rows unwritten"
        local_npl = dict(npl)
        local_npl["experts"] = {k: _slice(v, lo, hi) for k, v in npl["experts"].items()}
        loc = moe_forward(cfg, local_npl, xb, expert_range=(lo, hi))
        ref, ref_sq = loc["y"], loc["y_sq"]
        if with_shared:
            ref = ref + full["gamma"][:, None] * full["shared"]
            # the shared term's squares are among the whole layer's
            ref_sq = ref_sq + full["y_sq"]
        touched = ((full["idx"] >= lo) & (full["idx"] < hi)).any(axis=1) | with_shared
        assert (got[~touched] == 0).all(), f"{label}: share {g} wrote to untouched tokens"
        if touched.any():
            err = rel_l2_per_token(got[touched], ref[touched])
            assert err.max() <= OUT_RTOL, f"{label}: share {g} rel L2 {err}"
            # an FP32 partial: only the activations' BF16 hand-off rounds
            assert_elementwise(got[touched], ref[touched], ref_sq[touched],
                               f"{label}: share {g}", rounded_output=False)
        total += got
    covered = sorted(ranges) == ranges and ranges[0][0] == 0 and ranges[-1][1] == cfg["E"] and \
        all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))
    if covered:  # the shares partition the experts: their sum is the layer
        if has_shared and carrier is None:
            total += full["gamma"][:, None] * full["shared"]
        err = rel_l2_per_token(total, full["y"])
        assert err.max() <= OUT_RTOL, f"{label}: sum of shares rel L2 {err}"
        assert_elementwise(total, full["y"], full["y_sq"], f"{label}: sum of shares",
                           rounded_output=False)
        print(f"[share] {label}: sum rel L2 {err.max():.2e}", flush=True)
    return L


def _slice(p, lo, hi):
    q = dict(p)
    for key in ("data", "scales", "tensor_scale"):
        if q.get(key) is not None:
            q[key] = q[key][lo:hi]
    q["count"] = hi - lo
    return q


# ---- decode path (N <= 4) ---------------------------------------------------

@pytest.mark.parametrize("n", [1, 3, 4])
def test_decode_shares_tiny(n):
    _run_shares("tiny_bf16", n, 600 + n, _split(8, 4), carrier=1,
                label=f"decode tiny_bf16 n={n} G=4")


def test_decode_shares_slot_layer_shared_added_once_by_caller():
    # a slot-mode layer: the slot-order sum skips the other shares' slots
    _run_shares("tiny_bf16", 4, 610, _split(8, 3), carrier=None, accum="slot",
                label="decode tiny_bf16 slot G=3 no carrier")


def test_decode_shares_nvfp4_sigmoid_gated():
    cfg = synth.reduced("deepseek_v3_nvfp4", H=1024, I=256, E=32, k=8, I_s=256,
                        shared_gate=True, name="nvfp4_h1024_gated")
    _run_shares(cfg, 4, 611, _split(32, 8), carrier=7, label="decode nvfp4 gated G=8")


def test_decode_single_expert_shares():
    cfg = synth.reduced("tiny_bf16", E=4, k=2, name="e4")
    _run_shares(cfg, 2, 612, _split(4, 4), carrier=0, label="decode e4 G=4")


def test_decode_share_mxfp4_c2_shape():
    # the Qwen3-30B-A3B shape with MXFP4 experts, one token, 8 shares of 16
    _run_shares("qwen3_30b_a3b_mxfp4", 1, 613, _split(128, 8), label="decode qwen3 mxfp4 G=8")


# ---- grouped path -----------------------------------------------------------

@pytest.mark.parametrize("accum", ["slot", "atomic"])
def test_grouped_shares_tiny(accum):
    _run_shares("tiny_bf16", 17, 620, _split(8, 4), carrier=2, accum=accum,
                path="grouped", label=f"grouped tiny_bf16 n=17 accum={accum}")


def test_grouped_shares_fp8_zipf():
    cfg = synth.reduced("grouped_fp8_h4096", H=512, I=384, E=16, k=4, I_s=256,
                        name="fp8_h512_zipf_shared")
    _run_shares(cfg, 40, 621, _split(16, 3), carrier=None, path="grouped",
                label="grouped fp8 zipf G=3")


def test_grouped_shares_gated_e256():
    cfg = synth.reduced("grouped_fp8_h4096", H=512, I=256, E=256, k=8, I_s=256,
                        shared_gate=True, zipf=None, name="fp8_e256_gated_g")
    _run_shares(cfg, 33, 622, _split(256, 8), carrier=5, path="grouped",
                label="grouped fp8 e256 gated G=8")


def test_grouped_share_then_whole_layer_on_one_workspace():
    # a share, then the whole layer, then a share again, on one workspace
    from parity_util import check_against_oracle
    L = _run_shares("tiny_bf16", 9, 623, [(2, 6)], carrier=None, path="grouped",
                    label="grouped tiny_bf16 one share")
    layer = L.layer
    npl = synth.as_numpy(layer)
    x = synth.make_tokens(layer, 9, 624, accept=tie_free_filter(npl))
    out = torch.full_like(x, float("nan"))
    L.forward(x, out=out)
    torch.cuda.synchronize()
    full = moe_forward(npl["cfg"], npl, bits(x))
    err = rel_l2_per_token(bf16_to_f64(bits(out)), full["y"])
    assert err.max() <= OUT_RTOL
    assert_elementwise(bf16_to_f64(bits(out)), full["y"], full["y_sq"], "whole layer")
    part = L.forward_share(x, 0, 8, with_shared=True)
    torch.cuda.synchronize()
    err = rel_l2_per_token(part.cpu().numpy(), full["y"])
    assert err.max() <= OUT_RTOL
    assert_elementwise(part.cpu().numpy(), full["y"], full["y_sq"], "share of all experts",
                       rounded_output=False)
