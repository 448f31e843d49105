"""Parity of the HIP decode path against the FP64 oracle, through the C ABI.

Bar: top-k indices bit-exact (tie-free tokens; lowest index on exact ties),
routing weights within 1e-5 relative, every output written, every output
element within the element-wise bound of parity_util (the BF16 roundings of
the path), per-token relative L2 of the BF16 output within 1e-2.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import moe_forward
from parity_util import (OUT_RTOL, assert_elementwise, bits, check_against_oracle,
                         device_error, run_hip, tie_free_filter)

pytestmark = pytest.mark.gpu

DEV = "cuda"
# per-call counters at the head of the workspace
HEAD_BYTES = 384 + 64 * 128


def _case(cfg_or_name, n, seed=0, accum=None, rows=None, label=None):
    label = label or f"{cfg_or_name if isinstance(cfg_or_name, str) else cfg_or_name['name']} n={n} accum={accum}"
    print(f"[parity] {label}", flush=True)
    layer = synth.make_layer(cfg_or_name, device=DEV)
    npl = synth.as_numpy(layer)
    x = synth.make_tokens(layer, n, seed, accept=tie_free_filter(npl))
    res = check_against_oracle(layer, x, accum=accum, rows=rows, label=label)
    print(f"[parity] {label}: max rel L2 {res['rel_l2']:.2e}", flush=True)
    return res


# ---- small shapes: several tiles and ragged tails ---------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("accum", ["slot", "atomic"])
def test_tiny_bf16(n, accum):
    _case("tiny_bf16", n, seed=n, accum=accum)


MX_SMALL = synth.reduced("qwen3_30b_a3b_mxfp4", H=544, I=192, E=16, k=4, name="mxfp4_h544_i192")


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_mxfp4_ragged(n):
    _case(MX_SMALL, n, seed=10 + n)


NV_SMALL = synth.reduced("deepseek_v3_nvfp4", H=1024, I=256, E=32, k=8, I_s=384,
                         name="nvfp4_h1024_shared_bf16")


@pytest.mark.parametrize("accum", ["slot", "atomic"])
@pytest.mark.parametrize("n", [1, 4])
def test_nvfp4_sigmoid_bias_shared(n, accum):
    _case(NV_SMALL, n, seed=20 + n, accum=accum)


FP8_SMALL = synth.reduced("grouped_fp8_h4096", H=512, I=384, E=16, k=4, I_s=256, zipf=None,
                          name="fp8_h512_shared_fp8")


@pytest.mark.parametrize("n", [1, 3, 4])
def test_fp8_rowscale_decode(n):
    _case(FP8_SMALL, n, seed=30 + n)


def test_bf16_unit_variance_weights():
    cfg = synth.reduced("prefill_bf16_h4096", H=256, I=160, E=8, k=2, name="bf16_n01")
    _case(cfg, 4, seed=40)


def test_no_renorm_and_scaled_softmax():
    cfg = synth.reduced("qwen3_30b_a3b_mxfp4", H=256, I=64, E=8, k=3, renorm=False, rsf=1.75,
                        name="mxfp4_norenorm")
    _case(cfg, 3, seed=41)


def test_single_expert_top1():
    cfg = synth.reduced("tiny_bf16", E=1, k=1, I_s=0, name="one_expert")
    _case(cfg, 2, seed=42)


def test_dense_all_experts_selected():
    cfg = synth.reduced("tiny_bf16", E=4, k=4, name="dense_k_eq_e")
    _case(cfg, 3, seed=43)


def test_top1_of_many():
    cfg = synth.reduced("deepseek_v3_nvfp4", H=512, I=128, E=256, k=1, I_s=0, name="top1_e256")
    _case(cfg, 4, seed=44)


def test_max_topk():
    cfg = synth.reduced("qwen3_30b_a3b_mxfp4", H=256, I=64, E=64, k=16, name="k16")
    _case(cfg, 4, seed=45)


# ---- full sizes -------------------------------------------------------------

@pytest.mark.parametrize("accum", ["atomic", "slot"])
@pytest.mark.parametrize("n", [1, 3])
def test_qwen3_30b_a3b_full(n, accum):
    _case("qwen3_30b_a3b_mxfp4", n, seed=100 + n, accum=accum)


@pytest.mark.parametrize("accum", ["atomic", "slot"])
def test_deepseek_v3_full(accum):
    # all 7168 output rows of all 4 tokens
    _case("deepseek_v3_nvfp4", 4, seed=200, accum=accum)


# ---- properties -------------------------------------------------------------

def test_lowest_index_wins_exact_ties():
    print("[parity] exact ties", flush=True)
    cfg = synth.reduced("tiny_bf16", E=8, k=2, I_s=0, name="ties")
    layer = synth.make_layer(cfg, device=DEV)
    x = synth.make_tokens(layer, 1, 50)
    ref0 = moe_forward(synth.as_numpy(layer)["cfg"], synth.as_numpy(layer), bits(x))
    top = int(ref0["idx"][0, 0])
    for other in (top - 1, top + 1):
        if not 0 <= other < 8:
            continue
        wr = layer["router"]["weight"].clone()
        wr[other] = wr[top]
        lay = dict(layer, router={"weight": wr, "bias": None})
        npl = synth.as_numpy(lay)
        ref = moe_forward(npl["cfg"], npl, bits(x))
        assert sorted(ref["idx"][0].tolist()) == sorted([top, other])
        out, idx, w, _, _ = run_hip(lay, x)
        assert idx.cpu().numpy().tolist() == ref["idx"].tolist() == [[min(top, other), max(top, other)]]
        np.testing.assert_allclose(w.cpu().numpy(), ref["w"], rtol=1e-5)


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_near_ties_follow_own_logits(path):
    """Two router rows a few ULPs apart: their logits agree in all but the
    last mantissa bits, where a selection on truncated score bits could not
    decide. The chosen experts must be the top k of the kernel's own FP32
    logits, ordered by (logit, -expert)."""
    print(f"[parity] near ties {path}", flush=True)
    cfg = synth.reduced("tiny_bf16", E=16, k=4, I_s=0, name="near_ties")
    layer = synth.make_layer(cfg, device=DEV)
    x = synth.make_tokens(layer, 4, 70)
    xf = x.float().cpu()
    ref0 = moe_forward(synth.as_numpy(layer)["cfg"], synth.as_numpy(layer), bits(x))
    wr = layer["router"]["weight"].clone()
    h = int(torch.argmin(xf[0].abs()))  # the smallest activation of token 0
    for j in range(3):
        top = int(ref0["idx"][0, j])
        other = (top + 5) % 16
        wr[other] = wr[top]
        v = wr[other, h].view(torch.int16)
        wr[other, h] = (v + (1 if j % 2 else -1)).view(torch.bfloat16)  # one BF16 ULP
    lay = dict(layer, router={"weight": wr, "bias": None})
    out, idx, w, logits, L = run_hip(lay, x, path=path)
    z = logits.cpu().numpy()
    for t in range(4):
        order = sorted(range(16), key=lambda e: (-float(z[t, e]), e))[:4]
        assert idx[t].cpu().numpy().tolist() == order, (t, z[t].tolist())
    assert device_error(L) == 0


def test_slot_mode_is_deterministic():
    print("[parity] determinism", flush=True)
    layer = synth.make_layer(NV_SMALL, device=DEV)
    x = synth.make_tokens(layer, 4, 60)
    a = run_hip(layer, x, accum="slot")[0]
    b = run_hip(layer, x, accum="slot")[0]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_atomic_and_slot_agree():
    print("[parity] atomic vs slot", flush=True)
    layer = synth.make_layer(NV_SMALL, device=DEV)
    npl = synth.as_numpy(layer)
    x = synth.make_tokens(layer, 4, 61, accept=tie_free_filter(npl))
    a = run_hip(layer, x, accum="slot")[0].double()
    b = run_hip(layer, x, accum="atomic")[0].double()
    err = ((a - b).norm(dim=1) / a.norm(dim=1)).max().item()
    assert err <= OUT_RTOL / 2


@pytest.mark.parametrize("accum", ["atomic", "slot"])
def test_repeated_calls_reuse_workspace(accum):
    # counters, the plan and (atomic mode) the accumulator live in the
    # workspace; calls with other tokens and other N must not see the
    # previous call's state
    print(f"[parity] workspace reuse {accum}", flush=True)
    from mixture_experts_layer_35_amd import Layer
    from parity_util import device_error
    layer = synth.make_layer(NV_SMALL, device=DEV)
    npl = synth.as_numpy(layer)
    acc = tie_free_filter(npl)
    L = Layer(layer, 4, accum=accum)
    for seed, n in ((70, 4), (71, 2), (72, 3), (73, 1), (74, 4)):
        x = synth.make_tokens(layer, n, seed, accept=acc)
        out = L.forward(x)
        torch.cuda.synchronize()
        assert device_error(L) == 0
        ref = moe_forward(npl["cfg"], npl, bits(x))
        o = out.double().cpu().numpy()
        err = np.linalg.norm(o - ref["y"], axis=1) / np.linalg.norm(ref["y"], axis=1)
        assert err.max() <= OUT_RTOL, (seed, err)
    # counters are back to zero, no wait expired, and the call counter
    # advanced once per call (words: done 0, error 32, epoch 64, done groups
    # from 96, one 32-word line each)
    head = L.workspace[:HEAD_BYTES].view(torch.int32).cpu().numpy()
    assert head[0] == 0 and head[32] == 0 and head[64] == 5, head[[0, 32, 64]]
    assert not head[96:96 + 64 * 32].any()


@pytest.mark.parametrize("accum", ["atomic", "slot"])
@pytest.mark.parametrize("cfg", [NV_SMALL, "qwen3_30b_a3b_mxfp4"], ids=["nvfp4-small", "qwen3"])
def test_back_to_back_calls_without_host_sync(cfg, accum):
    # Calls enqueued back to back on one stream, one synchronisation at the
    # end: each call takes its tag from the call counter that the previous
    # kernel advanced (once every workgroup holds its tag, which can be before
    # the last ones finish), so every output must still be its own call's.
    # (The Qwen3-shaped layer's grid is resident at N = 1 and not at N = 3.)
    name = cfg if isinstance(cfg, str) else cfg["name"]
    print(f"[parity] back to back {name} {accum}", flush=True)
    from mixture_experts_layer_35_amd import Layer
    from parity_util import device_error
    layer = synth.make_layer(cfg, device=DEV)
    npl = synth.as_numpy(layer)
    acc = tie_free_filter(npl)
    L = Layer(layer, 4, accum=accum)
    seq = [(110 + i, (1, 4, 2, 3)[i % 4]) for i in range(12 if isinstance(cfg, dict) else 6)]
    xs = [synth.make_tokens(layer, n, seed, accept=acc) for seed, n in seq]
    torch.cuda.synchronize()
    outs = [L.forward(x) for x in xs]
    torch.cuda.synchronize()
    assert device_error(L) == 0
    for (seed, n), x, out in zip(seq, xs, outs):
        ref = moe_forward(npl["cfg"], npl, bits(x))
        o = out.double().cpu().numpy()
        err = np.linalg.norm(o - ref["y"], axis=1) / np.linalg.norm(ref["y"], axis=1)
        assert err.max() <= OUT_RTOL, (seed, n, err)
        assert_elementwise(o, ref["y"], ref["y_sq"], f"back to back n={n} seed={seed}")
    head = L.workspace[:HEAD_BYTES].view(torch.int32).cpu().numpy()
    assert head[0] == 0 and head[32] == 0 and head[64] == len(seq), head[[0, 32, 64]]


@pytest.mark.parametrize("accum", ["atomic", "slot"])
def test_decode_after_grouped_on_one_workspace(accum):
    # A grouped call leaves small integers (expert ids, counts, the ticket,
    # token masks) in its buffers, and a decode call's tags are small integers
    # too. Decode calls after grouped ones on the same workspace must find
    # none of them in their tagged hand-off words.
    print(f"[parity] decode after grouped {accum}", flush=True)
    from mixture_experts_layer_35_amd import Layer
    cfg = synth.reduced("qwen3_30b_a3b_mxfp4", H=512, I=256, E=128, k=8,
                        name="mxfp4_e128_mixed_paths")
    layer = synth.make_layer(cfg, device=DEV)
    npl = synth.as_numpy(layer)
    acc = tie_free_filter(npl)
    L = Layer(layer, 512, accum=accum)
    for seed, n in ((90, 16), (91, 1), (92, 3), (93, 512), (94, 4), (95, 1), (96, 2)):
        x = synth.make_tokens(layer, n, seed, accept=acc)
        out = L.forward(x)
        torch.cuda.synchronize()
        assert device_error(L) == 0, (seed, n)
        assert (L.num_launches(n) > 1) == (n > 4)
        tok = np.arange(n) if n <= 16 else np.arange(0, n, 37)
        ref = moe_forward(npl["cfg"], npl, bits(x)[tok])
        o = out.double().cpu().numpy()[tok]
        err = np.linalg.norm(o - ref["y"], axis=1) / np.linalg.norm(ref["y"], axis=1)
        assert err.max() <= OUT_RTOL, (seed, n, err)
        assert_elementwise(o, ref["y"], ref["y_sq"], f"n={n} seed={seed}")


# ---- shared-expert sigmoid gate ---------------------------------------------

@pytest.mark.parametrize("accum", ["slot", "atomic"])
@pytest.mark.parametrize("n", [1, 4])
def test_shared_gate_decode(n, accum):
    cfg = synth.reduced("tiny_bf16", shared_gate=True, name="tiny_gated")
    _case(cfg, n, seed=80 + n, accum=accum)


def test_shared_gate_nvfp4_e256_decode():
    # 256 experts: the gate is router row 256, past the logit rows
    cfg = synth.reduced("deepseek_v3_nvfp4", H=512, I=128, E=256, k=8, I_s=256,
                        shared_gate=True, name="nvfp4_e256_gated")
    _case(cfg, 3, seed=85, accum="atomic")
