"""Parity of the routing variants against the FP64 oracle, through the C ABI,
on both paths: the softmax+bias arm, zero experts (router width E + Z) and
hash routing (token-id table), plus the device error word for invalid hash
inputs ("forward_batched.rs": router_bias_one, the router width
num_experts + zero_expert_num, the hash-routing branch).

Bar as for the other parity tests: indices bit-exact (tie-free tokens for
score-based selection), weights within 1e-5, every grouping bit-exact,
per-token relative L2 within 1e-2.
"""

import numpy as np
import pytest
import torch

import synth
from parity_util import check_against_oracle, device_error, run_hip, tie_free_filter

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(cfg, n, seed, path="auto", accum=None, hashed=False):
    label = f"{cfg['name']} n={n} path={path} accum={accum}"
    print(f"[variant] {label}", flush=True)
    layer = synth.make_layer(cfg, device=DEV)
    npl = synth.as_numpy(layer)
    x = synth.make_tokens(layer, n, seed, accept=None if hashed else tie_free_filter(npl))
    ids = synth.make_token_ids(layer, n, seed) if hashed else None
    res = check_against_oracle(layer, x, accum=accum, label=label, path=path, token_ids=ids)
    print(f"[variant] {label}: max rel L2 {res['rel_l2']:.2e}", flush=True)
    return res


SMB_TINY = synth.reduced("tiny_bf16", bias_std=0.05, name="tiny_softmax_bias")
SMB_MX = synth.reduced("qwen3_30b_a3b_mxfp4", H=512, I=256, E=64, k=8, bias_std=0.02,
                       name="mxfp4_softmax_bias")


@pytest.mark.parametrize("n", [1, 4])
def test_softmax_bias_decode(n):
    _case(SMB_TINY, n, 700 + n)


def test_softmax_bias_mxfp4_decode():
    _case(SMB_MX, 3, 703)


@pytest.mark.parametrize("accum", ["slot", "atomic"])
def test_softmax_bias_grouped(accum):
    _case(SMB_TINY, 17, 704, path="grouped", accum=accum)


def test_softmax_bias_mxfp4_grouped():
    _case(SMB_MX, 40, 705, path="grouped")


ZE_SMB = synth.reduced("tiny_bf16", E=6, Z=2, k=3, bias_std=0.05, name="zero_experts_smb")
ZE_SIG = synth.reduced("deepseek_v3_nvfp4", H=1024, I=256, E=24, Z=8, k=6, I_s=256,
                       name="zero_experts_sigmoid_nvfp4")
ZE_WIDE_K = synth.reduced("tiny_bf16", E=4, Z=4, k=6, name="zero_experts_k_above_e")


@pytest.mark.parametrize("n", [1, 4])
def test_zero_experts_softmax_bias_decode(n):
    _case(ZE_SMB, n, 710 + n)


def test_zero_experts_softmax_bias_grouped():
    _case(ZE_SMB, 20, 712, path="grouped")


@pytest.mark.parametrize("path,n", [("decode", 4), ("grouped", 33)])
def test_zero_experts_sigmoid_nvfp4(path, n):
    _case(ZE_SIG, n, 713, path=path)


@pytest.mark.parametrize("path,n", [("decode", 3), ("grouped", 9)])
def test_zero_experts_top_k_above_expert_count(path, n):
    _case(ZE_WIDE_K, n, 714, path=path)


HASH_TINY = synth.reduced("tiny_bf16", hash_vocab=50, name="hash_tiny")
HASH_SIG = synth.reduced("deepseek_v3_nvfp4", H=1024, I=256, E=32, Z=4, k=8, I_s=256,
                         hash_vocab=300, name="hash_sigmoid_zero_experts")


@pytest.mark.parametrize("n", [1, 4])
def test_hash_decode(n):
    _case(HASH_TINY, n, 720 + n, hashed=True)


@pytest.mark.parametrize("accum", ["slot", "atomic"])
def test_hash_grouped(accum):
    _case(HASH_TINY, 17, 723, path="grouped", accum=accum, hashed=True)


@pytest.mark.parametrize("path,n", [("decode", 4), ("grouped", 64)])
def test_hash_sigmoid_zero_experts(path, n):
    _case(HASH_SIG, n, 724, path=path, hashed=True)


# ---- invalid hash inputs: the kernels check them and set bit 16 --------------

def _bad_hash_run(path, n, mutate):
    layer = synth.make_layer(HASH_TINY, device=DEV)
    ids = synth.make_token_ids(layer, n, 730)
    mutate(layer, ids)
    x = synth.make_tokens(layer, n, 730)
    out, idx, w, logits, L = _run_allow_error(layer, x, path, ids)
    return device_error(L), idx.cpu().numpy(), layer


def _run_allow_error(layer, x, path, ids):
    from mixture_experts_layer_35_amd import Layer
    n = x.shape[0]
    cfg = layer["cfg"]
    L = Layer(layer, n, path=path)
    idx = torch.full((n, cfg["k"]), 0xFFFF, dtype=torch.int32, device=DEV)
    w = torch.full((n, cfg["k"]), float("nan"), dtype=torch.float32, device=DEV)
    logits = torch.empty((n, cfg["E"]), dtype=torch.float32, device=DEV)
    out = torch.empty_like(x)
    L.forward(x, out=out, idx=idx, weights=w, logits=logits, token_ids=ids)
    torch.cuda.synchronize()
    return out, idx, w, logits, L


@pytest.mark.parametrize("path,n", [("decode", 3), ("grouped", 9)])
def test_hash_token_id_out_of_range_sets_error(path, n):
    def mutate(layer, ids):
        ids[1] = layer["router"]["tid2eid"].shape[0]  # one past the vocabulary
    err, idx, layer = _bad_hash_run(path, n, mutate)
    assert err & (1 << 16)
    assert (idx[1] == layer["cfg"]["E"]).all()  # the token's slots go past every expert


@pytest.mark.parametrize("path,n", [("decode", 3), ("grouped", 9)])
def test_hash_bad_table_row_sets_error(path, n):
    def mutate(layer, ids):
        t = layer["router"]["tid2eid"]
        ids[0] = 7
        ids[2] = 8
        t[7, 1] = t[7, 0]          # the same expert twice
        t[8, 0] = layer["cfg"]["E"] + 5  # an expert outside the router width
    err, idx, layer = _bad_hash_run(path, n, mutate)
    assert err & (1 << 16)
    assert idx[0, 1] == layer["cfg"]["E"] and idx[2, 0] == layer["cfg"]["E"]


# ---- NVFP4 router ("forward_k3.rs", "forward_atomic_c4.rs", "forward_ep.rs":
# the w4a16 router GEMV/GEMM taken when the layer has an NVFP4 gate) ---------

QR_MX = synth.reduced("qwen3_30b_a3b_mxfp4", H=1024, I=256, E=64, k=8, router_fmt="nvfp4",
                      name="nvfp4_router_mxfp4_experts")
QR_GATED = synth.reduced("deepseek_v3_nvfp4", H=1024, I=256, E=48, Z=4, k=8, I_s=256,
                         router_fmt="nvfp4", shared_gate=True, name="nvfp4_router_gated_z4")


@pytest.mark.parametrize("n", [1, 3])
def test_nvfp4_router_decode(n):
    _case(QR_MX, n, 740 + n)


def test_nvfp4_router_gated_decode():
    _case(QR_GATED, 4, 742)


@pytest.mark.parametrize("n", [16, 70])
def test_nvfp4_router_grouped(n):
    _case(QR_MX, n, 743 + n, path="grouped")


def test_nvfp4_router_gated_grouped():
    _case(QR_GATED, 33, 745, path="grouped")


def test_nvfp4_router_deepseek_v3_full():
    # the DeepSeek-V3 shape with its router in NVFP4 too, N = 4, every
    # output row checked
    cfg = synth.reduced("deepseek_v3_nvfp4", router_fmt="nvfp4", name="ds_v3_nvfp4_router")
    layer = synth.make_layer(cfg, device=DEV)
    npl = synth.as_numpy(layer)
    x = synth.make_tokens(layer, 4, 746, accept=tie_free_filter(npl))
    print("[variant] ds_v3_nvfp4_router n=4", flush=True)
    check_against_oracle(layer, x, label="ds_v3 nvfp4 router")
