"""Parity of the grouped path (router GEMM, top-k, grouping by expert, MFMA
expert GEMMs, combine) against the FP64 oracle, through the C ABI.

Bar: top-k indices bit-exact (tie-free tokens), routing weights within 1e-5
relative, the grouping (units, padded offsets, permutation and its inverse)
bit-exact against the oracle's stable grouping, every output written, every
output element within the element-wise bound of parity_util, and per-token
relative L2 of the BF16 output within 1e-2.
"""

import numpy as np
import pytest

import synth
from parity_util import check_against_oracle, tie_free_filter

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(cfg_or_name, n, seed=0, accum=None, rows=None, tokens=None, label=None):
    name = cfg_or_name if isinstance(cfg_or_name, str) else cfg_or_name["name"]
    label = label or f"grouped {name} n={n} accum={accum}"
    print(f"[parity] {label}", flush=True)
    layer = synth.make_layer(cfg_or_name, device=DEV)
    npl = synth.as_numpy(layer)
    x = synth.make_tokens(layer, n, seed, accept=tie_free_filter(npl))
    res = check_against_oracle(layer, x, accum=accum, rows=rows, label=label, path="grouped",
                               tokens=tokens)
    assert res["grouped"]
    print(f"[parity] {label}: max rel L2 {res['rel_l2']:.2e}", flush=True)
    return res


# ---- small shapes: ragged token counts, several tiles ------------------------

@pytest.mark.parametrize("n", [1, 5, 17, 40])
@pytest.mark.parametrize("accum", ["slot", "atomic"])
def test_tiny_bf16_grouped(n, accum):
    _case("tiny_bf16", n, seed=300 + n, accum=accum)


FP8_G = synth.reduced("grouped_fp8_h4096", H=512, I=384, E=16, k=4, I_s=256,
                      name="fp8_h512_zipf_shared")


@pytest.mark.parametrize("n", [16, 33, 64, 130])
def test_fp8_rowscale_zipf_grouped(n):
    # skewed routing: the hottest expert takes most tokens (several 16-row
    # tiles, and more than one 128-row pass at n = 130)
    _case(FP8_G, n, seed=310 + n)


MX_G = synth.reduced("qwen3_30b_a3b_mxfp4", H=512, I=256, E=32, k=4, name="mxfp4_h512_i256")


@pytest.mark.parametrize("n", [6, 24])
def test_mxfp4_grouped(n):
    # down K = 256: a short last weight block (FP4 blocks span 4 chunks)
    _case(MX_G, n, seed=320 + n)


NV_G = synth.reduced("deepseek_v3_nvfp4", H=1024, I=256, E=32, k=8, I_s=384,
                     name="nvfp4_h1024_sigmoid_shared_bf16")


@pytest.mark.parametrize("accum", ["slot", "atomic"])
def test_nvfp4_sigmoid_bias_grouped(accum):
    _case(NV_G, 20, seed=330, accum=accum)


def test_bf16_unit_variance_grouped():
    cfg = synth.reduced("prefill_bf16_h4096", H=512, I=256, E=16, k=8, name="bf16_n01_g")
    _case(cfg, 64, seed=340)


def test_router_rows_not_multiple_of_tile():
    cfg = synth.reduced("tiny_bf16", E=24, k=3, name="e24")
    _case(cfg, 9, seed=341)


def test_single_expert_grouped():
    cfg = synth.reduced("tiny_bf16", E=1, k=1, I_s=0, name="one_expert_g")
    _case(cfg, 7, seed=342)


def test_dense_all_experts_grouped():
    cfg = synth.reduced("tiny_bf16", E=4, k=4, name="dense_g")
    _case(cfg, 9, seed=343)


def test_max_topk_grouped():
    cfg = synth.reduced("qwen3_30b_a3b_mxfp4", H=512, I=128, E=64, k=16, name="k16_g")
    _case(cfg, 12, seed=344)


def test_many_experts_many_tokens():
    # 300 tokens: ten mask words per expert, 256 experts
    cfg = synth.reduced("deepseek_v3_nvfp4", H=256, I=128, E=256, k=2, I_s=0, name="e256_n300")
    _case(cfg, 300, seed=345)


def test_many_experts_max_tokens():
    # 256 experts and the largest batch: 128 mask words per expert, so the
    # grouping workgroup holds its largest LDS (about 147 KB); the grouping is
    # checked whole, the output on every row of 16 sampled tokens
    cfg = synth.reduced("deepseek_v3_nvfp4", H=256, I=128, E=256, k=8, I_s=0, name="e256_n4096")
    tokens = np.sort(np.random.default_rng(17).choice(4096, size=16, replace=False))
    _case(cfg, 4096, seed=347, tokens=tokens)


def test_decode_sized_batch_on_grouped_path():
    # the grouped path takes any N, also the decode sizes
    _case("tiny_bf16", 3, seed=346)


# ---- token tiles per pass above 64 tokens -------------------------------------
# The host picks 2, 4 or 8 tiles of 16 tokens from the weight format, the
# average rows per expert (N*k/E) and the shared expert: each case below lands
# on the tile count named with it.

BF16_E128 = synth.reduced("prefill_bf16_h4096", H=512, I=256, E=128, k=8, name="bf16_e128_g")


@pytest.mark.parametrize("cfg,n,tiles", [
    (MX_G, 100, 2),        # FP4, no shared expert, 12.5 rows per expert
    (MX_G, 300, 4),        # FP4, no shared expert, 37.5 rows per expert
    (NV_G, 100, 2),        # FP4 with a shared expert, up to 128 tokens
    (NV_G, 200, 4),        # FP4 with a shared expert, above 128 tokens
    (FP8_G, 56, 2),        # FP8 above 48 tokens takes the rule for larger batches
    (FP8_G, 256, 4),       # FP8 with a shared expert (Zipf-skewed routing)
    (BF16_E128, 128, 2),   # BF16, 8 rows per expert
    (BF16_E128, 160, 8),   # BF16, 10 rows per expert
], ids=["fp4-n100-t2", "fp4-n300-t4", "fp4sh-n100-t2", "fp4sh-n200-t4", "fp8sh-n56-t2",
        "fp8sh-n256-t4",
        "bf16-n128-t2", "bf16-n160-t8"])
def test_token_tile_choices(cfg, n, tiles):
    _case(cfg, n, seed=600 + n + tiles, label=f"grouped {cfg['name']} n={n} ({tiles} tiles)")


# ---- full sizes -------------------------------------------------------------

@pytest.mark.parametrize("n", [16, 32, 64])
def test_grouped_fp8_h4096_full(n):
    # every output row of every token
    _case("grouped_fp8_h4096", n, seed=400 + n)


def test_prefill_bf16_h4096_full_sampled_tokens():
    # all 512 tokens run and are routed and grouped (the grouping is checked
    # whole); the output is checked on every row of 24 sampled tokens (the
    # oracle's expert work covers only those)
    tokens = np.sort(np.random.default_rng(9).choice(512, size=24, replace=False))
    _case("prefill_bf16_h4096", 512, seed=500, tokens=tokens)


@pytest.mark.parametrize("name,n", [("qwen3_30b_a3b_mxfp4", 512), ("grouped_fp8_h4096", 256)])
def test_quantised_full_shape_above_64_tokens_sampled(name, n):
    # four tiles per pass at the full shapes (FP4 without and FP8 with a
    # shared expert); every row of 8 sampled tokens, the grouping checked whole
    tokens = np.sort(np.random.default_rng(13 + n).choice(n, size=8, replace=False))
    _case(name, n, seed=502 + n, tokens=tokens)


def test_prefill_bf16_h4096_max_tokens_sampled_tokens():
    # the largest batch the library takes (MOE_MAX_TOKENS = 4096): 128 mask
    # words per expert and 256 rows per expert on average, checked on every
    # row of 12 sampled tokens; the grouping is checked whole
    tokens = np.sort(np.random.default_rng(11).choice(4096, size=12, replace=False))
    _case("prefill_bf16_h4096", 4096, seed=501, tokens=tokens)


# ---- shared-expert sigmoid gate ---------------------------------------------

@pytest.mark.parametrize("accum", ["slot", "atomic"])
def test_shared_gate_grouped(accum):
    cfg = synth.reduced("tiny_bf16", shared_gate=True, name="tiny_gated_g")
    _case(cfg, 17, seed=350, accum=accum)


def test_shared_gate_fp8_e256_grouped():
    # 257 router rows: the gate row opens a third 128-row router block
    cfg = synth.reduced("grouped_fp8_h4096", H=512, I=256, E=256, k=8, I_s=256,
                        shared_gate=True, zipf=None, name="fp8_e256_gated_g")
    _case(cfg, 40, seed=351)
