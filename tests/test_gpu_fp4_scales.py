"""FP4 block scales on both paths: where the kernels read them in words and
wider loads, and where they fall back to per-chunk reads.

The C ABI asks only 1-byte (MXFP4) or 2-byte (NVFP4) alignment of the scale
array. Aligned scales are read a 32-bit word (decode) or a whole 4-chunk
block (grouped) at a time; scales at an odd address are read chunk by chunk,
and so are the short last blocks of rows whose chunk count is not a multiple
of four. Every case here meets the parity bar of parity_util against the
FP64 oracle: indices bit-exact, weights 1e-5, every output element within
the element-wise bound, per-token relative L2 within 1e-2.
"""

import pytest
import torch

import synth
from parity_util import check_against_oracle, tie_free_filter

pytestmark = pytest.mark.gpu

DEV = "cuda"

MX = synth.reduced("qwen3_30b_a3b_mxfp4", H=512, I=384, E=32, k=4, name="mxfp4_h512_i384")
NV = synth.reduced("deepseek_v3_nvfp4", H=1024, I=384, E=32, k=8, I_s=256,
                   name="nvfp4_h1024_i384")


def _shift_scales(layer, shift):
    """Move every FP4 scale array to an address `shift` bytes past an
    allocation's start (same values)."""
    for group in (layer["experts"], layer["shared"] or {}):
        for p in group.values():
            s = p["scales"]
            if s is None or s.dtype != torch.uint8:
                continue
            buf = torch.zeros(s.numel() + 64, dtype=torch.uint8, device=s.device)
            v = buf[shift:shift + s.numel()].view(s.shape)
            v.copy_(s)
            assert v.data_ptr() % 4 == shift % 4
            p["scales"] = v
    return layer


def _run(cfg, n, seed, path, shift=0, tokens=None, accum=None):
    label = f"{cfg['name'] if isinstance(cfg, dict) else cfg} {path} n={n} scale shift={shift}"
    print(f"[parity] {label}", flush=True)
    layer = synth.make_layer(cfg, device=DEV)
    if shift:
        _shift_scales(layer, shift)
    npl = synth.as_numpy(layer)
    x = synth.make_tokens(layer, n, seed, accept=tie_free_filter(npl))
    res = check_against_oracle(layer, x, accum=accum, label=label, path=path, tokens=tokens)
    print(f"[parity] {label}: max rel L2 {res['rel_l2']:.2e}", flush=True)
    return res


@pytest.mark.parametrize("path,n", [("decode", 3), ("grouped", 24)])
@pytest.mark.parametrize("cfg,shift", [(MX, 1), (MX, 3), (NV, 2)],
                         ids=["mxfp4+1", "mxfp4+3", "nvfp4+2"])
def test_fp4_scales_unaligned(cfg, shift, path, n):
    _run(cfg, n, 70 + shift, path, shift=shift)


@pytest.mark.parametrize("path,n", [("decode", 4), ("grouped", 40)])
@pytest.mark.parametrize("cfg", [MX, NV], ids=["mxfp4", "nvfp4"])
def test_fp4_scales_aligned_short_last_block(cfg, path, n):
    # I = 384: three 128-column chunks, so every down row ends in a short block
    _run(cfg, n, 80 + n, path)


def test_qwen3_mxfp4_full_shape_grouped():
    # H = 2048 (four whole blocks), I = 768 (one whole block and a short one)
    _run("qwen3_30b_a3b_mxfp4", 64, 91, "grouped", tokens=list(range(0, 64, 4)))


def test_deepseek_v3_nvfp4_full_shape_grouped():
    # H = 7168 and I = 2048: whole blocks only
    _run("deepseek_v3_nvfp4", 16, 92, "grouped", tokens=[0, 5, 10, 15], accum="atomic")
