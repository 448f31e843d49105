"""The workload generator packs each projection expert by expert into
preallocated arrays. Every scale of every format lies within one expert (row
scales, block scales along a row, the NVFP4 per-expert tensor scale), so that
must give exactly the bytes of quantising all experts' weights at once. This
checks it for each format on the CPU, with the same seeds."""

import pytest
import torch

import synth


def _all_at_once(cfg, tag, fmt, count, rows, cols, std):
    ws = []
    for e in range(count):
        g = synth._gen("cpu", cfg["cfg_id"], synth._TENSOR_IDS[tag], e)
        ws.append(torch.randn((rows, cols), generator=g, dtype=torch.float32) * std)
    return synth._quantize(torch.stack(ws), fmt)


@pytest.mark.parametrize("fmt", ["bf16", "fp8_rowscale", "mxfp4", "nvfp4"])
def test_per_expert_packing_matches_whole_tensor(fmt):
    cfg = synth.reduced("tiny_bf16", routed_fmt=fmt)
    count, rows, cols, std = 5, 48, 96, 0.02
    got = synth._projection(cfg, "cpu", "gate", fmt, count, rows, cols, std)
    want = _all_at_once(cfg, "gate", fmt, count, rows, cols, std)
    assert (got["count"], got["rows"], got["cols"]) == (count, rows, cols)
    for key in ("data", "scales", "tensor_scale"):
        if want[key] is None:
            assert got[key] is None
        else:
            assert got[key].dtype == want[key].dtype and got[key].shape == want[key].shape
            assert torch.equal(got[key].view(torch.uint8), want[key].view(torch.uint8)), key


def test_tokens_are_rows_of_their_own_draws():
    layer = synth.make_layer("tiny_bf16")
    x = synth.make_tokens(layer, 4, 7)
    for t in range(4):
        assert torch.equal(x[t].view(torch.int16),
                           synth._draw_token(layer["cfg"], "cpu", 4, 7, t, 0).view(torch.int16))
