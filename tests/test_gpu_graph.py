"""The layer forward captured in a HIP graph (through torch.cuda.CUDAGraph)
and replayed: every replay, with eager calls on the same workspace and
synchronisations in between, must give the eager call's result for the same
input (bit for bit in slot mode; in FP32-atomic mode, whose summation order
varies, up to that order: parity_util.assert_same_up_to_order) and match the
FP64 oracle. The library
enqueues only kernel launches, so the capture holds no memset node."""

import numpy as np
import pytest
import torch

import synth
from oracle import bf16_to_f64, moe_forward
from parity_util import (OUT_RTOL, assert_elementwise, assert_same_up_to_order, bits,
                         device_error, rel_l2_per_token, tie_free_filter)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("name,n,path,accum", [
    ("tiny_bf16", 3, "decode", "slot"),
    ("tiny_bf16", 3, "decode", "atomic"),
    ("tiny_bf16", 17, "grouped", "slot"),
    ("tiny_bf16", 17, "grouped", "atomic"),
    ("qwen3_30b_a3b_mxfp4", 1, "decode", "atomic"),
])
def test_graph_replays_match_eager(name, n, path, accum):
    from mixture_experts_layer_35_amd import Layer
    print(f"[graph] {name} n={n} {path} {accum}", flush=True)
    layer = synth.make_layer(name, device=DEV)
    npl = synth.as_numpy(layer)
    xs = [synth.make_tokens(layer, n, 900 + i, accept=tie_free_filter(npl)) for i in range(4)]
    L = Layer(layer, n, accum=accum, path=path)
    x_in = xs[0].clone()
    out = torch.empty_like(x_in)
    side = torch.cuda.Stream()
    call = L.prepare(x_in, out, stream=side.cuda_stream)
    with torch.cuda.stream(side):
        call()  # the first call outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        x_in.copy_(x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = L.forward(x)  # an eager call on the same workspace in between
        torch.cuda.synchronize()
        assert device_error(L) == 0
        ref = moe_forward(npl["cfg"], npl, bits(x))
        if accum == "slot":
            assert torch.equal(got, eager), f"replay {i} differs from the eager call"
        else:
            assert_same_up_to_order(got.double().cpu().numpy(), eager.double().cpu().numpy(),
                                    ref["y_sq"], f"replay {i}")
        err = rel_l2_per_token(bf16_to_f64(bits(got)), ref["y"])
        assert err.max() <= OUT_RTOL, f"replay {i}: rel L2 {err}"
        assert_elementwise(bf16_to_f64(bits(got)), ref["y"], ref["y_sq"], f"replay {i}")
