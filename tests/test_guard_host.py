"""The guard regions of the GPU guard tests, on the CPU: the 0xFF poison
decodes as a value no correct result is built from (NaN in every BF16, FP8,
block-scale and FP32 field; the largest magnitude in FP4), wrapping keeps a
tensor's bytes and places it at the start of its allocation, and a write into
a guard is seen."""

import numpy as np
import torch

from oracle import bf16_to_f64, e2m1_to_f64, e4m3fn_to_f64, e8m0_to_f64
from parity_util import GUARD, Guards


def test_poison_decodes_to_nan_or_the_largest_fp4():
    assert np.isnan(bf16_to_f64(np.array([0xFFFF], np.uint16))).all()
    assert np.isnan(e4m3fn_to_f64(np.array([0xFF], np.uint8))).all()
    assert np.isnan(e8m0_to_f64(np.array([0xFF], np.uint8))).all()
    assert np.isnan(np.frombuffer(b"\xff\xff\xff\xff", dtype=np.float32)).all()
    # a poisoned FP4 byte holds two codes 0xF: -6, the largest magnitude
    assert (e2m1_to_f64(np.array([0xF, 0xF], np.uint8)) == -6.0).all()


def test_wrap_keeps_bytes_and_guards_the_tail():
    G = Guards()
    src = torch.arange(-7, 25, dtype=torch.float32).reshape(4, 8).to(torch.bfloat16)
    v = G.wrap(src)
    assert v.dtype == src.dtype and v.shape == src.shape
    assert torch.equal(v.view(torch.int16), src.view(torch.int16))
    buf = G.bufs[-1]
    assert v.data_ptr() == buf.data_ptr() and buf.numel() == src.numel() * 2 + GUARD
    # the first BF16 value past the view is the poison
    nxt = buf[src.numel() * 2:src.numel() * 2 + 2].view(torch.int16).item() & 0xFFFF
    assert np.isnan(bf16_to_f64(np.array([nxt], np.uint16))).all()
    assert G.intact()
    buf[src.numel() * 2 + GUARD // 2] = 0
    assert not G.intact()
