"""Pins for the oracle's element decoders and block-scaled dequantisation.

The decoders are written from the bit-field definitions. They are pinned here
against things other than themselves: torch's own FP8/E8M0/BF16 conversions
(exhaustive over every code), the OCP Microscaling v1.0 E2M1 value table, hand
decoded byte patterns, and a round trip through the generator's independent
encoders.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (bf16_to_f64, dequant, e2m1_to_f64, e4m3fn_to_f64,
                    e8m0_to_f64, unpack_fp4)
import synth


def _same(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape
    assert np.array_equal(np.isnan(a), np.isnan(b))
    m = ~np.isnan(a)
    assert np.array_equal(a[m], b[m])
    # signed zeros too
    assert np.array_equal(np.signbit(a[m]), np.signbit(b[m]))


def test_e4m3fn_all_codes_match_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    _same(e4m3fn_to_f64(np.arange(256)), ref)


def test_e8m0_all_codes_match_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    _same(e8m0_to_f64(np.arange(256)), ref)


def test_bf16_matches_torch():
    g = np.random.default_rng(1)
    bits = g.integers(0, 1 << 16, size=4096, dtype=np.int64).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    _same(bf16_to_f64(bits), ref)


def test_e2m1_matches_ocp_mx_table():
    # OCP Microscaling Formats v1.0, FP4 E2M1 element table: magnitudes of
    # codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    want = mags + [-m for m in mags]
    _same(e2m1_to_f64(np.arange(16)), want)


def test_e2m1_via_e4m3_embedding():
    # Every E2M1 value is an E4M3 value: exponent field e>0 maps to E4M3
    # exponent e+6 with the mantissa bit moved to the top mantissa bit; the
    # subnormal 0.5 is E4M3 exponent 6 with zero mantissa. Decode through
    # torch's E4M3 conversion, independent of the oracle's E2M1 formula.
    out = []
    for c in range(16):
        s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
        if e > 0:
            byte = (s << 7) | ((e + 6) << 3) | (m << 2)
        elif m == 1:
            byte = (s << 7) | (6 << 3)
        else:
            byte = s << 7
        out.append(byte)
    ref = torch.tensor(out, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    _same(e2m1_to_f64(np.arange(16)), ref.numpy())


def test_spot_values():
    assert e4m3fn_to_f64(0x7E) == 448.0          # S.1111.110 = 1.75 * 2^8
    assert e4m3fn_to_f64(0x01) == 2.0 ** -9       # smallest subnormal
    assert e4m3fn_to_f64(0x08) == 2.0 ** -6       # smallest normal
    assert e4m3fn_to_f64(0x38) == 1.0
    assert e4m3fn_to_f64(0xB8) == -1.0
    assert math.isnan(e4m3fn_to_f64(0x7F)) and math.isnan(e4m3fn_to_f64(0xFF))
    assert e8m0_to_f64(127) == 1.0 and e8m0_to_f64(128) == 2.0
    assert e8m0_to_f64(0) == 2.0 ** -127 and math.isnan(e8m0_to_f64(255))
    assert bf16_to_f64(np.uint16(0x3F80)) == 1.0
    assert bf16_to_f64(np.uint16(0xC040)) == -3.0


# The byte pattern 0x10,0x32,...,0xFE holds codes 0..15 in column order when
# the even column sits in the low nibble.
_ROW = np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE] * 2, dtype=np.uint8)
_CODES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
          -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_unpack_low_nibble_first():
    assert unpack_fp4(_ROW[None, :2]).tolist() == [[0, 1, 2, 3]]


def test_mxfp4_hand_decoded_row():
    w = dict(format="mxfp4", rows=1, cols=32, count=1,
             data=_ROW[None, None, :], scales=np.array([[[0x81]]], np.uint8),
             tensor_scale=None)
    # scale byte 0x81 = 2^(129-127) = 4
    _same(dequant(w, 0)[0], [4.0 * v for v in _CODES * 2])


def test_nvfp4_hand_decoded_row():
    w = dict(format="nvfp4", rows=1, cols=32, count=1,
             data=_ROW[None, None, :],
             scales=np.array([[[0x38, 0x40]]], np.uint8),   # E4M3 1.0, 2.0
             tensor_scale=np.array([0.5], np.float32))
    want = [0.5 * v for v in _CODES] + [1.0 * v for v in _CODES]
    _same(dequant(w, 0)[0], want)


def test_fp8_rowscale_hand_decoded():
    data = np.array([[[0x38, 0x40, 0xB8, 0x7E, 0x01, 0x00, 0x80, 0x30] * 2]], np.uint8)
    w = dict(format="fp8_rowscale", rows=1, cols=16, count=1, data=data,
             scales=np.array([[0.25]], np.float32), tensor_scale=None)
    base = [1.0, 2.0, -1.0, 448.0, 2.0 ** -9, 0.0, -0.0, 0.5]
    _same(dequant(w, 0)[0], [0.25 * v for v in base * 2])


def test_dequant_second_expert_and_row_select():
    data = np.stack([np.zeros((3, 16), np.uint8), np.tile(_ROW, (3, 1))])
    sc = np.stack([np.full((3, 1), 127, np.uint8), np.array([[127], [128], [126]], np.uint8)])
    w = dict(format="mxfp4", rows=3, cols=32, count=2, data=data, scales=sc,
             tensor_scale=None)
    full = dequant(w, 1)
    _same(full[1], [2.0 * v for v in _CODES * 2])
    _same(full[2], [0.5 * v for v in _CODES * 2])
    _same(dequant(w, 1, rows=[2, 0]), full[[2, 0]])
    assert not dequant(w, 0).any()


def _torch_dequant(p, e):
    """Independent dequant: torch's E4M3/E8M0/BF16 decoders plus the E2M1
    embedding into E4M3."""
    fmt = p["format"]
    if fmt == "bf16":
        return p["data"][e].to(torch.float64)
    if fmt == "fp8_rowscale":
        return (p["data"][e].view(torch.float8_e4m3fn).to(torch.float64)
                * p["scales"][e].to(torch.float64)[:, None])
    packed = p["data"][e]
    codes = torch.stack([packed & 15, packed >> 4], dim=-1).reshape(packed.shape[0], -1)
    s, ex, m = (codes >> 3) & 1, (codes >> 1) & 3, codes & 1
    byte = torch.where(ex > 0, (s << 7) | ((ex + 6) << 3) | (m << 2),
                       torch.where(m == 1, (s << 7) | (6 << 3), s << 7)).to(torch.uint8)
    vals = byte.view(torch.float8_e4m3fn).to(torch.float64)
    if fmt == "mxfp4":
        sc = p["scales"][e].view(torch.float8_e8m0fnu).to(torch.float64)
        return vals * sc.repeat_interleave(32, dim=1)
    sc = p["scales"][e].view(torch.float8_e4m3fn).to(torch.float64)
    return vals * sc.repeat_interleave(16, dim=1) * float(p["tensor_scale"][e])


@pytest.mark.parametrize("fmt", ["bf16", "fp8_rowscale", "mxfp4", "nvfp4"])
def test_dequant_matches_torch_decoders(fmt):
    cfg = synth.reduced("tiny_bf16", H=64, I=32, E=3, k=2, I_s=0, routed_fmt=fmt)
    layer = synth.make_layer(cfg)
    npl = synth.as_numpy(layer)
    for name in ("gate", "down"):
        for e in range(3):
            ref = _torch_dequant(layer["experts"][name], e).numpy()
            _same(dequant(npl["experts"][name], e), ref)


def test_generator_encoders_round_trip_exact_grid():
    # Values already on the E2M1 grid times a power-of-two block scale come
    # back exactly through the generator's MXFP4 encoder and the oracle.
    g = torch.Generator().manual_seed(3)
    grid = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    vals = grid[torch.randint(0, 8, (2, 4, 64), generator=g)]
    vals = vals * torch.where(torch.rand(vals.shape, generator=g) < 0.5, -1.0, 1.0)
    vals[..., 0::32] = 6.0          # each block's amax is 6 -> exponent 0
    scale = torch.tensor([2.0 ** -7, 2.0 ** 3]).view(2, 1, 1)
    w = (vals * scale).float()
    q = synth._quantize(w, "mxfp4")
    p = {k: (v.numpy() if isinstance(v, torch.Tensor) else v) for k, v in q.items()}
    p.update(rows=4, cols=64, count=2)
    for e in range(2):
        # the encoder writes -0 as +0, so compare values, not sign bits
        assert np.array_equal(dequant(p, e), w[e].double().numpy())
