"""Seeded synthetic workloads for the routed MoE layer.

This module draws inputs and packs weights into the canonical byte layouts the
library takes. It holds none of the layer's arithmetic: it never decodes a
weight, never projects a token and never routes. Tests and the benchmark feed
the same generated tensors to the FP64 oracle and to the HIP path.

Canonical layouts (per projection, ``count`` experts, ``rows`` outputs,
``cols`` reduction):
  bf16          data  [count, rows, cols]      BF16
  fp8_rowscale  data  [count, rows, cols]      OCP E4M3FN bytes
                scales[count, rows]            FP32 (one per output row)
  mxfp4         data  [count, rows, cols/2]    E2M1 pairs, even column in the low nibble
                scales[count, rows, cols/32]   E8M0 bytes
  nvfp4         data  [count, rows, cols/2]    E2M1 pairs, even column in the low nibble
                scales[count, rows, cols/16]   OCP E4M3FN bytes
                tensor_scale [count]           FP32
gate and up are [count, I, H]; down is [count, H, I].
"""

from __future__ import annotations

import copy
import math

import numpy as np
import torch

__all__ = ["CONFIGS", "seed_for", "make_layer", "make_tokens", "make_token_ids", "as_numpy",
           "layer_bytes", "reduced", "clone_weights"]

# The five workloads. Sizes and distributions as stated for each shape.
CONFIGS = {
    # tiny BF16 layer with one BF16 shared expert
    "tiny_bf16": dict(cfg_id=0, H=256, I=128, E=8, k=2, I_s=128, scoring="softmax",
                      renorm=True, rsf=1.0, routed_fmt="bf16", shared_fmt="bf16",
                      w_std=0.02, bias_std=None, zipf=None, n_list=(3,),
                      accum="slot"),
    # Qwen3-30B-A3B-shaped layer, MXFP4 routed experts, no shared expert;
    # FP32 atomic accumulation (at N = 1 it finishes sooner than the
    # slot-order sum, which stays available and tested)
    "qwen3_30b_a3b_mxfp4": dict(cfg_id=1, H=2048, I=768, E=128, k=8, I_s=0,
                                scoring="softmax", renorm=True, rsf=1.0,
                                routed_fmt="mxfp4", shared_fmt=None, w_std=0.02,
                                bias_std=None, zipf=None, n_list=(1, 3),
                                accum="atomic"),
    # DeepSeek-V3-shaped layer, NVFP4 routed experts, BF16 shared expert,
    # sigmoid router with FP32 correction bias, FP32 atomic accumulation
    "deepseek_v3_nvfp4": dict(cfg_id=2, H=7168, I=2048, E=256, k=8, I_s=2048,
                              scoring="sigmoid", renorm=True, rsf=2.5,
                              routed_fmt="nvfp4", shared_fmt="bf16", w_std=0.02,
                              bias_std=0.1, zipf=None, n_list=(4,),
                              accum="atomic"),
    # batched decode grouped by expert, FP8 experts with per-row scales
    "grouped_fp8_h4096": dict(cfg_id=3, H=4096, I=1536, E=128, k=8, I_s=4096,
                              scoring="softmax", renorm=True, rsf=1.0,
                              routed_fmt="fp8_rowscale", shared_fmt="fp8_rowscale",
                              w_std=0.02, bias_std=None, zipf=1.1,
                              n_list=(16, 32, 64), accum="slot"),
    # prefill-sized grouped GEMM, BF16 experts N(0,1)
    "prefill_bf16_h4096": dict(cfg_id=4, H=4096, I=1536, E=128, k=8, I_s=0,
                               scoring="softmax", renorm=True, rsf=1.0,
                               routed_fmt="bf16", shared_fmt=None, w_std=1.0,
                               bias_std=None, zipf=None, n_list=(512,),
                               accum="slot"),
}

_TENSOR_IDS = {"router": 1, "bias": 2, "gate": 3, "up": 4, "down": 5, "shared_gate": 11,
               "sgate": 6, "sup": 7, "sdown": 8, "x": 9, "zipf": 10, "tid2eid": 12,
               "token_ids": 13}


def seed_for(*parts) -> int:
    """Deterministic 63-bit seed from integer parts (NumPy SeedSequence)."""
    st = np.random.SeedSequence([int(p) for p in parts]).generate_state(2, dtype=np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def reduced(base: str, **over) -> dict:
    """A copy of config ``base`` with some fields replaced (smaller shapes for
    tests that the oracle finishes in seconds)."""
    c = copy.deepcopy(CONFIGS[base])
    c.update(over)
    c["name"] = over.get("name", base + "_reduced")
    return c


def _cfg(name_or_cfg) -> dict:
    if isinstance(name_or_cfg, dict):
        c = dict(name_or_cfg)
        c.setdefault("name", "custom")
        return c
    c = copy.deepcopy(CONFIGS[name_or_cfg])
    c["name"] = name_or_cfg
    return c


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(35, *parts))
    return g


# ---------------------------- encoders ------------------------------------

def _e2m1_codes(v: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even onto the E2M1 grid {0,.5,1,1.5,2,3,4,6} with
    saturation at 6; returns 4-bit codes (sign in bit 3)."""
    a = v.abs()
    mag = ((a > 0.25).to(torch.uint8) + (a >= 0.75).to(torch.uint8)
           + (a > 1.25).to(torch.uint8) + (a >= 1.75).to(torch.uint8)
           + (a > 2.5).to(torch.uint8) + (a >= 3.5).to(torch.uint8)
           + (a > 5.0).to(torch.uint8))
    neg = ((v < 0) & (mag > 0)).to(torch.uint8)
    return mag | (neg << 3)


def _pack_nibbles(codes: torch.Tensor) -> torch.Tensor:
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).contiguous()


def _e4m3_bytes(v: torch.Tensor) -> torch.Tensor:
    """RNE to OCP E4M3FN with saturation at +-448 (torch's cast does the
    rounding; the clamp keeps it from producing NaN)."""
    return v.float().clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def _quantize(w: torch.Tensor, fmt: str) -> dict:
    """w: float32 [count, rows, cols] on any device -> packed projection."""
    cnt, rows, cols = w.shape
    if fmt == "bf16":
        return dict(format=fmt, data=w.to(torch.bfloat16).contiguous(), scales=None,
                    tensor_scale=None)
    if fmt == "fp8_rowscale":
        amax = w.abs().amax(dim=2)
        rs = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).float()
        q = _e4m3_bytes(w / rs[..., None])
        return dict(format=fmt, data=q.contiguous(), scales=rs.contiguous(),
                    tensor_scale=None)
    if fmt == "mxfp4":
        g = w.reshape(cnt, rows, cols // 32, 32)
        amax = g.abs().amax(dim=3)
        # OCP MX rule: shared exponent = floor(log2(amax)) - emax(E2M1)=2
        ex = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2.0,
                         torch.zeros_like(amax)).clamp(-127.0, 127.0)
        scale = torch.exp2(ex)
        codes = _e2m1_codes(g / scale[..., None]).reshape(cnt, rows, cols)
        sbytes = (ex + 127.0).to(torch.uint8)
        return dict(format=fmt, data=_pack_nibbles(codes), scales=sbytes.contiguous(),
                    tensor_scale=None)
    if fmt == "nvfp4":
        amax_t = w.abs().reshape(cnt, -1).amax(dim=1)
        ts = torch.where(amax_t > 0, amax_t / (6.0 * 448.0), torch.ones_like(amax_t)).float()
        g = w.reshape(cnt, rows, cols // 16, 16)
        amax_b = g.abs().amax(dim=3)
        sb = _e4m3_bytes(amax_b / (6.0 * ts[:, None, None]))
        sf = sb.view(torch.float8_e4m3fn).float()
        denom = (sf * ts[:, None, None])[..., None]
        safe = torch.where(denom > 0, denom, torch.ones_like(denom))
        codes = _e2m1_codes(torch.where(denom > 0, g / safe, torch.zeros_like(g)))
        codes = codes.reshape(cnt, rows, cols)
        return dict(format=fmt, data=_pack_nibbles(codes), scales=sb.contiguous(),
                    tensor_scale=ts.contiguous())
    raise ValueError(fmt)


def _packed_shapes(fmt: str, count: int, rows: int, cols: int) -> dict:
    """Shapes and dtypes of a packed projection's arrays (None: absent)."""
    if fmt == "bf16":
        return {"data": ((count, rows, cols), torch.bfloat16), "scales": None,
                "tensor_scale": None}
    if fmt == "fp8_rowscale":
        return {"data": ((count, rows, cols), torch.uint8),
                "scales": ((count, rows), torch.float32), "tensor_scale": None}
    if fmt == "mxfp4":
        return {"data": ((count, rows, cols // 2), torch.uint8),
                "scales": ((count, rows, cols // 32), torch.uint8), "tensor_scale": None}
    if fmt == "nvfp4":
        return {"data": ((count, rows, cols // 2), torch.uint8),
                "scales": ((count, rows, cols // 16), torch.uint8),
                "tensor_scale": ((count,), torch.float32)}
    raise ValueError(fmt)


def _projection(cfg, device, tag: str, fmt: str, count: int, rows: int, cols: int,
                std: float) -> dict:
    """Draw N(0, std) float32 weights expert by expert and pack each one
    straight into its slice of preallocated arrays (every scale of every
    format lies within one expert, so packing per expert gives the same bytes
    as packing all experts at once)."""
    out = {"format": fmt, "rows": rows, "cols": cols, "count": count}
    for key, spec in _packed_shapes(fmt, count, rows, cols).items():
        out[key] = None if spec is None else torch.empty(spec[0], dtype=spec[1], device=device)
    w = torch.empty((rows, cols), dtype=torch.float32, device=device)
    for e in range(count):
        g = _gen(device, cfg["cfg_id"], _TENSOR_IDS[tag], e)
        torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32, out=w)
        q = _quantize((w * std).unsqueeze(0), fmt)
        for key in ("data", "scales", "tensor_scale"):
            if out[key] is not None:
                out[key][e].copy_(q[key][0])
    return out


def make_layer(name_or_cfg, device="cpu") -> dict:
    """Router, routed experts and shared expert for a config, on ``device``."""
    cfg = _cfg(name_or_cfg)
    H, I, E, I_s = cfg["H"], cfg["I"], cfg["E"], cfg["I_s"]
    EW = E + cfg.get("Z", 0)  # router width: the experts and the zero experts
    g = _gen(device, cfg["cfg_id"], _TENSOR_IDS["router"])
    wr = torch.randn((EW, H), generator=g, device=device) / math.sqrt(H)
    if cfg.get("zipf"):
        # Zipf(s) skew as a log-prior: a seeded rank r_e in 1..E and offset
        # -s*ln(r_e) in the last router column; tokens carry 1.0 there.
        gz = _gen("cpu", cfg["cfg_id"], _TENSOR_IDS["zipf"])
        ranks = torch.randperm(EW, generator=gz).to(torch.float64) + 1.0
        wr[:, H - 1] = (-cfg["zipf"] * torch.log(ranks)).to(wr.dtype).to(device)
    router = {"weight": wr.to(torch.bfloat16).contiguous(), "bias": None, "shared_gate": None}
    if cfg.get("router_fmt") == "nvfp4":
        # the same N(0, 1/sqrt(H)) rows, quantised to NVFP4 (one projection of
        # count 1); the BF16 weight is then absent
        q = _quantize(wr.float().unsqueeze(0), "nvfp4")
        q.update({"format": "nvfp4", "rows": EW, "cols": H, "count": 1})
        router["weight_q"] = q
        router["weight"] = None
    if cfg.get("shared_gate") and I_s > 0:
        # the shared-expert gate vector, N(0, 1/sqrt(H)) like a router row
        gg = _gen(device, cfg["cfg_id"], _TENSOR_IDS["shared_gate"])
        router["shared_gate"] = (torch.randn((H,), generator=gg, device=device)
                                 / math.sqrt(H)).to(torch.bfloat16).contiguous()
    if cfg.get("bias_std"):
        gb = _gen(device, cfg["cfg_id"], _TENSOR_IDS["bias"])
        router["bias"] = (torch.randn((EW,), generator=gb, device=device)
                          * cfg["bias_std"]).float().contiguous()
    if cfg.get("hash_vocab"):
        # hash routing: each of `hash_vocab` token ids lists k distinct experts
        # of the router width, a seeded permutation prefix per row
        gh = _gen("cpu", cfg["cfg_id"], _TENSOR_IDS["tid2eid"])
        rows = [torch.randperm(EW, generator=gh)[:cfg["k"]] for _ in range(cfg["hash_vocab"])]
        router["tid2eid"] = torch.stack(rows).to(torch.int32).to(device).contiguous()
    std = cfg["w_std"]
    experts = {
        "gate": _projection(cfg, device, "gate", cfg["routed_fmt"], E, I, H, std),
        "up": _projection(cfg, device, "up", cfg["routed_fmt"], E, I, H, std),
        "down": _projection(cfg, device, "down", cfg["routed_fmt"], E, H, I, std),
    }
    shared = None
    if I_s > 0:
        sf = cfg["shared_fmt"]
        shared = {
            "gate": _projection(cfg, device, "sgate", sf, 1, I_s, H, std),
            "up": _projection(cfg, device, "sup", sf, 1, I_s, H, std),
            "down": _projection(cfg, device, "sdown", sf, 1, H, I_s, std),
        }
    return {"cfg": cfg, "router": router, "experts": experts, "shared": shared}


def make_tokens(layer: dict, n: int, batch_seed: int = 0, accept=None,
                max_attempts: int = 64) -> torch.Tensor:
    """[n, H] BF16 tokens, x ~ N(0, 1). ``accept`` (optional) takes a BF16
    [m, H] CPU tensor and returns a boolean array of tokens to keep; rejected
    tokens are redrawn with the next attempt number."""
    cfg = layer["cfg"]
    H = cfg["H"]
    device = layer["experts"]["gate"]["data"].device
    x = torch.empty((n, H), dtype=torch.bfloat16, device=device)
    for t in range(n):
        x[t].copy_(_draw_token(cfg, device, n, batch_seed, t, 0))
    if accept is not None:
        attempt = 0
        while True:
            ok = np.asarray(accept(x.cpu()), dtype=bool)
            if ok.all():
                break
            attempt += 1
            if attempt >= max_attempts:
                raise RuntimeError("could not draw tokens accepted by the filter")
            for t in np.nonzero(~ok)[0]:
                x[t] = _draw_token(cfg, device, n, batch_seed, int(t), attempt)
    return x.contiguous()


def make_token_ids(layer: dict, n: int, batch_seed: int = 0) -> torch.Tensor:
    """[n] int32 token ids, uniform over the layer's hash vocabulary."""
    cfg = layer["cfg"]
    g = _gen("cpu", cfg["cfg_id"], _TENSOR_IDS["token_ids"], n, batch_seed)
    ids = torch.randint(0, cfg["hash_vocab"], (n,), generator=g, dtype=torch.int64)
    return ids.to(torch.int32).to(layer["experts"]["gate"]["data"].device).contiguous()


def _draw_token(cfg, device, n, batch_seed, t, attempt) -> torch.Tensor:
    g = _gen(device, cfg["cfg_id"], _TENSOR_IDS["x"], n, batch_seed, t, attempt)
    v = torch.randn((cfg["H"],), generator=g, device=device)
    if cfg.get("zipf"):
        v[cfg["H"] - 1] = 1.0
    return v.to(torch.bfloat16)


# ---------------------------- helpers -------------------------------------

def _np(t):
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_numpy(layer: dict) -> dict:
    """Host NumPy copy of a layer (BF16 as uint16 bit patterns)."""
    def proj(p):
        return {k: (_np(v) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    out = {"cfg": dict(layer["cfg"]),
           "router": {"weight": _np(layer["router"]["weight"]),
                      "weight_q": (None if layer["router"].get("weight_q") is None else
                                   {k: (_np(v) if isinstance(v, torch.Tensor) else v)
                                    for k, v in layer["router"]["weight_q"].items()}),
                      "bias": _np(layer["router"]["bias"]),
                      "shared_gate": _np(layer["router"].get("shared_gate")),
                      "tid2eid": _np(layer["router"].get("tid2eid"))},
           "experts": {k: proj(v) for k, v in layer["experts"].items()},
           "shared": None}
    if layer["shared"] is not None:
        out["shared"] = {k: proj(v) for k, v in layer["shared"].items()}
    return out


def clone_weights(layer: dict) -> dict:
    """Same values at new addresses (used to rotate weight copies so repeated
    calls do not find the weights in cache)."""
    def proj(p):
        return {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    out = dict(layer)
    out["router"] = {k: (proj(v) if isinstance(v, dict) else
                         (v.clone() if v is not None else None))
                     for k, v in layer["router"].items()}
    out["experts"] = {k: proj(v) for k, v in layer["experts"].items()}
    out["shared"] = None if layer["shared"] is None else {
        k: proj(v) for k, v in layer["shared"].items()}
    return out


def projection_bytes(p: dict, experts: int = 1) -> int:
    """Bytes of ``experts`` experts of a projection (values + scales)."""
    per = p["data"][0].numel() * p["data"].element_size()
    if p["scales"] is not None:
        per += p["scales"][0].numel() * p["scales"].element_size()
    if p["tensor_scale"] is not None:
        per += 4
    return per * experts


def layer_bytes(layer: dict) -> dict:
    """Per-unit byte counts: one routed expert (gate+up+down), the shared
    expert, the router (+ bias)."""
    ex = layer["experts"]
    b_e = sum(projection_bytes(ex[k]) for k in ("gate", "up", "down"))
    b_s = 0
    if layer["shared"] is not None:
        b_s = sum(projection_bytes(layer["shared"][k]) for k in ("gate", "up", "down"))
    r = layer["router"]
    b_r = (projection_bytes(r["weight_q"]) if r.get("weight_q") is not None
           else r["weight"].numel() * 2)
    b_r += 0 if r["bias"] is None else r["bias"].numel() * 4
    if r.get("shared_gate") is not None:
        b_r += r["shared_gate"].numel() * 2
    b_e_gu = sum(projection_bytes(ex[k]) for k in ("gate", "up"))
    return {"expert": b_e, "expert_gate_up": b_e_gu, "expert_down": b_e - b_e_gu,
            "shared": b_s, "router": b_r}
