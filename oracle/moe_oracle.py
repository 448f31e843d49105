"""FP64 CPU oracle for the routed mixture-of-experts layer forward.

TEST INFRASTRUCTURE ONLY. The HIP path's results are compared against this
module's. Only the test suite, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run it; the product path
never does, and it shares no code, table or constant with the HIP kernels.

Everything is plain NumPy in float64 and follows the order the reference pages
give for the layer: router projection, top-k routing, per-expert SwiGLU over
block-scaled weights, top-k weighted sum, shared-expert blend.

Sources (the four reference pages, cited by title and section):
  * "spark_model/layers/moe/forward_k3.rs", ``MoeLayer::forward_k3``: the
    doc comment lists the five stages (router GEMV, batched top-K, fused expert
    gate+up, fused silu+down, fused weighted sum + blend); step 2 chooses
    sigmoid plus a correction bias or softmax and passes ``norm_topk_prob`` and
    ``routed_scaling_factor``; the E8M0 guard comment and
    ``k3_e8m0_needs_per_token`` fix the scale-group sizes (GS16 E4M3 for
    NVFP4, GS32 E8M0 for MXFP4, ``inter*h/16`` against ``inter*h/32`` scale
    bytes); the NVFP4 branches pass one ``scale2`` value per expert and
    projection; the EP all-reduce block adds the shared expert once, by a plain
    residual add when the layer has no shared-expert gate.
  * "spark_model/layers/moe/forward_atomic_c4.rs",
    ``MoeLayer::forward_atomic_c4_decode``: routed down projections are summed
    in FP32 with their routing weights, then cast to BF16 and blended with the
    shared expert.
  * "metrale_model_layers/layers/moe/forward_batched.rs",
    ``MoeLayer::forward_batched``: one router GEMM for all N tokens, then per
    token routing, expert pair and blend; the grouped FP8 decode comment states
    that grouping by expert keeps the per-token result.

Readings where the pages are silent (each also listed in the design notes):
  R1  softmax is taken over all E logits, then the top k are selected (under
      renormalisation the order of the two does not matter);
  R2  selection uses the logit (softmax) or sigmoid(logit)+bias (sigmoid),
      never the exponentiated probabilities;
  R3  the correction bias steers selection only; weights use sigmoid(logit);
  R4  no group-limited routing;
  R5  renormalisation (w /= sum w, no epsilon) comes first, then the routed
      scaling factor multiplies the routed weights, in both scoring modes;
  R6  equal selection scores resolve to the lowest expert index, and the
      selected indices are listed in descending score order;
  R7  scale groups run along the reduction (column) axis of each row;
  R8  FP4 packing puts the even column in the low nibble;
  R9  E4M3 is OCP E4M3FN (no infinities, S.1111.111 is NaN, max 448);
  R10 NVFP4 carries one FP32 tensor scale per expert per projection;
  R11 FP8 weights carry one FP32 scale per output row;
  R12 the shared expert is added with gate 1 when the layer has no
      shared-expert gate; with a gate vector w_sg it is added with weight
      sigmoid(x . w_sg) per token (the gated blend);
  R13 an expert-parallel share holds the experts of one index range; routing
      stays global, slots whose expert is outside the range add nothing, and
      the shared expert is left to the caller, who adds it once after summing
      the shares;
  R14 the softmax+bias arm ("forward_batched.rs", router_bias_one) selects on
      softmax(logit) + bias, the softmax counterpart of sigmoid(logit) + bias;
      the weights stay the unbiased softmax probabilities;
  R15 hash routing ("forward_batched.rs", the hash-routing branch) takes the k
      experts of the token's table row, in the row's order; their weights are
      the layer's own weight rule (softmax over the whole router width, or
      sigmoid) at those experts, then renormalisation and the routed scaling
      factor; the correction bias plays no part;
  R16 zero experts ("forward_batched.rs", the router width num_experts +
      zero_expert_num) are router columns E..E+Z-1 with no weights: routing
      runs over all E+Z columns, and a slot that chooses a zero expert adds
      nothing to the output while its weight still counts in the
      renormalisation;
  R17 an NVFP4 router is dequantised exactly like the NVFP4 experts (E2M1
      values, E4M3 scale per 16 columns, one FP32 tensor scale) and the
      logits are x . W in full precision; the shared-expert gate stays BF16.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "e2m1_to_f64", "e8m0_to_f64", "e4m3fn_to_f64", "bf16_to_f64",
    "unpack_fp4", "dequant", "router_matrix", "router_logits", "selection_scores", "route",
    "softmax_rows", "routing_weights", "route_hash",
    "silu", "swiglu_expert", "moe_forward", "group_slots", "shared_gate_weight", "FORMATS",
]

FORMATS = ("bf16", "fp8_rowscale", "mxfp4", "nvfp4")


# --------------------------------------------------------------------------
# Element codes, decoded from their bit fields by formula.
# --------------------------------------------------------------------------

def e2m1_to_f64(codes) -> np.ndarray:
    """FP4 E2M1 code (4 bits: sign, 2-bit exponent with bias 1, 1-bit
    mantissa) to float64. Exponent 0 is subnormal: value = 0.5*m.
    Format named on "forward_k3.rs" (E8M0 guard: native MXFP4 values) and
    used for NVFP4 values in the NVFP4 branches."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    normal = np.ldexp(1.0 + 0.5 * m, e - 1)
    sub = 0.5 * m
    mag = np.where(e == 0, sub, normal)
    return np.where(s == 1, -mag, mag)


def e8m0_to_f64(b) -> np.ndarray:
    """E8M0 scale byte (unsigned exponent, bias 127, no mantissa) to float64:
    2**(b-127); 0xFF is NaN. The MXFP4 per-32 block scale ("forward_k3.rs",
    E8M0 guard comment)."""
    v = np.asarray(b).astype(np.int64)
    out = np.ldexp(1.0, v - 127)
    return np.where(v == 255, np.nan, out)


def e4m3fn_to_f64(b) -> np.ndarray:
    """OCP E4M3FN byte (sign, 4-bit exponent with bias 7, 3-bit mantissa) to
    float64. Exponent 0 is subnormal: (m/8)*2**-6. S.1111.111 is NaN; there
    are no infinities. Used for NVFP4 block scales (GS16, "forward_k3.rs"
    E8M0 guard comment) and for FP8 expert weights (FP8 batch3 branch)."""
    v = np.asarray(b).astype(np.int64)
    s = (v >> 7) & 1
    e = (v >> 3) & 15
    m = v & 7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, -6)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def bf16_to_f64(u16) -> np.ndarray:
    """BF16 bit pattern (the high half of an IEEE binary32) to float64."""
    u = np.asarray(u16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Block-scaled dequantisation (exact in float64).
# --------------------------------------------------------------------------

def unpack_fp4(packed) -> np.ndarray:
    """[rows, cols/2] bytes -> [rows, cols] 4-bit codes. Reading R8: the low
    nibble holds the even column."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = p & 0x0F
    hi = p >> 4
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def _decode(fn, codes, ncodes: int) -> np.ndarray:
    """Apply a per-code decoder to an array of codes by decoding each of the
    ``ncodes`` possible codes once and indexing (same values as calling
    ``fn`` element by element)."""
    table = fn(np.arange(ncodes))
    return table[np.asarray(codes, dtype=np.intp)]


def dequant(w: dict, e: int, rows=None) -> np.ndarray:
    """Dense float64 [rows, cols] of expert ``e`` of projection ``w``.

    ``w`` holds ``format`` (one of FORMATS), ``data`` ([count, rows, bytes per
    row] uint8, or uint16 BF16 bits), ``scales``, ``tensor_scale``, ``rows``,
    ``cols``, ``count``. ``rows`` optionally selects output rows.

      mxfp4:        W = e2m1(q) * e8m0(s[r, c // 32])
      nvfp4:        W = e2m1(q) * e4m3(s[r, c // 16]) * tensor_scale[e]
      fp8_rowscale: W = e4m3(q) * rowscale[r]
      bf16:         W = bf16(q)

    Group sizes and scale counts follow "forward_k3.rs" (E8M0 guard comment
    and ``k3_e8m0_needs_per_token``: ``inter*h/16`` E4M3 bytes against
    ``inter*h/32`` E8M0 bytes); the per-expert ``scale2_vals`` of the NVFP4
    branches give the tensor scale (reading R10); reading R11 gives the FP8
    row scale.
    """
    fmt = w["format"]
    sel = slice(None) if rows is None else np.asarray(rows)
    data = np.asarray(w["data"][e])[sel]
    cols = int(w["cols"])
    if fmt == "bf16":
        return bf16_to_f64(data)
    if fmt == "fp8_rowscale":
        rs = np.asarray(w["scales"][e], dtype=np.float64)[sel]
        return _decode(e4m3fn_to_f64, data, 256) * rs[:, None]
    vals = _decode(e2m1_to_f64, unpack_fp4(data), 16)
    sc = np.asarray(w["scales"][e])[sel]
    nrows = vals.shape[0]
    if fmt == "mxfp4":
        s = _decode(e8m0_to_f64, sc, 256)
        return (vals.reshape(nrows, cols // 32, 32) * s[:, :, None]).reshape(nrows, cols)
    if fmt == "nvfp4":
        s = _decode(e4m3fn_to_f64, sc, 256)
        ts = float(np.asarray(w["tensor_scale"], dtype=np.float64)[e])
        return (vals.reshape(nrows, cols // 16, 16) * (s * ts)[:, :, None]).reshape(nrows, cols)
    raise ValueError(f"unknown format {fmt!r}")


# --------------------------------------------------------------------------
# Router and routing.
# --------------------------------------------------------------------------

def router_matrix(router: dict) -> np.ndarray:
    """The router as FP64 [E + Z, H]: the BF16 ``weight``, or the dequantised
    NVFP4 ``weight_q`` (a projection dict with count 1), the router GEMV and
    GEMM that "forward_k3.rs", "forward_atomic_c4.rs" and "forward_ep.rs"
    take when the layer has an NVFP4 gate (reading R17)."""
    if router.get("weight_q") is not None:
        return dequant(router["weight_q"], 0)
    return bf16_to_f64(np.asarray(router["weight"]))


def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """z[t, e] = sum_h x[t, h] * Wr[e, h]: one projection for all N tokens
    ("forward_k3.rs" step 1, the gate GEMV that reads the router once for
    the batch; "forward_batched.rs", one gate GEMM with M = N)."""
    return np.asarray(x, np.float64) @ np.asarray(wr, np.float64).T


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Softmax over each row (all router columns)."""
    z = np.asarray(z, np.float64)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)


def selection_scores(z: np.ndarray, scoring: str, bias=None) -> np.ndarray:
    """Score used to pick the experts: the logit for softmax routing,
    softmax(logit) + correction bias for the softmax+bias arm, or
    sigmoid(logit) + correction bias for sigmoid routing ("forward_k3.rs"
    step 2, sigmoid+bias for DeepSeek-V3-style routers; "forward_batched.rs",
    router_bias_one; readings R2, R3, R14)."""
    z = np.asarray(z, np.float64)
    if scoring == "softmax":
        if bias is not None:
            return softmax_rows(z) + np.asarray(bias, np.float64)[None, :]
        return z.copy()
    if scoring == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-z))
        if bias is not None:
            s = s + np.asarray(bias, np.float64)[None, :]
        return s
    raise ValueError(f"unknown scoring {scoring!r}")


def route(z: np.ndarray, k: int, scoring: str, bias=None,
          renorm: bool = True, rsf: float = 1.0):
    """Top-k routing for every token ("forward_k3.rs" step 2 and
    "forward_atomic_c4.rs": ``moe_topk_{sigmoid,softmax}_batched`` with
    ``norm_topk_prob`` and ``routed_scaling_factor``).

    Returns ``idx`` [N, k] int64 in descending score order (lowest index first
    among equal scores, reading R6) and ``w`` [N, k] float64.
    """
    z = np.asarray(z, np.float64)
    n, num_e = z.shape
    s = selection_scores(z, scoring, bias)
    idx = np.empty((n, k), dtype=np.int64)
    w = np.empty((n, k), dtype=np.float64)
    ar = np.arange(num_e)
    for t in range(n):
        # primary key: score descending; secondary: index ascending
        order = np.lexsort((ar, -s[t]))
        sel = order[:k]
        idx[t] = sel
        w[t] = routing_weights(z[t], sel, scoring, renorm, rsf)
    return idx, w


def routing_weights(zt: np.ndarray, sel, scoring: str, renorm: bool, rsf: float) -> np.ndarray:
    """Weights of the chosen experts ``sel`` of one token: softmax over all
    router columns (softmax) or sigmoid of the chosen logits (sigmoid), no
    bias (R1, R3), then w /= sum w (with renorm) and times rsf (R5)."""
    zt = np.asarray(zt, np.float64)
    if scoring == "softmax":
        p = np.exp(zt - zt.max())
        p = p / p.sum()
        wt = p[sel]
    else:
        wt = 1.0 / (1.0 + np.exp(-zt[sel]))
    if renorm:
        wt = wt / wt.sum()
    return wt * rsf


def route_hash(z: np.ndarray, tid2eid, token_ids, k: int, scoring: str,
               renorm: bool = True, rsf: float = 1.0):
    """Hash routing ("forward_batched.rs", the hash-routing branch, reading
    R15): token t takes the experts ``tid2eid[token_ids[t], :k]`` in that
    order, weighted by :func:`routing_weights`."""
    z = np.asarray(z, np.float64)
    table = np.asarray(tid2eid, np.int64)
    ids = np.asarray(token_ids, np.int64)
    n = z.shape[0]
    idx = table[ids, :k].copy()
    w = np.empty((n, k), dtype=np.float64)
    for t in range(n):
        w[t] = routing_weights(z[t], idx[t], scoring, renorm, rsf)
    return idx, w


# --------------------------------------------------------------------------
# Experts.
# --------------------------------------------------------------------------

def silu(v):
    """silu(v) = v / (1 + exp(-v))."""
    v = np.asarray(v, np.float64)
    return v / (1.0 + np.exp(-v))


def swiglu_expert(wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, xt: np.ndarray):
    """One expert on one token x (a vector) or on several (rows of a
    matrix): g = Wg x, u = Wu x, a = silu(g) * u, d = Wd a (the gate+up then
    silu+down kernel pair named on every page). Returns (g, u, a, d), one row
    per token when xt is a matrix."""
    g = xt @ wg.T
    u = xt @ wu.T
    a = silu(g) * u
    d = a @ wd.T
    return g, u, a, d


def shared_gate_weight(x: np.ndarray, w_sg) -> np.ndarray:
    """Per-token weight of the shared expert ("forward_k3.rs", the EP
    all-reduce block: without a shared-expert gate weight the shared output is
    added by a residual add, with one it goes through the batched blend with
    a sigmoid gate): gamma[t] = sigmoid(x[t] . w_sg), or 1 without a gate
    (reading R12)."""
    x = np.asarray(x, np.float64)
    if w_sg is None:
        return np.ones(x.shape[0])
    g = x @ np.asarray(w_sg, np.float64)
    return 1.0 / (1.0 + np.exp(-g))


def moe_forward(cfg: dict, layer: dict, x_bits, rows=None, expert_range=None,
                token_ids=None) -> dict:
    """The whole layer for N tokens, in float64.

    ``cfg`` keys: H, I, E, k, I_s, scoring ('softmax' | 'sigmoid'), renorm,
    rsf. ``layer`` holds ``router`` {weight: BF16 bits [E, H], bias: [E] or
    None}, ``experts`` {gate, up, down} and ``shared`` (same, count 1) or None,
    each projection a dict as taken by :func:`dequant`. ``x_bits`` is the BF16
    bit pattern of the [N, H] input. ``rows`` optionally restricts the output
    to those hidden rows (the down projections then use only those rows).
    ``expert_range`` = (lo, hi) computes one expert-parallel share instead
    (reading R13): only slots with lo <= idx < hi contribute, the layer's
    ``experts`` hold experts lo..hi-1 only, and there is no shared term.
    ``cfg["Z"]`` zero experts widen the router (R16); a router with a
    ``tid2eid`` table routes by the tokens' ``token_ids`` (R15).

    y[t] = sum_j w[t, j] * d_{idx[t, j]}(x_t) + gamma[t] * s(x_t)   (R12)

    Besides y, the result holds ``y_sq``: for every output element, the sum
    of the squares of the terms it adds up, w[t, j] * Wd[r, i] * a_i over the
    routed slots and gamma[t] * Wsd[r, i] * as_i for the shared expert. It is
    not part of the layer; it sizes an error. Were every intermediate
    activation a_i (and as_i) scaled by its own independent factor
    (1 + delta_i) with mean 0 and variance v, y[r] would move by a zero-mean
    amount of variance v * y_sq[r] (a sum of independent terms), which is what
    storing the activations in a narrower format does.
    """
    x = bf16_to_f64(np.asarray(x_bits))
    n, h = x.shape
    assert h == cfg["H"]
    wr = router_matrix(layer["router"])
    bias = layer["router"].get("bias")
    bias = None if bias is None else np.asarray(bias, np.float64)
    z = router_logits(x, wr)
    if layer["router"].get("tid2eid") is not None:
        idx, w = route_hash(z, layer["router"]["tid2eid"], token_ids, cfg["k"], cfg["scoring"],
                            cfg["renorm"], cfg["rsf"])
    else:
        idx, w = route(z, cfg["k"], cfg["scoring"], bias, cfg["renorm"], cfg["rsf"])

    out_rows = np.arange(h) if rows is None else np.asarray(rows)
    k = cfg["k"]
    ex = layer["experts"]
    a_slots = np.zeros((n, k, cfg["I"]), dtype=np.float64)
    d_slots = np.zeros((n, k, out_rows.size), dtype=np.float64)
    sq_slots = np.zeros((n, k, out_rows.size), dtype=np.float64)
    # one expert's weights at a time (dequantised once for all of its slots)
    lo, hi = (0, cfg["E"]) if expert_range is None else expert_range
    for e in np.unique(idx):
        if not lo <= e < hi:
            continue  # a zero expert (e >= E) or another share's expert: nothing
        wg, wu = dequant(ex["gate"], int(e) - lo), dequant(ex["up"], int(e) - lo)
        wd = dequant(ex["down"], int(e) - lo, rows=out_rows)
        ts, js = np.nonzero(idx == e)
        _, _, a, d = swiglu_expert(wg, wu, wd, x[ts])
        a_slots[ts, js] = a
        d_slots[ts, js] = d
        sq_slots[ts, js] = (a * a) @ (wd * wd).T  # sum_i (Wd[r, i] a_i)^2
    y = np.zeros((n, out_rows.size), dtype=np.float64)
    y_sq = np.zeros((n, out_rows.size), dtype=np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * d_slots[:, j]
        y_sq += (w[:, j:j + 1] ** 2) * sq_slots[:, j]
    s_out = None
    gamma = None
    if expert_range is None and layer.get("shared") is not None and cfg.get("I_s", 0) > 0:
        sh = layer["shared"]
        wg = dequant(sh["gate"], 0)
        wu = dequant(sh["up"], 0)
        wd = dequant(sh["down"], 0, rows=out_rows)
        _, _, a_s, s_out = swiglu_expert(wg, wu, wd, x)
        gamma = shared_gate_weight(x, None if layer["router"].get("shared_gate") is None
                                   else bf16_to_f64(layer["router"]["shared_gate"]))
        y = y + gamma[:, None] * s_out
        y_sq = y_sq + (gamma[:, None] ** 2) * ((a_s * a_s) @ (wd * wd).T)
    return {"y": y, "y_sq": y_sq, "z": z, "idx": idx, "w": w, "a": a_slots,
            "shared": s_out, "gamma": gamma, "rows": out_rows}


# --------------------------------------------------------------------------
# Grouping by expert.
# --------------------------------------------------------------------------

def group_slots(idx, num_experts: int, pad: int = 16, expert_range=None) -> dict:
    """Order of the N*k routing slots when the batch is grouped by expert
    ("forward_batched.rs", ``MoeLayer::forward_batched``: the grouped FP8
    decode comment, each expert streamed once for all of its rows; the
    prefill workload sorts tokens per expert and pads each expert to 16-row
    tiles).

    Slot s = t*k + j is token t's j-th choice. Experts are laid out in
    ascending order, each starting at a multiple of ``pad`` rows; within an
    expert the slots keep ascending slot order (a stable sort by expert).
    Rows past an expert's count up to its padded size are padding (-1).

    ``expert_range`` = (lo, hi) groups one expert-parallel share (reading
    R13): only slots whose expert lies in [lo, hi) are placed, experts are
    numbered locally (e - lo), and the other slots get inv = -1.

    Returns counts [E_local], offsets [E_local+1] (padded starts), perm_slot
    and perm_tok [offsets[-1]] (-1 on padding), inv [N*k] (row of each slot)
    and units (local experts with at least one slot, ascending).
    """
    idx = np.asarray(idx, dtype=np.int64)
    n, k = idx.shape
    lo, hi = (0, num_experts) if expert_range is None else expert_range
    flat = idx.reshape(-1)
    counts = np.zeros(hi - lo, dtype=np.int64)
    for e in flat:
        if lo <= e < hi:
            counts[e - lo] += 1
    padded = (counts + pad - 1) // pad * pad
    offsets = np.zeros(hi - lo + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    perm_slot = np.full(offsets[-1], -1, dtype=np.int64)
    perm_tok = np.full(offsets[-1], -1, dtype=np.int64)
    inv = np.full(n * k, -1, dtype=np.int64)
    fill = offsets[:-1].copy()
    for s in range(n * k):  # ascending slot order: a stable counting sort
        if not lo <= flat[s] < hi:
            continue
        e = flat[s] - lo
        perm_slot[fill[e]] = s
        perm_tok[fill[e]] = s // k
        inv[s] = fill[e]
        fill[e] += 1
    units = np.nonzero(counts)[0]
    return {"counts": counts, "offsets": offsets, "perm_slot": perm_slot,
            "perm_tok": perm_tok, "inv": inv, "units": units}
