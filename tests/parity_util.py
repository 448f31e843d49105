"""Shared helpers for the GPU parity tests: tie-free token filter (through
the oracle), running the HIP path, and the comparison bar."""

import numpy as np
import torch

import synth
from oracle import (bf16_to_f64, group_slots, moe_forward, route, route_hash, router_logits,
                    router_matrix, selection_scores)

# consecutive gap among the top k+1 selection scores; about 100x the FP32
# error of a router logit at H = 7168
TIE_GAP = 1e-3
# per-token relative L2 error of the BF16 output
OUT_RTOL = 1e-2
# routing weights
W_RTOL = 1e-5
# Element-wise bar. Both HIP paths keep every intermediate in FP32 except
# the SwiGLU activations a (routed and shared), which are stored in BF16 on
# their way from the gate+up step to the down step, and the output, which is
# rounded to BF16. Round to nearest even with 8 significant bits scales each
# a_i by (1 + delta_i), |delta_i| <= U_BF16, and for values spread over a
# binade the delta_i are independent with mean 0 and variance below
# U_BF16^2 / 3. So an output element moves by a zero-mean amount of variance
# below (U_BF16^2 / 3) * y_sq (the oracle's sum of squared terms of that
# element), and its own rounding adds at most U_BF16 * |y|. FP32
# accumulation over K <= 7168 terms adds about sqrt(K) * 2^-24 relative to the
# same scale, four orders of magnitude less. The bar allows ELEM_Z standard
# deviations: a 1-in-10^11 event per element for a Gaussian, and the error is
# a sum of many bounded terms, whose tails are lighter still.
U_BF16 = 2.0 ** -8
ELEM_Z = 7.0


def tie_free_filter(npl, gap=TIE_GAP):
    cfg = npl["cfg"]
    wr = router_matrix(npl["router"])
    bias = npl["router"]["bias"]
    k = cfg["k"]

    def accept(x_cpu):
        xb = x_cpu.view(torch.int16).numpy().view(np.uint16)
        s = selection_scores(router_logits(bf16_to_f64(xb), wr), cfg["scoring"], bias)
        srt = -np.sort(-s, axis=1)[:, :min(k + 1, s.shape[1])]
        if srt.shape[1] < 2:
            return np.ones(s.shape[0], bool)
        return (np.diff(-srt, axis=1) >= gap).all(axis=1)

    return accept


def bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def run_hip(layer, x, accum=None, out=None, path="auto", token_ids=None):
    from mixture_experts_layer_35_amd import Layer
    n = x.shape[0]
    cfg = layer["cfg"]
    L = Layer(layer, n, accum=accum, path=path)
    dev = x.device
    idx = torch.full((n, cfg["k"]), 0xFFFF, dtype=torch.int32, device=dev)
    w = torch.full((n, cfg["k"]), float("nan"), dtype=torch.float32, device=dev)
    width = cfg["E"] + cfg.get("Z", 0)
    logits = torch.full((n, width), float("nan"), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.full_like(x, float("nan"))
    L.forward(x, out=out, idx=idx, weights=w, logits=logits, token_ids=token_ids)
    torch.cuda.synchronize()
    assert device_error(L) == 0, "a workgroup wait expired"
    return out, idx, w, logits, L


def device_error(L):
    """The sticky error word at bytes 128..131 of the workspace."""
    return int(L.workspace[128:132].view(torch.int32).item())


def rel_l2_per_token(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    num = np.linalg.norm(got - want, axis=1)
    den = np.linalg.norm(want, axis=1)
    return num / den


def elementwise_bound(y, y_sq, rounded_output=True):
    """Largest allowed |got - y| per element (see ELEM_Z): ELEM_Z standard
    deviations of the BF16 hand-off of the activations, plus the BF16 output
    rounding when the output is BF16."""
    y = np.asarray(y, np.float64)
    b = ELEM_Z * (U_BF16 / np.sqrt(3.0)) * np.sqrt(np.asarray(y_sq, np.float64))
    if rounded_output:
        b = b + U_BF16 * np.abs(y)
    return b


def assert_elementwise(got, y, y_sq, label, rounded_output=True):
    """Every element within elementwise_bound; returns the largest ratio of
    error to bound."""
    got = np.asarray(got, np.float64)
    y = np.asarray(y, np.float64)
    bound = elementwise_bound(y, y_sq, rounded_output)
    diff = np.abs(got - y)
    bad = diff > bound
    if bad.any():
        t, r = np.argwhere(bad)[0]
        raise AssertionError(
            f"{label}: {int(bad.sum())} of {bad.size} elements off, e.g. [{t}, {r}]: "
            f"got {got[t, r]!r}, want {y[t, r]!r}, bound {bound[t, r]!r}")
    return float((diff / np.where(bound > 0, bound, 1.0)).max())


def assert_same_up_to_order(a, b, y_sq, label):
    """Two BF16 outputs of the FP32-atomic mode for the same input. The
    atomic adds land in a different order each run, so the FP32 sums may
    differ by reassociation, about sqrt(K) * 2^-24 * sqrt(y_sq) for K terms
    (y_sq: the oracle's sum of squared terms), and the BF16 rounding may then
    fall on either side: allowed, one BF16 step of the larger value plus
    1e-4 * sqrt(y_sq), which is 30 times the reassociation error at K = 2^16."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    tol = np.maximum(np.abs(a), np.abs(b)) * 2.0 ** -7 + 1e-4 * np.sqrt(np.asarray(y_sq))
    bad = np.abs(a - b) > tol
    assert not bad.any(), (f"{label}: {int(bad.sum())} elements differ, e.g. "
                           f"{a[bad][:3]} vs {b[bad][:3]}")


def check_grouping(L, n, ref_idx, num_experts, expert_range=None):
    """The grouped path's permutation against the oracle's, bit for bit
    (of one expert-parallel share's experts, with ``expert_range``)."""
    g = L.grouping(n)
    ref = group_slots(ref_idx, num_experts, pad=16,
                      expert_range=(0, num_experts) if expert_range is None else expert_range)
    units = ref["units"]
    U = len(units)
    assert g["U"] == U, (g["U"], U)
    assert g["M"] == ref["offsets"][-1]
    assert np.array_equal(g["uexp"][:U], units)
    assert np.array_equal(g["ubase"][:U], ref["offsets"][units])
    assert np.array_equal(g["ucount"][:U], ref["counts"][units])
    M = g["M"]
    assert np.array_equal(g["perm_slot"][:M], ref["perm_slot"])
    assert np.array_equal(g["perm_tok"][:M], ref["perm_tok"])
    assert np.array_equal(g["inv"], ref["inv"])


def check_against_oracle(layer, x, accum=None, rows=None, label="", path="auto", tokens=None,
                         token_ids=None):
    """Run the HIP path and the oracle on the same inputs and assert the
    bar: indices bit-exact, weights within W_RTOL, logits within 1e-5 (abs,
    relative to their scale), every output element within elementwise_bound
    and per-token relative L2 of the output within OUT_RTOL; on the grouped
    path also the grouping, bit for bit.

    ``rows`` restricts the output check to those hidden rows and ``tokens``
    to those tokens (the oracle's expert work then covers only them; routing
    is still checked for every token). Returns the measured errors."""
    npl = synth.as_numpy(layer)
    cfg = npl["cfg"]
    xb = bits(x)
    n = xb.shape[0]
    out, idx, w, logits, L = run_hip(layer, x, accum=accum, path=path, token_ids=token_ids)
    ids = None if token_ids is None else token_ids.cpu().numpy()
    # routing of every token
    z = router_logits(bf16_to_f64(xb), router_matrix(npl["router"]))
    if npl["router"].get("tid2eid") is not None:
        ref_idx, ref_w = route_hash(z, npl["router"]["tid2eid"], ids, cfg["k"], cfg["scoring"],
                                    cfg["renorm"], cfg["rsf"])
    else:
        ref_idx, ref_w = route(z, cfg["k"], cfg["scoring"], npl["router"]["bias"],
                               cfg["renorm"], cfg["rsf"])
    got_idx = idx.cpu().numpy().astype(np.int64)
    assert np.array_equal(got_idx, ref_idx), f"{label}: indices differ\n{got_idx}\n{ref_idx}"
    got_w = w.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got_w, ref_w, rtol=W_RTOL, atol=0, err_msg=label)
    got_z = logits.cpu().numpy().astype(np.float64)
    zscale = np.abs(z).max()
    assert np.abs(got_z - z).max() <= 1e-5 * max(1.0, zscale), label
    grouped = L.num_launches(n) > 1
    if grouped:
        check_grouping(L, n, ref_idx, cfg["E"])
    o = bf16_to_f64(bits(out))
    assert np.isfinite(o).all(), f"{label}: non-finite output (unwritten rows?)"
    tok = np.arange(n) if tokens is None else np.asarray(tokens)
    ref = moe_forward(cfg, npl, xb[tok], rows=rows, token_ids=None if ids is None else ids[tok])
    sel = ref["rows"]
    err = rel_l2_per_token(o[tok][:, sel], ref["y"])
    assert err.max() <= OUT_RTOL, f"{label}: rel L2 {err}"
    ratio = assert_elementwise(o[tok][:, sel], ref["y"], ref["y_sq"], label)
    assert device_error(L) == 0, f"{label}: device error word set"
    return {"rel_l2": float(err.max()), "elem_ratio": ratio, "out": out, "grouped": grouped}


# ---- guard regions after the caller's buffers ---------------------------
# 0xFF bytes: NaN in BF16, FP8 E4M3, E8M0, E4M3 and FP32; -6 in FP4 E2M1.

GUARD = 4096  # bytes of 0xFF after each buffer


class Guards:
    """Copies tensors into allocations with a 0xFF tail and remembers them."""

    def __init__(self):
        self.bufs = []

    def wrap(self, t):
        if t is None:
            return None
        t = t.contiguous()
        nb = t.numel() * t.element_size()
        buf = torch.full((nb + GUARD,), 0xFF, dtype=torch.uint8, device=t.device)
        buf[:nb].copy_(t.view(torch.uint8).reshape(-1))
        self.bufs.append(buf)
        return buf[:nb].view(t.dtype).view(t.shape)

    def intact(self):
        return all(bool((b[-GUARD:] == 0xFF).all().item()) for b in self.bufs)


def _guard_proj(p, G):
    if p is None:
        return None
    q = dict(p)
    for key in ("data", "scales", "tensor_scale"):
        if q.get(key) is not None:
            q[key] = G.wrap(q[key])
    return q


def guard_layer(layer, G):
    r = dict(layer["router"])
    for key in ("weight", "bias", "shared_gate", "tid2eid"):
        if r.get(key) is not None:
            r[key] = G.wrap(r[key])
    if r.get("weight_q") is not None:
        r["weight_q"] = _guard_proj(r["weight_q"], G)
    experts = {k: _guard_proj(v, G) for k, v in layer["experts"].items()}
    shared = None
    if layer["shared"] is not None:
        shared = {k: _guard_proj(v, G) for k, v in layer["shared"].items()}
    return {"cfg": layer["cfg"], "router": r, "experts": experts, "shared": shared}
