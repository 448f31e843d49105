"""ctypes binding of libmoe_mi355x.so (argument marshalling only).

Every step of the layer runs in the library's HIP kernels; this module only
turns torch tensors into the C structs of ``include/moe_mi355x.h``. It raises
if the library has not been built: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
SCORING = {"softmax": 0, "sigmoid": 1}
ACCUM = {"slot": 0, "atomic": 1}
PATH = {"auto": 0, "decode": 1, "grouped": 2}
FORMAT = {"bf16": 0, "fp8_rowscale": 1, "mxfp4": 2, "nvfp4": 3}

EXPORTED = ("moe_abi_version", "moe_last_error", "moe_status_str", "moe_workspace_bytes",
            "moe_validate", "moe_num_launches", "moe_group_layout", "moe_forward",
            "moe_forward_ep_partial", "moe_forward_no_alloc")


class MoeCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("scoring", ctypes.c_int32),
                ("norm_topk_prob", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("accum_mode", ctypes.c_int32), ("path", ctypes.c_int32),
                ("zero_experts", ctypes.c_int32)]


class MoeRouter(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("shared_gate", ctypes.c_void_p), ("tid2eid", ctypes.c_void_p),
                ("vocab", ctypes.c_int32), ("token_ids", ctypes.c_void_p),
                ("weight_q", ctypes.c_void_p)]


class MoeWeight(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("data_bytes", ctypes.c_size_t), ("scales", ctypes.c_void_p),
                ("scale_bytes", ctypes.c_size_t), ("tensor_scale", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("count", ctypes.c_int32)]


class MoeExperts(ctypes.Structure):
    _fields_ = [("gate", MoeWeight), ("up", MoeWeight), ("down", MoeWeight)]


class MoeTopkOut(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("weights", ctypes.c_void_p),
                ("logits", ctypes.c_void_p)]


class MoeTrace(ctypes.Structure):
    _fields_ = [("events", ctypes.c_void_p), ("count", ctypes.c_int32)]


class MoeGroupView(ctypes.Structure):
    _fields_ = [("info", ctypes.c_size_t), ("perm_tok", ctypes.c_size_t),
                ("perm_slot", ctypes.c_size_t), ("inv", ctypes.c_size_t),
                ("rows", ctypes.c_int32)]


_lib = None


def _torch():
    import torch
    return torch


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_35_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_abi_version.restype = ctypes.c_int32
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(MoeCfg), ctypes.c_int32]
        L.moe_validate.restype = ctypes.c_int
        L.moe_validate.argtypes = [ctypes.POINTER(MoeCfg), ctypes.POINTER(MoeRouter),
                                   ctypes.POINTER(MoeExperts), ctypes.POINTER(MoeExperts),
                                   ctypes.c_int32, ctypes.c_size_t]
        L.moe_group_layout.restype = ctypes.c_int
        L.moe_group_layout.argtypes = [ctypes.POINTER(MoeCfg), ctypes.c_int32,
                                       ctypes.POINTER(MoeGroupView)]
        L.moe_num_launches.restype = ctypes.c_int32
        L.moe_num_launches.argtypes = [ctypes.POINTER(MoeCfg), ctypes.c_int32]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward.argtypes = [ctypes.POINTER(MoeCfg), ctypes.POINTER(MoeRouter),
                                  ctypes.POINTER(MoeExperts), ctypes.POINTER(MoeExperts),
                                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.POINTER(MoeTopkOut), ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.POINTER(MoeTrace)]
        L.moe_forward_ep_partial.restype = ctypes.c_int
        L.moe_forward_ep_partial.argtypes = [
            ctypes.POINTER(MoeCfg), ctypes.POINTER(MoeRouter), ctypes.POINTER(MoeExperts),
            ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(MoeExperts), ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(MoeTopkOut), ctypes.c_void_p,
            ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(MoeTrace)]
        L.moe_forward_no_alloc.restype = ctypes.c_int
        L.moe_forward_no_alloc.argtypes = [
            ctypes.POINTER(MoeCfg), ctypes.POINTER(MoeRouter), ctypes.POINTER(MoeExperts),
            ctypes.POINTER(MoeExperts), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
            ctypes.POINTER(MoeTopkOut), ctypes.c_void_p, ctypes.POINTER(MoeTrace)]
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def last_error() -> str:
    return lib().moe_last_error().decode()


def abi_version() -> int:
    return int(lib().moe_abi_version())


# ------------------------------------------------------------------ structs

def make_cfg(cfg: dict, accum: str | None = None, path: str = "auto") -> MoeCfg:
    c = MoeCfg()
    c.hidden = cfg["H"]
    c.inter = cfg["I"]
    c.num_experts = cfg["E"]
    c.top_k = cfg["k"]
    c.shared_inter = cfg.get("I_s", 0) or 0
    c.scoring = SCORING[cfg["scoring"]]
    c.norm_topk_prob = 1 if cfg["renorm"] else 0
    c.routed_scaling_factor = float(cfg["rsf"])
    c.accum_mode = ACCUM[accum or cfg.get("accum", "slot")]
    c.path = PATH[path]
    c.zero_experts = cfg.get("Z", 0) or 0
    return c


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def make_weight(p: dict) -> MoeWeight:
    w = MoeWeight()
    w.format = FORMAT[p["format"]]
    w.data = _ptr(p["data"])
    w.data_bytes = _nbytes(p["data"])
    w.scales = _ptr(p.get("scales"))
    w.scale_bytes = _nbytes(p.get("scales"))
    w.tensor_scale = _ptr(p.get("tensor_scale"))
    w.rows, w.cols, w.count = p["rows"], p["cols"], p["count"]
    return w


def make_experts(s: dict | None) -> MoeExperts | None:
    if s is None:
        return None
    e = MoeExperts()
    e.gate = make_weight(s["gate"])
    e.up = make_weight(s["up"])
    e.down = make_weight(s["down"])
    return e


def slice_experts(s: dict, lo: int, hi: int) -> dict:
    """Experts lo..hi-1 of a packed set: views of the same device tensors
    (the expert index is the leading dimension of every array)."""
    out = {}
    for name in ("gate", "up", "down"):
        p = dict(s[name])
        for key in ("data", "scales", "tensor_scale"):
            if p.get(key) is not None:
                p[key] = p[key][lo:hi]
        p["count"] = hi - lo
        out[name] = p
    return out


def make_router(r: dict) -> MoeRouter:
    m = MoeRouter()
    m.weight = _ptr(r["weight"])
    m.bias = _ptr(r.get("bias"))
    m.shared_gate = _ptr(r.get("shared_gate"))
    table = r.get("tid2eid")
    if table is not None:
        m.tid2eid = _ptr(table)
        m.vocab = int(table.shape[0])
    if r.get("weight_q") is not None:
        # the struct must outlive every call: it rides on the router object
        m._weight_q = make_weight(r["weight_q"])
        m.weight_q = ctypes.addressof(m._weight_q)
    return m


def _ref(obj):
    return None if obj is None else ctypes.byref(obj)


# ------------------------------------------------------------------ calls

def workspace_bytes(cfg: MoeCfg, max_tokens: int) -> int:
    n = lib().moe_workspace_bytes(ctypes.byref(cfg), int(max_tokens))
    if n == 0:
        raise MoeError(MOE_ERR_INVALID_ARG, last_error())
    return int(n)


def num_launches(cfg: MoeCfg, n_tokens: int) -> int:
    return int(lib().moe_num_launches(ctypes.byref(cfg), int(n_tokens)))


def group_layout(cfg: MoeCfg, n_tokens: int) -> MoeGroupView:
    v = MoeGroupView()
    st = lib().moe_group_layout(ctypes.byref(cfg), int(n_tokens), ctypes.byref(v))
    if st != MOE_OK:
        raise MoeError(st, last_error())
    return v


def validate(cfg: MoeCfg, router: MoeRouter, experts: MoeExperts, shared: MoeExperts | None,
             n_tokens: int, ws_bytes: int) -> int:
    return int(lib().moe_validate(ctypes.byref(cfg), ctypes.byref(router), _ref(experts),
                                  _ref(shared), int(n_tokens), int(ws_bytes)))


class Layer:
    """A packed layer (dict of device tensors from ``synth.make_layer`` or the
    caller's own) bound to the C structs, plus its workspace."""

    def __init__(self, layer: dict, max_tokens: int, accum: str | None = None,
                 path: str = "auto"):
        import torch
        self.layer = layer
        self.cfg = make_cfg(layer["cfg"], accum, path)
        self.router = make_router(layer["router"])
        self.experts = make_experts(layer["experts"])
        self.shared = make_experts(layer["shared"])
        self.max_tokens = max_tokens
        nbytes = workspace_bytes(self.cfg, max_tokens)
        dev = layer["experts"]["gate"]["data"].device
        # zero-filled once: the counter head must start at zero (calls keep it so)
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=dev)

    def prepare(self, x, out, idx=None, weights=None, logits=None, stream=None, events=None,
                share=None, with_shared=False, token_ids=None):
        """Marshal one call's arguments once; returns a no-argument callable
        that enqueues the call (raises MoeError on a refused call).

        share=(lo, hi) makes it an expert-parallel share (moe_forward_ep_partial):
        only experts lo..hi-1 are computed, out is FP32 [N, H], and the shared
        expert's term is added only if with_shared. token_ids: device int32
        [N] for a layer with a hash-routing table."""
        import torch
        n = x.shape[0]
        topk = None
        if idx is not None or weights is not None or logits is not None:
            topk = MoeTopkOut(_ptr(idx), _ptr(weights), _ptr(logits))
        trace = None
        keep = []
        if events is not None:
            arr = (ctypes.c_void_p * len(events))(*[int(e) for e in events])
            keep.append(arr)
            trace = MoeTrace(ctypes.cast(arr, ctypes.c_void_p), len(events))
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        router = self.router
        if token_ids is not None:
            # the ids are per call: this call gets its own copy of the router
            router = MoeRouter.from_buffer_copy(self.router)
            router.token_ids = _ptr(token_ids)
            keep += [router, token_ids]
        tail = (ctypes.c_void_p(x.data_ptr()), ctypes.c_int32(n),
                ctypes.c_void_p(out.data_ptr()), _ref(topk),
                ctypes.c_void_p(self.workspace.data_ptr()),
                ctypes.c_size_t(self.workspace.numel()), ctypes.c_void_p(stream), _ref(trace))
        if share is None:
            fn = lib().moe_forward
            args = (ctypes.byref(self.cfg), ctypes.byref(router), _ref(self.experts),
                    _ref(self.shared)) + tail
        else:
            lo, hi = int(share[0]), int(share[1])
            local = make_experts(slice_experts(self.layer["experts"], lo, hi))
            keep.append(local)
            fn = lib().moe_forward_ep_partial
            args = (ctypes.byref(self.cfg), ctypes.byref(router), _ref(local),
                    ctypes.c_int32(lo), ctypes.c_int32(hi),
                    _ref(self.shared if with_shared else None)) + tail
        keep += [topk, trace, x, out, idx, weights, logits]

        def call():
            st = fn(*args)
            if st != MOE_OK:
                raise MoeError(st, last_error())
            return keep
        return call

    def forward_no_alloc(self, x, out=None, idx=None, weights=None, logits=None, stream=None,
                         token_ids=None):
        """The layer forward through moe_forward_no_alloc: the library's static
        device scratch instead of this object's workspace."""
        import torch
        if out is None:
            out = torch.empty_like(x)
        topk = None
        if idx is not None or weights is not None or logits is not None:
            topk = MoeTopkOut(_ptr(idx), _ptr(weights), _ptr(logits))
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        router = self.router
        if token_ids is not None:
            router = MoeRouter.from_buffer_copy(self.router)
            router.token_ids = _ptr(token_ids)
        st = lib().moe_forward_no_alloc(ctypes.byref(self.cfg), ctypes.byref(router),
                                        _ref(self.experts), _ref(self.shared),
                                        ctypes.c_void_p(x.data_ptr()), ctypes.c_int32(x.shape[0]),
                                        ctypes.c_void_p(out.data_ptr()), _ref(topk),
                                        ctypes.c_void_p(stream), None)
        if st != MOE_OK:
            raise MoeError(st, last_error())
        return out

    def num_launches(self, n_tokens: int) -> int:
        return num_launches(self.cfg, n_tokens)

    def grouping(self, n_tokens: int) -> dict:
        """The grouping step's result of the last grouped-path call with
        n_tokens tokens, read from the workspace (host NumPy int32 arrays)."""
        v = group_layout(self.cfg, n_tokens)
        ws = self.workspace
        k = self.cfg.top_k

        def arr(off, count):
            return ws[off:off + 4 * count].view(dtype=_torch().int32).cpu().numpy()
        info = arr(v.info, 32 + 3 * 256)
        return {"U": int(info[0]), "M": int(info[1]), "uexp": info[32:288],
                "ubase": info[288:544], "ucount": info[544:800],
                "perm_tok": arr(v.perm_tok, v.rows), "perm_slot": arr(v.perm_slot, v.rows),
                "inv": arr(v.inv, n_tokens * k)}

    def forward(self, x, out=None, idx=None, weights=None, logits=None, stream=None,
                events=None, token_ids=None):
        import torch
        if out is None:
            out = torch.empty_like(x)
        self.prepare(x, out, idx, weights, logits, stream, events, token_ids=token_ids)()
        return out

    def forward_share(self, x, lo: int, hi: int, with_shared=False, out=None, idx=None,
                      weights=None, logits=None, stream=None, events=None, token_ids=None):
        """One expert-parallel share: FP32 [N, H] partial output of experts
        lo..hi-1 (plus the shared expert's term if with_shared)."""
        import torch
        if out is None:
            out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
        self.prepare(x, out, idx, weights, logits, stream, events, share=(lo, hi),
                     with_shared=with_shared, token_ids=token_ids)()
        return out
