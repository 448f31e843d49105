"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and refuses bad calls by name before enqueueing anything.
No GPU: moe_validate and moe_workspace_bytes never touch device memory."""

import ctypes
import os
import re

import pytest

import mixture_experts_layer_35_amd as moe
from mixture_experts_layer_35_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "moe_mi355x.h")

FAKE = 0x7f0000000000  # never dereferenced: validation only reads sizes and alignment


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", txt)))


def test_header_symbols_exported():
    lib = moe.lib()
    names = _declared()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version():
    assert moe.abi_version() == 5


def _fake_weight(fmt, rows, cols, count, base):
    w = B.MoeWeight()
    w.format = B.FORMAT[fmt]
    w.rows, w.cols, w.count = rows, cols, count
    w.data = base
    if fmt == "bf16":
        w.data_bytes = count * rows * cols * 2
    elif fmt == "fp8_rowscale":
        w.data_bytes = count * rows * cols
        w.scales, w.scale_bytes = base + (1 << 36), count * rows * 4
    elif fmt == "mxfp4":
        w.data_bytes = count * rows * cols // 2
        w.scales, w.scale_bytes = base + (1 << 36), count * rows * cols // 32
    else:
        w.data_bytes = count * rows * cols // 2
        w.scales, w.scale_bytes = base + (1 << 36), count * rows * cols // 16
        w.tensor_scale = base + (1 << 37)
    return w


def _fake_set(fmt, H, inter, count, base):
    s = B.MoeExperts()
    s.gate = _fake_weight(fmt, inter, H, count, base)
    s.up = _fake_weight(fmt, inter, H, count, base + (1 << 32))
    s.down = _fake_weight(fmt, H, inter, count, base + (2 << 32))
    return s


def _c3():
    cfg = dict(H=7168, I=2048, E=256, k=8, I_s=2048, scoring="sigmoid", renorm=True, rsf=2.5)
    c = B.make_cfg(cfg, accum="atomic")
    r = B.MoeRouter(FAKE, FAKE + 4096)
    ex = _fake_set("nvfp4", 7168, 2048, 256, FAKE)
    sh = _fake_set("bf16", 7168, 2048, 1, FAKE + (8 << 32))
    return c, r, ex, sh


def test_valid_call_passes_validation():
    c, r, ex, sh = _c3()
    ws = B.workspace_bytes(c, 4)
    assert B.validate(c, r, ex, sh, 4, ws) == B.MOE_OK
    assert B.num_launches(c, 4) == 1


def test_workspace_too_small_names_need_and_have():
    c, r, ex, sh = _c3()
    ws = B.workspace_bytes(c, 4)
    assert B.validate(c, r, ex, sh, 4, 1) == B.MOE_ERR_WORKSPACE
    msg = B.last_error()
    need = int(re.search(r"need (\d+) bytes", msg).group(1))
    assert "have 1" in msg and 0 < need <= ws
    assert B.validate(c, r, ex, sh, 4, need - 1) == B.MOE_ERR_WORKSPACE
    assert f"need {need} bytes" in B.last_error() and f"have {need - 1}" in B.last_error()
    assert B.validate(c, r, ex, sh, 4, need) == B.MOE_OK


def test_workspace_regions():
    c, *_ = _c3()
    # the decode region is sized for the largest decode call: one size
    # serves 1..4 tokens
    assert B.workspace_bytes(c, 1) == B.workspace_bytes(c, 4)
    # the grouped region comes after it and grows with the tokens
    assert B.workspace_bytes(c, 4) < B.workspace_bytes(c, 16) < B.workspace_bytes(c, 512)
    for n in (5, 16, 512):
        v = B.group_layout(c, n)
        assert min(v.info, v.perm_tok, v.perm_slot, v.inv) >= B.workspace_bytes(c, 4)


def test_scale_byte_count_mismatch_refused():
    # the GS16-kernel-on-GS32-buffer class: a scale buffer sized for a
    # different group size is refused before anything runs
    c, r, ex, sh = _c3()
    ex.gate.scale_bytes = 256 * 2048 * 7168 // 32
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    assert "scales" in B.last_error()


def test_data_byte_count_mismatch_refused():
    c, r, ex, sh = _c3()
    ex.down.data_bytes += 16
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG


def test_misaligned_and_null_refused():
    c, r, ex, sh = _c3()
    ex.up.data = FAKE + 8
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    c, r, ex, sh = _c3()
    ex.up.data = None
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    c, r, ex, sh = _c3()
    r.weight = None
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG


def test_missing_tensor_scale_refused():
    c, r, ex, sh = _c3()
    ex.gate.tensor_scale = None
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG


def test_shape_mismatch_refused():
    c, r, ex, sh = _c3()
    ex.down = _fake_weight("nvfp4", 2048, 7168, 256, FAKE)   # transposed
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG


def test_group_size_divisibility_refused():
    cfg = dict(H=2048 + 16, I=768, E=8, k=2, I_s=0, scoring="softmax", renorm=True, rsf=1.0)
    c = B.make_cfg(cfg, accum="slot")
    ex = _fake_set("mxfp4", 2048 + 16, 768, 8, FAKE)
    st = B.validate(c, B.MoeRouter(FAKE, None), ex, None, 1, 1 << 40)
    assert st == B.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("field,val", [("top_k", 0), ("top_k", 17), ("num_experts", 257),
                                       ("hidden", 0), ("scoring", 5), ("accum_mode", 9),
                                       ("norm_topk_prob", 2)])
def test_bad_cfg_refused(field, val):
    c, r, ex, sh = _c3()
    setattr(c, field, val)
    assert B.validate(c, r, ex, sh, 4, 1 << 40) != B.MOE_OK


def test_topk_above_num_experts_refused():
    c, r, ex, sh = _c3()
    c.num_experts, c.top_k = 4, 8
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("n", [0, -1, 5000])
def test_token_count_range(n):
    c, r, ex, sh = _c3()
    assert B.validate(c, r, ex, sh, n, 1 << 40) != B.MOE_OK


def test_decode_token_limit_and_path_choice():
    c, r, ex, sh = _c3()
    c.path = B.PATH["decode"]
    assert B.validate(c, r, ex, sh, 5, 1 << 40) == B.MOE_ERR_UNSUPPORTED
    c.path = B.PATH["auto"]
    assert B.validate(c, r, ex, sh, 16, 1 << 40) == B.MOE_OK
    assert B.num_launches(c, 4) == 1      # decode: one fused kernel
    assert B.num_launches(c, 16) == 5     # grouped: router, top-k + grouping, gate+up, down, combine
    c.path = B.PATH["grouped"]
    assert B.num_launches(c, 1) == 5
    assert B.validate(c, r, ex, sh, 1, 1 << 40) == B.MOE_OK


def test_grouped_shape_limits():
    # the grouped path steps K in 128-column chunks
    c, r, ex, sh = _c3()
    c.path = B.PATH["grouped"]
    c.hidden, c.inter, c.shared_inter = 544, 192, 0
    ex = _fake_set("mxfp4", 544, 192, 256, FAKE)
    assert B.validate(c, r, ex, None, 16, 1 << 40) == B.MOE_ERR_UNSUPPORTED
    assert "multiples of 128" in B.last_error()
    c.path = B.PATH["auto"]
    assert B.validate(c, r, ex, None, 4, 1 << 40) == B.MOE_OK   # decode takes it


def test_workspace_covers_every_smaller_call():
    c, r, ex, sh = _c3()
    ws = B.workspace_bytes(c, 300)
    for n in (1, 4, 5, 16, 64, 129, 255, 300):
        assert B.validate(c, r, ex, sh, n, ws) == B.MOE_OK, n


def test_shared_presence_must_match_cfg():
    c, r, ex, sh = _c3()
    assert B.validate(c, r, ex, None, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    c.shared_inter = 0
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG


def test_shared_format_must_be_bf16_or_routed():
    c, r, ex, sh = _c3()
    sh = _fake_set("mxfp4", 7168, 2048, 1, FAKE)
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_UNSUPPORTED


def test_mixed_formats_within_set_refused():
    c, r, ex, sh = _c3()
    ex.down = _fake_weight("mxfp4", 7168, 2048, 256, FAKE)
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_UNSUPPORTED


def test_softmax_with_bias_accepted():
    # the softmax+bias arm
    c, r, ex, sh = _c3()
    c.scoring = B.SCORING["softmax"]
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_OK
    r.bias = FAKE + 4098
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG


def test_status_strings():
    assert moe.status_str(0) == "MOE_OK"
    assert moe.status_str(3) == "MOE_ERR_WORKSPACE"


def test_shared_gate_needs_shared_expert_and_alignment():
    c, r, ex, sh = _c3()
    r.shared_gate = FAKE
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_OK
    r.shared_gate = FAKE + 2
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    r.shared_gate = FAKE
    c.shared_inter = 0
    assert B.validate(c, r, ex, None, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    assert "shared expert" in B.last_error()


def _share_call(c, r, local, lo, hi, shared, n=4, ws=1 << 40, partial=FAKE + 4096,
                workspace=FAKE):
    # every argument fails validation before anything is enqueued
    return int(B.lib().moe_forward_ep_partial(
        ctypes.byref(c), ctypes.byref(r), None if local is None else ctypes.byref(local),
        lo, hi, None if shared is None else ctypes.byref(shared), ctypes.c_void_p(FAKE), n,
        ctypes.c_void_p(partial), None, ctypes.c_void_p(workspace), ws, None, None))


def test_ep_share_range_checked():
    c, r, _, sh = _c3()
    for lo, hi in ((5, 5), (9, 3), (-1, 8), (250, 257)):
        cnt = max(1, hi - lo)
        local = _fake_set("nvfp4", 7168, 2048, cnt, FAKE)
        assert _share_call(c, r, local, lo, hi, None) == B.MOE_ERR_INVALID_ARG, (lo, hi)
        assert "expert range" in B.last_error()


def test_ep_share_local_count_must_match_range():
    c, r, _, sh = _c3()
    local = _fake_set("nvfp4", 7168, 2048, 64, FAKE)
    # 64 local experts for a 32-expert range: refused at the count check; a
    # workspace of 1 byte would fail later, so the count check comes first
    assert _share_call(c, r, local, 32, 64, None, ws=1) == B.MOE_ERR_INVALID_ARG
    assert "expected [32," in B.last_error()


def test_ep_share_shared_expert_optional_but_consistent():
    c, r, _, sh = _c3()
    local = _fake_set("nvfp4", 7168, 2048, 32, FAKE)
    # with or without the shared expert, a bad output alignment is what is left
    for s in (None, sh):
        assert _share_call(c, r, local, 0, 32, s, partial=FAKE + 4) == B.MOE_ERR_INVALID_ARG
        assert "out" in B.last_error()
    c.shared_inter = 0
    assert _share_call(c, r, local, 0, 32, sh) == B.MOE_ERR_INVALID_ARG
    assert "shared_inter == 0" in B.last_error()


def test_ep_share_workspace_checked_against_the_same_size():
    c, r, _, sh = _c3()
    ws = B.workspace_bytes(c, 4)
    local = _fake_set("nvfp4", 7168, 2048, 16, FAKE)
    assert _share_call(c, r, local, 16, 32, sh, ws=ws - 1, partial=FAKE + 4) in (
        B.MOE_ERR_INVALID_ARG, B.MOE_ERR_WORKSPACE)
    assert _share_call(c, r, local, 16, 32, sh, ws=ws // 4) == B.MOE_ERR_WORKSPACE


def test_workspace_covers_a_decode_share_of_a_slot_mode_layer():
    # the one workspace size covers a share's call as well as the layer's
    cfg = dict(H=2048, I=768, E=128, k=8, I_s=0, scoring="softmax", renorm=True, rsf=1.0)
    c = B.make_cfg(cfg, accum="slot")
    r = B.MoeRouter(FAKE, None)
    ws = B.workspace_bytes(c, 4)
    local = _fake_set("mxfp4", 2048, 768, 32, FAKE)
    for n in (1, 3, 4):
        assert _share_call(c, r, local, 0, 32, None, n=n, ws=1) == B.MOE_ERR_WORKSPACE
        need = int(re.search(r"need (\d+) bytes", B.last_error()).group(1))
        assert need <= ws, n
        assert _share_call(c, r, local, 0, 32, None, n=n, ws=ws,
                           partial=FAKE + 4) == B.MOE_ERR_INVALID_ARG


def test_zero_expert_router_width():
    c, r, ex, sh = _c3()
    c.zero_experts = 1  # 256 + 1 router columns
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_UNSUPPORTED
    assert "router width" in B.last_error()
    c.num_experts = 192
    c.zero_experts = 64
    ex = _fake_set("nvfp4", 7168, 2048, 192, FAKE)
    assert B.validate(c, r, ex, sh, 4, B.workspace_bytes(c, 4)) == B.MOE_OK
    c.zero_experts = -1
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_UNSUPPORTED
    # top_k may exceed E when zero experts widen the router
    c.num_experts, c.zero_experts, c.top_k = 4, 4, 6
    ex = _fake_set("nvfp4", 7168, 2048, 4, FAKE)
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_OK
    c.top_k = 9
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG


def test_zero_experts_grow_the_grouped_router_partials():
    c, r, ex, sh = _c3()
    c.num_experts, c.top_k = 128, 8
    ex = _fake_set("nvfp4", 7168, 2048, 128, FAKE)
    # 16 tokens: one token group, so the router's K split is capped by the
    # 56 column chunks with and without the extra router rows, and the
    # partials [N, ksplit, E + Z] grow with Z
    w0 = B.workspace_bytes(c, 16)
    c.zero_experts = 64
    assert B.workspace_bytes(c, 16) > w0


def test_hash_routing_arguments():
    c, r, ex, sh = _c3()
    r.tid2eid = FAKE
    r.vocab = 1000
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    assert "token_ids" in B.last_error()
    r.token_ids = FAKE + 8192
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_OK
    r.vocab = 0
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    r.vocab = 1000
    r.token_ids = FAKE + 8194
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    r.tid2eid = None
    r.token_ids = FAKE + 8192
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    assert "without a hash table" in B.last_error()


def test_nvfp4_router_arguments():
    c, r, ex, sh = _c3()
    wq = _fake_weight("nvfp4", 256, 7168, 1, FAKE + (16 << 32))
    r.weight_q = ctypes.addressof(wq)
    # both a BF16 weight and a quantised one
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    assert "exactly one" in B.last_error()
    r.weight = None
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_OK
    # rows must be the router width E + Z
    c.zero_experts = 0
    wq.rows = 255
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG
    wq.rows = 256
    # only NVFP4
    mx = _fake_weight("mxfp4", 256, 7168, 1, FAKE + (16 << 32))
    r.weight_q = ctypes.addressof(mx)
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_UNSUPPORTED
    r.weight_q = None
    assert B.validate(c, r, ex, sh, 4, 1 << 40) == B.MOE_ERR_INVALID_ARG


def test_no_alloc_refuses_calls_beyond_the_static_scratch():
    # the allocation-free entry point checks its need against the 16 MiB
    # static scratch before it looks the scratch up or enqueues anything, so
    # an oversized call is refused by name here, without a device
    c, r, ex, sh = _c3()
    c.path = B.PATH["grouped"]
    lib = moe.lib()
    st = lib.moe_forward_no_alloc(ctypes.byref(c), ctypes.byref(r), ctypes.byref(ex),
                                  ctypes.byref(sh), FAKE, 512, FAKE, None, None, None)
    assert st == B.MOE_ERR_WORKSPACE
    msg = B.last_error()
    m = re.search(r"static scratch holds (\d+) bytes and this call needs (\d+)", msg)
    assert m and int(m.group(1)) == 16 << 20 and int(m.group(2)) > 16 << 20, msg
    # invalid arguments are refused the same way as by moe_forward
    st = lib.moe_forward_no_alloc(ctypes.byref(c), ctypes.byref(r), ctypes.byref(ex),
                                  ctypes.byref(sh), FAKE, 0, FAKE, None, None, None)
    assert st == B.MOE_ERR_INVALID_ARG and "n_tokens=0" in B.last_error()


def test_profile_driver_refuses_bad_arguments():
    """The stand-alone profiling driver (built next to the library) checks
    its arguments on the host before it touches a GPU."""
    import subprocess
    drv = os.path.join(os.path.dirname(B.LIB_PATH), "moe_profile_driver")
    if not os.path.exists(drv):
        pytest.skip("profiling driver not built (run __graft_entry__.build())")
    for args in ([], ["layer", "no_such_workload", "1", "1"], ["layer", "tiny_bf16", "0", "1"],
                 ["layer", "tiny_bf16", "3", "1", "fp16"], ["copy", "0", "1"], ["read", "16", "1000"]):
        r = subprocess.run([drv] + args, capture_output=True, text=True, timeout=60)
        assert r.returncode == 2, (args, r.returncode, r.stderr)
        assert "usage" in r.stderr or "unknown workload" in r.stderr, (args, r.stderr)
