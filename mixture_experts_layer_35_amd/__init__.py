"""Routed mixture-of-experts layer forward for small token batches on
AMD Instinct MI355X (gfx950): HIP kernels behind a C ABI
(include/moe_mi355x.h) with a thin ctypes binding."""

from .binding import (Layer, MoeError, abi_version, last_error, lib, make_cfg,  # noqa: F401
                      make_experts, make_router, num_launches, status_str, validate,
                      workspace_bytes)
