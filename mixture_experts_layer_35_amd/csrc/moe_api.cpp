// Host entry points of the C ABI: argument validation, workspace planning and
// dispatch. Validation follows the reference pages' habit of refusing by name
// instead of falling back silently ("forward_k3.rs", MoeLayer::forward_k3,
// zero-expert guard; "forward_atomic_c4.rs", the scratch size check with its
// need/have message; "forward_k3.rs", the E8M0 guard, whose GS16 kernel would
// over-read a GS32 scale buffer: here every weight and scale buffer's byte
// count is checked against its format before anything is enqueued).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>

#include "../../include/moe_mi355x.h"
#include "moe_internal.h"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int values_per_chunk(int fmt) {
  switch (fmt) {
    case MOE_FMT_BF16: return 8;
    case MOE_FMT_FP8_ROWSCALE: return 16;
    case MOE_FMT_MXFP4:
    case MOE_FMT_NVFP4: return 32;
    default: return 0;
  }
}

// Expected data / scale bytes per expert for a (format, rows, cols) matrix.
void expected_bytes(int fmt, int64_t rows, int64_t cols, int64_t* data, int64_t* scales) {
  switch (fmt) {
    case MOE_FMT_BF16: *data = rows * cols * 2; *scales = 0; break;
    case MOE_FMT_FP8_ROWSCALE: *data = rows * cols; *scales = rows * 4; break;
    case MOE_FMT_MXFP4: *data = rows * cols / 2; *scales = rows * cols / 32; break;
    case MOE_FMT_NVFP4: *data = rows * cols / 2; *scales = rows * cols / 16; break;
    default: *data = *scales = -1; break;
  }
}

const char* fmt_name(int fmt) {
  switch (fmt) {
    case MOE_FMT_BF16: return "BF16";
    case MOE_FMT_FP8_ROWSCALE: return "FP8_ROWSCALE";
    case MOE_FMT_MXFP4: return "MXFP4";
    case MOE_FMT_NVFP4: return "NVFP4";
    default: return "?";
  }
}

moe_status check_weight(const moe_weight& w, const char* name, int rows, int cols, int count) {
  if (w.format < MOE_FMT_BF16 || w.format > MOE_FMT_NVFP4)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown format %d", name, w.format);
  if (w.rows != rows || w.cols != cols || w.count != count)
    return fail(MOE_ERR_INVALID_ARG, "%s: shape [%d,%d,%d], expected [%d,%d,%d]", name, w.count,
                w.rows, w.cols, count, rows, cols);
  const int vpc = values_per_chunk(w.format);
  if (cols % vpc != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: %s needs cols %% %d == 0 (cols=%d)", name,
                fmt_name(w.format), vpc, cols);
  if (!w.data) return fail(MOE_ERR_INVALID_ARG, "%s: null data", name);
  if (!aligned(w.data, 16)) return fail(MOE_ERR_INVALID_ARG, "%s: data not 16-byte aligned", name);
  int64_t db, sb;
  expected_bytes(w.format, rows, cols, &db, &sb);
  db *= count;
  sb *= count;
  if ((int64_t)w.data_bytes != db)
    return fail(MOE_ERR_INVALID_ARG, "%s: %s data is %zu bytes, expected %lld", name,
                fmt_name(w.format), w.data_bytes, (long long)db);
  if (sb == 0) {
    if (w.scales || w.scale_bytes)
      return fail(MOE_ERR_INVALID_ARG, "%s: BF16 weights take no scales", name);
  } else {
    if (!w.scales) return fail(MOE_ERR_INVALID_ARG, "%s: null scales", name);
    if ((int64_t)w.scale_bytes != sb)
      return fail(MOE_ERR_INVALID_ARG, "%s: %s scales are %zu bytes, expected %lld", name,
                  fmt_name(w.format), w.scale_bytes, (long long)sb);
    const size_t sa = w.format == MOE_FMT_FP8_ROWSCALE ? 4 : (w.format == MOE_FMT_NVFP4 ? 2 : 1);
    if (!aligned(w.scales, sa))
      return fail(MOE_ERR_INVALID_ARG, "%s: scales not %zu-byte aligned", name, sa);
  }
  if (w.format == MOE_FMT_NVFP4) {
    if (!w.tensor_scale) return fail(MOE_ERR_INVALID_ARG, "%s: NVFP4 needs tensor_scale", name);
    if (!aligned(w.tensor_scale, 4))
      return fail(MOE_ERR_INVALID_ARG, "%s: tensor_scale not 4-byte aligned", name);
  } else if (w.tensor_scale) {
    return fail(MOE_ERR_INVALID_ARG, "%s: tensor_scale is only for NVFP4", name);
  }
  return MOE_OK;
}

moe_status check_set(const moe_experts* s, const char* name, int H, int inter, int count) {
  char buf[64];
  snprintf(buf, sizeof buf, "%s.gate", name);
  moe_status st = check_weight(s->gate, buf, inter, H, count);
  if (st) return st;
  snprintf(buf, sizeof buf, "%s.up", name);
  st = check_weight(s->up, buf, inter, H, count);
  if (st) return st;
  snprintf(buf, sizeof buf, "%s.down", name);
  st = check_weight(s->down, buf, H, inter, count);
  if (st) return st;
  if (s->up.format != s->gate.format || s->down.format != s->gate.format)
    return fail(MOE_ERR_UNSUPPORTED, "%s: gate/up/down must share one format", name);
  return MOE_OK;
}

moe_status check_cfg(const moe_cfg* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "null cfg");
  if (c->hidden <= 0 || c->inter <= 0 || c->shared_inter < 0)
    return fail(MOE_ERR_INVALID_ARG, "sizes must be positive (H=%d I=%d I_s=%d)", c->hidden,
                c->inter, c->shared_inter);
  if (c->num_experts < 1 || c->num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "num_experts=%d outside 1..%d", c->num_experts,
                MOE_MAX_EXPERTS);
  if (c->top_k < 1 || c->top_k > c->num_experts || c->top_k > MOE_MAX_TOPK)
    return fail(MOE_ERR_INVALID_ARG, "top_k=%d must be in 1..min(E=%d, %d)", c->top_k,
                c->num_experts, MOE_MAX_TOPK);
  if (c->scoring != MOE_SCORE_SOFTMAX && c->scoring != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "unknown scoring %d", c->scoring);
  if (c->norm_topk_prob != 0 && c->norm_topk_prob != 1)
    return fail(MOE_ERR_INVALID_ARG, "norm_topk_prob must be 0 or 1");
  if (!std::isfinite(c->routed_scaling_factor) || c->routed_scaling_factor <= 0.f)
    return fail(MOE_ERR_INVALID_ARG, "routed_scaling_factor must be finite and > 0");
  if (c->accum_mode != MOE_ACCUM_SLOT && c->accum_mode != MOE_ACCUM_ATOMIC_F32)
    return fail(MOE_ERR_INVALID_ARG, "unknown accum_mode %d", c->accum_mode);
  if (c->path < MOE_PATH_AUTO || c->path > MOE_PATH_GROUPED)
    return fail(MOE_ERR_INVALID_ARG, "unknown path %d", c->path);
  if (c->hidden % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "hidden %% 8 != 0 (H=%d)", c->hidden);
  return MOE_OK;
}

moe_status resolve_path(const moe_cfg* c, int32_t n, int* path) {
  if (n < 1 || n > MOE_MAX_TOKENS)
    return fail(MOE_ERR_INVALID_ARG, "n_tokens=%d outside 1..%d", n, MOE_MAX_TOKENS);
  int p = c->path;
  if (p == MOE_PATH_AUTO) p = (n <= MOE_MAX_DECODE_TOKENS) ? MOE_PATH_DECODE : MOE_PATH_GROUPED;
  if (p == MOE_PATH_DECODE && n > MOE_MAX_DECODE_TOKENS)
    return fail(MOE_ERR_UNSUPPORTED, "decode path takes at most %d tokens (n=%d)",
                MOE_MAX_DECODE_TOKENS, n);
  if (p == MOE_PATH_GROUPED)
    return fail(MOE_ERR_UNSUPPORTED, "grouped path is not built yet (n=%d)", n);
  // x (and a) rows of every token of a unit are staged in LDS
  const int maxc = c->hidden > c->inter ? c->hidden : c->inter;
  const int maxc2 = maxc > c->shared_inter ? maxc : c->shared_inter;
  if ((size_t)moe::kNmax * maxc2 * 2 > 65536)
    return fail(MOE_ERR_UNSUPPORTED, "decode path stages %d x %d BF16 in LDS; max width 8192",
                moe::kNmax, maxc2);
  *path = p;
  return MOE_OK;
}

// Workspace layout for the decode path (offsets from the base, 256-aligned).
moe::Workspace layout(const moe_cfg* c, int32_t n, char* base) {
  moe::Workspace w;
  const size_t N = n, E = c->num_experts, k = c->top_k, H = c->hidden, I = c->inter,
               Is = c->shared_inter;
  const size_t maxu = (N * k < E) ? N * k : E;
  size_t off = 256;  // counters
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return base ? base + o : nullptr;
  };
  w.logits = (float*)take(N * E * 4);
  w.idx = (uint32_t*)take(N * k * 4);
  w.wts = (float*)take(N * k * 4);
  w.num_units = (int32_t*)take(16);
  w.unit_expert = (int32_t*)take(maxu * 4);
  w.unit_slot = (int32_t*)take(maxu * moe::kNmax * 4);
  w.unit_w = (float*)take(maxu * moe::kNmax * 4);
  w.a_routed = (uint16_t*)take(N * k * I * 2);
  w.a_shared = (uint16_t*)take(N * (Is ? Is : 1) * 2);
  if (c->accum_mode == MOE_ACCUM_ATOMIC_F32)
    w.acc = (float*)take(N * H * 4);
  else
    w.dbuf = (float*)take((N * k + N) * H * 4);
  w.total = off;
  return w;
}

moe::DevProj to_dev(const moe_weight& w) {
  moe::DevProj p;
  p.data = static_cast<const uint8_t*>(w.data);
  p.scales = static_cast<const uint8_t*>(w.scales);
  p.tensor_scale = w.tensor_scale;
  p.expert_bytes = (int64_t)(w.data_bytes / (size_t)w.count);
  p.scale_expert_bytes = (int64_t)(w.scale_bytes / (size_t)w.count);
  int64_t db, sb;
  expected_bytes(w.format, w.rows, w.cols, &db, &sb);
  p.row_bytes = (int32_t)(db / w.rows);
  p.scale_row_bytes = (int32_t)(sb / w.rows);
  p.rows = w.rows;
  p.cols = w.cols;
  p.fmt = w.format;
  return p;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

size_t moe_workspace_bytes(const moe_cfg* cfg, int32_t max_tokens) {
  if (check_cfg(cfg)) return 0;
  int path;
  if (resolve_path(cfg, max_tokens, &path)) return 0;
  return layout(cfg, max_tokens, nullptr).total;
}

moe_status moe_validate(const moe_cfg* cfg, const moe_router* router, const moe_experts* experts,
                        const moe_experts* shared, int32_t n_tokens, size_t workspace_bytes) {
  g_err[0] = 0;
  moe_status st = check_cfg(cfg);
  if (st) return st;
  int path;
  st = resolve_path(cfg, n_tokens, &path);
  if (st) return st;
  if (!router || !router->weight) return fail(MOE_ERR_INVALID_ARG, "null router weight");
  if (!aligned(router->weight, 16))
    return fail(MOE_ERR_INVALID_ARG, "router weight not 16-byte aligned");
  if (cfg->scoring == MOE_SCORE_SOFTMAX && router->bias)
    return fail(MOE_ERR_UNSUPPORTED, "a correction bias with softmax scoring is not supported");
  if (router->bias && !aligned(router->bias, 4))
    return fail(MOE_ERR_INVALID_ARG, "router bias not 4-byte aligned");
  if (!experts) return fail(MOE_ERR_INVALID_ARG, "null experts");
  st = check_set(experts, "experts", cfg->hidden, cfg->inter, cfg->num_experts);
  if (st) return st;
  if (cfg->shared_inter > 0) {
    if (!shared) return fail(MOE_ERR_INVALID_ARG, "shared_inter=%d but shared is null",
                             cfg->shared_inter);
    st = check_set(shared, "shared", cfg->hidden, cfg->shared_inter, 1);
    if (st) return st;
    if (shared->gate.format != MOE_FMT_BF16 && shared->gate.format != experts->gate.format)
      return fail(MOE_ERR_UNSUPPORTED,
                  "shared expert format must be BF16 or the routed format (%s), got %s",
                  fmt_name(experts->gate.format), fmt_name(shared->gate.format));
  } else if (shared) {
    return fail(MOE_ERR_INVALID_ARG, "shared is given but shared_inter == 0");
  }
  const size_t need = layout(cfg, n_tokens, nullptr).total;
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: need %zu bytes, have %zu", need,
                workspace_bytes);
  return MOE_OK;
}

int32_t moe_num_launches(const moe_cfg* cfg, int32_t n_tokens) {
  if (check_cfg(cfg)) return -1;
  int path;
  if (resolve_path(cfg, n_tokens, &path)) return -1;
  return moe::decode_num_launches();
}

moe_status moe_forward(const moe_cfg* cfg, const moe_router* router, const moe_experts* experts,
                       const moe_experts* shared, const void* x, int32_t n_tokens, void* out,
                       const moe_topk_out* topk, void* workspace, size_t workspace_bytes,
                       void* stream, const moe_trace* trace) {
  moe_status st = moe_validate(cfg, router, experts, shared, n_tokens, workspace_bytes);
  if (st) return st;
  if (!x || !aligned(x, 16)) return fail(MOE_ERR_INVALID_ARG, "x null or not 16-byte aligned");
  if (!out || !aligned(out, 16))
    return fail(MOE_ERR_INVALID_ARG, "out null or not 16-byte aligned");
  if (!workspace || !aligned(workspace, 256))
    return fail(MOE_ERR_INVALID_ARG, "workspace null or not 256-byte aligned");
  if (topk) {
    if ((topk->idx && !aligned(topk->idx, 4)) || (topk->weights && !aligned(topk->weights, 4)) ||
        (topk->logits && !aligned(topk->logits, 4)))
      return fail(MOE_ERR_INVALID_ARG, "top-k outputs must be 4-byte aligned");
  }
  const int launches = moe::decode_num_launches();
  if (trace && (!trace->events || trace->count < launches + 1))
    return fail(MOE_ERR_INVALID_ARG, "trace needs %d events", launches + 1);

  moe::Call c;
  c.N = n_tokens;
  c.H = cfg->hidden;
  c.I = cfg->inter;
  c.E = cfg->num_experts;
  c.k = cfg->top_k;
  c.I_s = cfg->shared_inter;
  c.scoring = cfg->scoring;
  c.renorm = cfg->norm_topk_prob;
  c.atomic = cfg->accum_mode == MOE_ACCUM_ATOMIC_F32;
  c.rsf = cfg->routed_scaling_factor;
  c.maxu = (c.N * c.k < c.E) ? c.N * c.k : c.E;
  c.x = static_cast<const uint16_t*>(x);
  c.out = static_cast<uint16_t*>(out);
  c.router_w = static_cast<const uint16_t*>(router->weight);
  c.router_bias = router->bias;
  c.gate = to_dev(experts->gate);
  c.up = to_dev(experts->up);
  c.down = to_dev(experts->down);
  if (c.I_s > 0) {
    c.sgate = to_dev(shared->gate);
    c.sup = to_dev(shared->up);
    c.sdown = to_dev(shared->down);
  } else {
    c.sgate.fmt = c.sup.fmt = c.sdown.fmt = moe::FMT_NONE_HOST;
  }
  c.gu_r = moe::plan_stage(c.gate.fmt, c.H, c.I, c.maxu, true);
  c.dn_r = moe::plan_stage(c.down.fmt, c.I, c.H, c.maxu, false);
  if (c.I_s > 0) {
    c.gu_s = moe::plan_stage(c.sgate.fmt, c.H, c.I_s, 1, true);
    c.dn_s = moe::plan_stage(c.sdown.fmt, c.I_s, c.H, 1, false);
  } else {
    c.gu_s.tiles = 0;
    c.dn_s.tiles = 0;
  }
  // the shared unit shares the row-per-lane choice of its kernel launch
  c.gu_s.rpl = c.gu_r.rpl;
  c.gu_s.rows_per_wg = (moe::kThreads / 64) * (64 / c.gu_s.lpr) * c.gu_s.rpl;
  if (c.I_s > 0) c.gu_s.tiles = (c.I_s + c.gu_s.rows_per_wg - 1) / c.gu_s.rows_per_wg;
  c.dn_s.rpl = c.dn_r.rpl;
  c.dn_s.rows_per_wg = (moe::kThreads / 64) * (64 / c.dn_s.lpr) * c.dn_s.rpl;
  if (c.I_s > 0) c.dn_s.tiles = (c.H + c.dn_s.rows_per_wg - 1) / c.dn_s.rows_per_wg;
  c.ws = layout(cfg, n_tokens, static_cast<char*>(workspace));
  if (topk) {
    c.out_idx = topk->idx;
    c.out_w = topk->weights;
    c.out_logits = topk->logits;
  }
  hipEvent_t* ev = trace ? reinterpret_cast<hipEvent_t*>(trace->events) : nullptr;
  hipError_t err = moe::launch_decode(c, static_cast<hipStream_t>(stream), ev);
  if (err != hipSuccess)
    return fail(MOE_ERR_HIP, "launch failed: %s", hipGetErrorString(err));
  return MOE_OK;
}

}  // extern "C"
