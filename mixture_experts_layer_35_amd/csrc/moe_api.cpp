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
#include <cstddef>
#include <mutex>

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
  if (c->zero_experts < 0 || c->num_experts + c->zero_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "router width E + Z = %d + %d outside 1..%d",
                c->num_experts, c->zero_experts, MOE_MAX_EXPERTS);
  if (c->top_k < 1 || c->top_k > c->num_experts + c->zero_experts || c->top_k > MOE_MAX_TOPK)
    return fail(MOE_ERR_INVALID_ARG, "top_k=%d must be in 1..min(E+Z=%d, %d)", c->top_k,
                c->num_experts + c->zero_experts, MOE_MAX_TOPK);
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

// Shape limits of each path (named refusals; no silent fallback).
moe_status check_path_shape(const moe_cfg* c, int path) {
  if (path == MOE_PATH_DECODE) {
    // x (and a) rows of every token of a unit are staged in LDS
    const int maxc = c->hidden > c->inter ? c->hidden : c->inter;
    const int maxc2 = maxc > c->shared_inter ? maxc : c->shared_inter;
    if ((size_t)moe::kNmax * maxc2 * 2 > 65536)
      return fail(MOE_ERR_UNSUPPORTED, "decode path stages %d x %d BF16 in LDS; max width 8192",
                  moe::kNmax, maxc2);
  } else {
    // the expert GEMMs step K in 128-column chunks
    if (c->hidden % moe::kGKC || c->inter % moe::kGKC || c->shared_inter % moe::kGKC)
      return fail(MOE_ERR_UNSUPPORTED,
                  "grouped path needs H, I and I_shared to be multiples of %d (H=%d I=%d I_s=%d)",
                  moe::kGKC, c->hidden, c->inter, c->shared_inter);
  }
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
  moe_status st = check_path_shape(c, p);
  if (st) return st;
  *path = p;
  return MOE_OK;
}

// Launch plan of the grouped path for n tokens.
struct GPlan {
  int nt, W, maxu, max_items, ksplit, kcps, r_rb, r_tg, s_tg, gu_s, gu_r, dn_s, dn_r;
  size_t mcap;  // rows of the permuted buffers
};

// 16-token tiles per pass of the expert kernels for a call of n tokens.
// Up to 64 tokens: one (a unit with more rows than that is split into several
// work items, one workgroup each, so the kernel keeps the registers of one
// tile and four workgroups per compute unit), except FP8 experts above 48
// tokens, which take the rule for larger batches (two tiles at these sizes):
// same-session timings of the grouped FP8 layer (H = 4096, E = 128, k = 8,
// FP8 shared expert) read 3.5% faster with two at 56 and 64 tokens and 1-3%
// slower at 40 and 48, while the DeepSeek-V3-shaped NVFP4 layer read 17%
// slower with two at 48 tokens. Above 64 tokens the kernels' registers
// grow with the tile count (one workgroup per compute unit with eight tiles,
// two with four, three with two), and FP8 and FP4 weights put fewer bytes in
// flight per load than BF16, so they need the occupancy of fewer tiles. The
// rule, from same-session timings of 1, 2, 4 and 8 tiles at 128 to 1024
// tokens: BF16 experts take two tiles while the batch averages at most 8 rows
// per expert and eight above; FP8 and FP4 experts take two while it averages
// at most 16 rows per expert (with a shared expert, whose passes cover every
// token: up to 128 tokens) and four above. Then more, if the work items would
// not fit their list.
int grouped_tiles(const moe_cfg* c, int n, int routed_fmt, bool has_shared) {
  if (n <= (routed_fmt == MOE_FMT_FP8_ROWSCALE ? 48 : 64)) return 1;
  const int64_t slots = (int64_t)n * c->top_k;
  const int64_t per_expert = slots / c->num_experts;  // average rows per expert
  int nt;
  if (routed_fmt == MOE_FMT_BF16)
    nt = per_expert <= 8 ? 2 : 8;
  else
    nt = (has_shared ? n <= 128 : per_expert <= 16) ? 2 : 4;
  const int64_t maxu = slots < c->num_experts ? slots : c->num_experts;
  while (nt < 8 && maxu + (slots + 16 * nt - 1) / (16 * nt) > moe::kMaxItems) nt <<= 1;
  return nt;
}

// nt: the call's tiles per pass (grouped_tiles), or 0 for the workspace
// layout, which takes the largest choice (one up to 48 tokens, eight above):
// the router partials' buffer only grows with the tile count, and nothing
// else in the layout depends on it.
GPlan gplan(const moe_cfg* c, int n, bool gated, int nt = 0) {
  GPlan g;
  // router rows: E experts and Z zero experts in blocks of 128, plus a block
  // of its own for the shared gate's row
  const int EW = c->num_experts + c->zero_experts;
  g.nt = nt > 0 ? nt : (n <= 48 ? 1 : 8);
  const int T = 16 * g.nt;
  g.W = (n + 31) / 32;
  const int64_t slots = (int64_t)n * c->top_k;
  g.maxu = (int)(slots < c->num_experts ? slots : c->num_experts);
  g.max_items = g.maxu + (int)((slots + T - 1) / T);
  const int chunks = c->hidden / moe::kGKC;
  g.r_rb = (EW + moe::kGRowsPerWG - 1) / moe::kGRowsPerWG + (gated ? 1 : 0);
  g.r_tg = (n + T - 1) / T;
  // split H so that the router has about 256 workgroups
  int want = (256 + g.r_rb * g.r_tg - 1) / (g.r_rb * g.r_tg);
  want = want < 1 ? 1 : (want > chunks ? chunks : want);
  g.kcps = (chunks + want - 1) / want;
  g.ksplit = (chunks + g.kcps - 1) / g.kcps;
  g.s_tg = (n + T - 1) / T;
  g.gu_r = c->inter / 64;
  g.dn_r = c->hidden / moe::g_down_rows(g.nt);
  g.gu_s = c->shared_inter > 0 ? (c->shared_inter / 64) * g.s_tg : 0;
  g.dn_s = c->shared_inter > 0 ? g.dn_r * g.s_tg : 0;
  g.mcap = align_up((size_t)slots + (size_t)15 * g.maxu, 16);
  return g;
}

// Workspace layout, three regions in this order:
//   head     decode-path counters and the decode FP32 accumulator; fixed size
//            for a given cfg, zero at rest (every decode call leaves it zero;
//            the grouped path only ever sets bits of the error word in it)
//   decode   the decode path's tagged hand-off words (activations, slot-mode
//            down rows), always sized for kNmax tokens in slot mode, so that
//            its offsets do not depend on N or on the accumulation mode
//   grouped  the grouped path's per-call buffers (their size depends on N)
// The decode region holds nothing but tagged words of decode calls: a
// grouped call never writes there, so no word of it can carry a value a
// later decode call would take for its own tag (a grouped buffer holds small
// integers such as expert ids and counts, and tags are small integers too).
// The grouped path writes every buffer it reads within the same call.
struct Layout {
  size_t head_bytes = 0;
  size_t total = 0;
  // decode
  size_t blend_ctr = 0, acc = 0;
  size_t a_routed = 0, a_shared = 0, dbuf = 0;
  // grouped
  size_t g_zpart = 0, g_gamma = 0, g_ticket = 0, g_mask = 0, g_idx = 0, g_wts = 0, g_info = 0, g_ptok = 0, g_pslot = 0,
         g_inv = 0, g_aperm = 0, g_ashared = 0, g_dperm = 0, g_dshared = 0, g_acc = 0;
};

// Largest decode-path widths (the decode path stages kNmax rows of each in
// 64 KiB of LDS) and top-k: the universal layout sizes its head and decode
// region for them.
// the grouping workgroup of the largest call the library takes fits the 160 KB
// of LDS a workgroup may hold
static_assert(moe::group_lds_layout(MOE_MAX_EXPERTS, (MOE_MAX_TOKENS + 31) / 32).bytes <=
                  160 * 1024,
              "grouping LDS");

constexpr size_t kDecodeMaxWidth = 8192;
constexpr size_t kUniversalTopk = MOE_MAX_TOPK;

// universal: the layout of the allocation-free entry point's static scratch,
// which every layer on a device shares. Its head and decode region are sized
// for the largest decode call of any cfg, so that their offsets do not depend
// on the cfg either: the zero-at-rest head of one layer never lies where
// another layer's tagged words are, and no layer's grouped buffers lie where
// any layer's decode words are.
Layout layout(const moe_cfg* c, int32_t n, int path, bool gated, bool universal = false) {
  Layout L;
  const size_t N = n, k = c->top_k, H = c->hidden, I = c->inter, Is = c->shared_inter,
               E = c->num_experts, Nd = moe::kNmax;
  const bool atomic = c->accum_mode == MOE_ACCUM_ATOMIC_F32;
  const size_t Hh = universal ? kDecodeMaxWidth : H;  // head and decode region sizes
  const size_t Ih = universal ? kDecodeMaxWidth : I;
  const size_t Ish = universal ? kDecodeMaxWidth : Is;
  const size_t kh = universal ? kUniversalTopk : k;
  size_t off = sizeof(moe::Ctl);
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.blend_ctr = take((Hh + 3) / 4 * moe::kLineWords * 4);
  // the decode accumulator is part of the head in both modes, so that calls
  // of either mode can share a workspace (it is zero at rest)
  L.acc = take(Nd * Hh * 4);
  L.head_bytes = off;
  // decode region: tagged BF16 pairs (one 8-byte word per two activations)
  // and tagged FP32 slot-mode down rows, sized for the largest decode call
  L.a_routed = take(Nd * kh * Ih / 2 * 8);
  L.a_shared = take(Nd * (Ish ? Ish : 2) / 2 * 8);
  L.dbuf = take((Nd * kh + Nd) * Hh * 8);
  if (path == MOE_PATH_GROUPED) {
    const GPlan g = gplan(c, n, gated);
    L.g_mask = take((E * (g.W | 1) + 1) * 4);  // rows of W | 1 words, one word more
    L.g_ticket = take(4);
    L.g_idx = take(N * k * 4);
    L.g_wts = take(N * k * 4);
    L.g_info = take(sizeof(moe::GroupInfo));
    L.g_ptok = take(g.mcap * 4);
    L.g_pslot = take(g.mcap * 4);
    L.g_inv = take(N * k * 4);
    L.g_aperm = take(g.mcap * I * 2);
    if (Is) L.g_ashared = take(N * Is * 2);
    if (atomic) {
      L.g_acc = take(N * H * 4);
    } else {
      L.g_dperm = take(g.mcap * H * 4);
      if (Is) L.g_dshared = take(N * H * 4);
    }
    L.g_zpart = take((size_t)g.ksplit * N * (E + c->zero_experts + (gated ? 1 : 0)) * 4);
    L.g_gamma = take(N * 4);
  }
  L.total = off;
  return L;
}

// Bytes a call with n tokens needs (0 if such a call is refused).
size_t need_bytes(const moe_cfg* c, int32_t n) {
  int path;
  if (resolve_path(c, n, &path)) return 0;
  // a call may bring a shared-expert gate: size for the larger layout (of
  // either accumulation mode, so that one workspace serves both)
  size_t most = 0;
  for (int acc = MOE_ACCUM_SLOT; acc <= MOE_ACCUM_ATOMIC_F32; ++acc) {
    moe_cfg cc = *c;
    cc.accum_mode = acc;
    for (int gated = 0; gated <= (c->shared_inter > 0 ? 1 : 0); ++gated) {
      const size_t b = layout(&cc, n, path, gated != 0).total;
      most = b > most ? b : most;
    }
  }
  return most;
}

// What a call computes: the whole layer (experts 0..E-1, BF16 output, the
// shared expert included) or one expert-parallel share (experts lo..hi-1,
// whose weights are the only ones given, an FP32 partial output, and the
// shared expert only if this share carries it).
struct Share {
  int lo = 0, hi = 0;
  bool partial = false;
};

// Gate+up geometry: a workgroup stages x once (tokens * H BF16 into LDS) and
// then streams `sub` row blocks, enough that the staged bytes stay under a
// quarter of the weight bytes, while keeping about two workgroups per compute
// unit, and at most max_tiles workgroups per unit.
moe::StageGeom gate_up_geom(int fmt, int H, int rows, int rpl, int tokens, int units,
                            int max_tiles) {
  int64_t db, sb;
  expected_bytes(fmt, 1, H, &db, &sb);
  const int64_t row_bytes = db + sb;
  const moe::StageGeom one = moe::stage_geom(fmt, H, rows, rpl, 1);
  const int64_t block_bytes = (int64_t)one.rows_per_wg * 2 * row_bytes;
  const int64_t staged = (int64_t)tokens * H * 2;
  int sub = (int)((4 * staged + block_bytes - 1) / block_bytes);
  sub = sub < 1 ? 1 : (sub > 8 ? 8 : sub);
  while (sub < 16 &&
         (rows + one.rows_per_wg * sub - 1) / (one.rows_per_wg * sub) > max_tiles)
    ++sub;
  while (sub > 1 &&
         (int64_t)units * ((rows + one.rows_per_wg * sub - 1) / (one.rows_per_wg * sub)) < 512 &&
         (rows + one.rows_per_wg * (sub - 1) - 1) / (one.rows_per_wg * (sub - 1)) <= max_tiles)
    --sub;
  return moe::stage_geom(fmt, H, rows, rpl, sub);
}

// Down geometry: a workgroup stages its unit's activations once (tagged BF16
// pairs, 4 bytes per value and token) and streams `sub` row blocks, enough
// that the staged bytes stay under an eighth of the weight bytes, while the
// grid keeps at least min_wgs workgroups. sub stays a power of two, so that row
// tiles of the routed and the shared expert nest in the blend blocks.
moe::StageGeom down_geom(int fmt, int I, int H, int rpl, int tokens, int units, int min_wgs) {
  int64_t db, sb;
  expected_bytes(fmt, 1, I, &db, &sb);
  const moe::StageGeom one = moe::stage_geom(fmt, I, H, rpl, 1);
  const int64_t block_bytes = (int64_t)one.rows_per_wg * (db + sb);
  const int64_t staged = (int64_t)tokens * I * 4;
  int sub = 1;
  while (sub < 16 && sub * block_bytes < 8 * staged) sub <<= 1;
  auto tiles = [&](int s) { return (H + one.rows_per_wg * s - 1) / (one.rows_per_wg * s); };
  while (sub > 1 && (int64_t)units * tiles(sub) < min_wgs) sub >>= 1;
  return moe::stage_geom(fmt, I, H, rpl, sub);
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

moe_status forward_grouped(const moe_cfg* cfg, const moe_router* router,
                           const moe_experts* experts, const moe_experts* shared, const void* x,
                           int32_t n, void* out, const moe_topk_out* topk, void* workspace,
                           hipStream_t hs, hipEvent_t* ev, const Share& sh, bool universal) {
  moe::GroupedArgs a{};
  a.N = n;
  a.H = cfg->hidden;
  a.I = cfg->inter;
  a.E = cfg->num_experts;
  a.k = cfg->top_k;
  a.I_s = shared ? cfg->shared_inter : 0;
  a.e_lo = sh.lo;
  a.EL = sh.hi - sh.lo;
  a.scoring = cfg->scoring;
  a.renorm = cfg->norm_topk_prob;
  a.atomic = cfg->accum_mode == MOE_ACCUM_ATOMIC_F32;
  a.rsf = cfg->routed_scaling_factor;
  a.x = static_cast<const uint16_t*>(x);
  if (sh.partial)
    a.out_f32 = static_cast<float*>(out);
  else
    a.out = static_cast<uint16_t*>(out);
  a.router_w = static_cast<const uint16_t*>(router->weight);
  a.router_fmt = router->weight_q ? moe::FMT_NVFP4_HOST : moe::FMT_BF16_HOST;
  if (router->weight_q) a.router_q = to_dev(*router->weight_q);
  a.router_bias = router->bias;
  // the gate weights the shared expert's output: without it in this call,
  // its router row is not needed
  a.shared_gate = a.I_s > 0 ? static_cast<const uint16_t*>(router->shared_gate) : nullptr;
  const bool gated = a.shared_gate != nullptr;
  a.EW = a.E + cfg->zero_experts;
  a.ER = a.EW + (gated ? 1 : 0);
  a.tid2eid = router->tid2eid;
  a.token_ids = router->token_ids;
  a.vocab = router->vocab;
  a.err = &reinterpret_cast<moe::Ctl*>(workspace)->error;
  a.gate = to_dev(experts->gate);
  a.up = to_dev(experts->up);
  a.down = to_dev(experts->down);
  const int fr = experts->gate.format;
  int fs = moe::FMT_NONE_HOST;
  if (a.I_s > 0) {
    a.sgate = to_dev(shared->gate);
    a.sup = to_dev(shared->up);
    a.sdown = to_dev(shared->down);
    fs = shared->gate.format;
  }
  const GPlan g = gplan(cfg, n, gated, grouped_tiles(cfg, n, fr, a.I_s > 0));
  a.nt = g.nt;
  a.W = g.W;
  a.WP = g.W | 1;
  a.maxu = g.maxu < a.EL ? g.maxu : a.EL;
  a.max_items = a.maxu + (g.max_items - g.maxu);
  if (a.max_items > moe::kMaxItems)
    return fail(MOE_ERR_UNSUPPORTED, "grouped path: %d work items exceed %d", a.max_items,
                moe::kMaxItems);
  a.ksplit = g.ksplit;
  a.kcps = g.kcps;
  a.r_rb = g.r_rb;
  a.r_tg = g.r_tg;
  a.s_tg = g.s_tg;
  a.gu_s = g.gu_s;
  a.gu_r = g.gu_r;
  a.dn_s = g.dn_s;
  a.dn_r = g.dn_r;
  if (a.I_s == 0) a.s_tg = a.gu_s = a.dn_s = 0;  // a share without the shared expert
  char* base = static_cast<char*>(workspace);
  const Layout L = layout(cfg, n, MOE_PATH_GROUPED, gated, universal);
  a.zpart = reinterpret_cast<float*>(base + L.g_zpart);
  a.gamma = reinterpret_cast<float*>(base + L.g_gamma);
  a.mask = reinterpret_cast<uint32_t*>(base + L.g_mask);
  a.ticket = reinterpret_cast<unsigned*>(base + L.g_ticket);
  a.idx = reinterpret_cast<int*>(base + L.g_idx);
  a.wts = reinterpret_cast<float*>(base + L.g_wts);
  a.info = reinterpret_cast<moe::GroupInfo*>(base + L.g_info);
  a.perm_tok = reinterpret_cast<int*>(base + L.g_ptok);
  a.perm_slot = reinterpret_cast<int*>(base + L.g_pslot);
  a.inv = reinterpret_cast<int*>(base + L.g_inv);
  a.a_perm = reinterpret_cast<uint16_t*>(base + L.g_aperm);
  a.a_shared = a.I_s ? reinterpret_cast<uint16_t*>(base + L.g_ashared) : nullptr;
  a.d_perm = a.atomic ? nullptr : reinterpret_cast<float*>(base + L.g_dperm);
  a.d_shared = (!a.atomic && a.I_s) ? reinterpret_cast<float*>(base + L.g_dshared) : nullptr;
  a.acc = a.atomic ? reinterpret_cast<float*>(base + L.g_acc) : nullptr;
  if (topk) {
    a.out_idx = topk->idx;
    a.out_w = topk->weights;
    a.out_logits = topk->logits;
  }
  hipError_t err = moe::launch_grouped(a, fr, fs, hs, ev);
  if (err != hipSuccess)
    return fail(MOE_ERR_HIP, "launch failed: %s", hipGetErrorString(err));
  return MOE_OK;
}

moe_status validate_impl(const moe_cfg* cfg, const moe_router* router,
                         const moe_experts* experts, const moe_experts* shared, int32_t n_tokens,
                         size_t workspace_bytes, const Share& sh, bool universal = false) {
  g_err[0] = 0;
  moe_status st = check_cfg(cfg);
  if (st) return st;
  int path;
  st = resolve_path(cfg, n_tokens, &path);
  if (st) return st;
  if (!router) return fail(MOE_ERR_INVALID_ARG, "null router");
  if (!router->weight == !router->weight_q)
    return fail(MOE_ERR_INVALID_ARG, "give exactly one of router weight (BF16) and weight_q");
  if (router->weight && !aligned(router->weight, 16))
    return fail(MOE_ERR_INVALID_ARG, "router weight not 16-byte aligned");
  if (router->weight_q) {
    if (router->weight_q->format != MOE_FMT_NVFP4)
      return fail(MOE_ERR_UNSUPPORTED, "a quantised router must be NVFP4, got %s",
                  fmt_name(router->weight_q->format));
    st = check_weight(*router->weight_q, "router", cfg->num_experts + cfg->zero_experts,
                      cfg->hidden, 1);
    if (st) return st;
  }
  if (router->bias && !aligned(router->bias, 4))
    return fail(MOE_ERR_INVALID_ARG, "router bias not 4-byte aligned");
  if (router->tid2eid) {
    if (!router->token_ids)
      return fail(MOE_ERR_INVALID_ARG, "hash routing needs token_ids");
    if (router->vocab <= 0)
      return fail(MOE_ERR_INVALID_ARG, "hash routing needs vocab > 0 (vocab=%d)", router->vocab);
    if (!aligned(router->tid2eid, 4) || !aligned(router->token_ids, 4))
      return fail(MOE_ERR_INVALID_ARG, "tid2eid and token_ids must be 4-byte aligned");
  } else if (router->token_ids) {
    return fail(MOE_ERR_INVALID_ARG, "token_ids given without a hash table (tid2eid)");
  }
  const bool with_shared = !sh.partial || shared != nullptr;
  if (router->shared_gate && with_shared) {
    if (cfg->shared_inter <= 0)
      return fail(MOE_ERR_INVALID_ARG, "a shared-expert gate needs a shared expert (shared_inter=0)");
    if (!aligned(router->shared_gate, 16))
      return fail(MOE_ERR_INVALID_ARG, "shared_gate not 16-byte aligned");
  }
  if (sh.lo < 0 || sh.hi > cfg->num_experts || sh.lo >= sh.hi)
    return fail(MOE_ERR_INVALID_ARG, "expert range [%d, %d) must be non-empty within [0, %d)",
                sh.lo, sh.hi, cfg->num_experts);
  if (!experts) return fail(MOE_ERR_INVALID_ARG, "null experts");
  st = check_set(experts, "experts", cfg->hidden, cfg->inter, sh.hi - sh.lo);
  if (st) return st;
  if (cfg->shared_inter > 0 && with_shared) {
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
  const size_t need =
      layout(cfg, n_tokens, path, router->shared_gate != nullptr && with_shared, universal).total;
  if (workspace_bytes < need) {
    if (universal)
      return fail(MOE_ERR_WORKSPACE,
                  "the static scratch holds %zu bytes and this call needs %zu (fewer tokens, "
                  "or moe_forward with a workspace of its own)",
                  workspace_bytes, need);
    return fail(MOE_ERR_WORKSPACE, "workspace too small: need %zu bytes, have %zu", need,
                workspace_bytes);
  }
  return MOE_OK;
}

moe_status forward_impl(const moe_cfg* cfg, const moe_router* router, const moe_experts* experts,
                        const moe_experts* shared, const void* x, int32_t n_tokens, void* out,
                        const moe_topk_out* topk, void* workspace, size_t workspace_bytes,
                        void* stream, const moe_trace* trace, const Share& sh,
                        bool universal = false) {
  moe_status st =
      validate_impl(cfg, router, experts, shared, n_tokens, workspace_bytes, sh, universal);
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
  int path;
  resolve_path(cfg, n_tokens, &path);
  const int launches = path == MOE_PATH_DECODE ? 1 : moe::kGLaunches;
  if (trace && (!trace->events || trace->count < 2 * launches))
    return fail(MOE_ERR_INVALID_ARG, "trace needs %d events (start and stop of each launch), got %d",
                2 * launches, trace ? trace->count : 0);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = trace ? reinterpret_cast<hipEvent_t*>(trace->events) : nullptr;
  if (path == MOE_PATH_GROUPED)
    return forward_grouped(cfg, router, experts, shared, x, n_tokens, out, topk, workspace, hs,
                           ev, sh, universal);

  moe::DecodeArgs a{};
  a.N = n_tokens;
  a.H = cfg->hidden;
  a.I = cfg->inter;
  a.E = cfg->num_experts;
  a.EW = a.E + cfg->zero_experts;
  a.tid2eid = router->tid2eid;
  a.token_ids = router->token_ids;
  a.vocab = router->vocab;
  a.k = cfg->top_k;
  a.I_s = shared ? cfg->shared_inter : 0;
  a.scoring = cfg->scoring;
  a.renorm = cfg->norm_topk_prob;
  a.atomic = cfg->accum_mode == MOE_ACCUM_ATOMIC_F32;
  a.rsf = cfg->routed_scaling_factor;
  a.e_lo = sh.lo;
  a.e_hi = sh.hi;
  a.slot_flags = (a.EW > a.E || sh.partial || router->tid2eid) ? 1 : 0;
  a.maxu = (a.N * a.k < sh.hi - sh.lo) ? a.N * a.k : sh.hi - sh.lo;
  a.x = static_cast<const uint16_t*>(x);
  if (sh.partial)
    a.out_f32 = static_cast<float*>(out);
  else
    a.out = static_cast<uint16_t*>(out);
  a.router_w = static_cast<const uint16_t*>(router->weight);
  a.router_fmt = router->weight_q ? moe::FMT_NVFP4_HOST : moe::FMT_BF16_HOST;
  if (router->weight_q) a.router_q = to_dev(*router->weight_q);
  a.router_bias = router->bias;
  a.shared_gate = a.I_s > 0 ? static_cast<const uint16_t*>(router->shared_gate) : nullptr;
  a.gate = to_dev(experts->gate);
  a.up = to_dev(experts->up);
  a.down = to_dev(experts->down);
  const int fr = experts->gate.format;
  int fs = moe::FMT_NONE_HOST;
  if (a.I_s > 0) {
    a.sgate = to_dev(shared->gate);
    a.sup = to_dev(shared->up);
    a.sdown = to_dev(shared->down);
    fs = shared->gate.format;
  }
  // two rows per lane group only when the routed gate+up grid still gives
  // about eight workgroups per compute unit with them (a large layer such as
  // H = 7168); smaller grids run faster as more, lighter workgroups
  const moe::StageGeom g2 = moe::stage_geom(fr, a.H, a.I, 2, 1);
  const int rpl = ((long)a.maxu * g2.tiles >= 2048) ? 2 : 1;
  // at most 64 gate+up workgroups per routed unit (32 for the large layers,
  // whose longer workgroups measured faster), 256 for the shared expert,
  // which streams from the start
  a.gr = gate_up_geom(fr, a.H, a.I, rpl, 1, a.maxu, rpl == 2 ? 32 : 64);
  // the down phase of the two-row kernels streams four rows per lane group
  const int rpl_down = rpl == 2 ? 4 : rpl;
  a.dr = down_geom(fr, a.I, a.H, rpl_down, a.N, a.maxu, 512);
  if (a.I_s > 0) {
    a.gs = gate_up_geom(fs, a.H, a.I_s, rpl, a.N, 1, 256);
    a.ds = down_geom(fs, a.I_s, a.H, rpl_down, a.N, 1, 64);
  }
  // router: up to four waves per row, enough that each lane holds about one
  // 16-byte chunk of the row (+ one row for the shared gate)
  const int rcpr = a.H / (router->weight_q ? 32 : 8);
  a.r_wpr = 1;
  while (a.r_wpr < 4 && a.r_wpr * 64 < rcpr) a.r_wpr <<= 1;
  const int rrows = a.EW + (a.shared_gate ? 1 : 0);
  const int rows_per_wg = 4 / a.r_wpr;
  a.nR = (rrows + rows_per_wg - 1) / rows_per_wg;
  a.nGs = a.I_s > 0 ? a.gs.tiles : 0;
  a.nGr = a.maxu * a.gr.tiles;
  a.nDs = a.I_s > 0 ? a.ds.tiles : 0;
  a.nDr = a.maxu * a.dr.tiles;
  a.blend_rows = a.dr.rows_per_wg;
  if (a.I_s > 0 && a.ds.rows_per_wg > a.blend_rows) a.blend_rows = a.ds.rows_per_wg;
  a.spin_limit = 1u << 22;
  // When the whole grid is resident (small calls), the down workgroups read
  // the plan together with the gate+up workgroups, and their first weight
  // requests would share the memory system with the gate+up weights that the
  // chain waits for. They hold back for about as long as those bytes take to
  // stream at about 6 TB/s (100 MHz ticks; at most 10 us). Below 0.5 us
  // there is nothing to gain and they start at once.
  {
    const double gu = (double)a.maxu * (a.gate.expert_bytes + a.gate.scale_expert_bytes +
                                        a.up.expert_bytes + a.up.scale_expert_bytes) +
                      (a.I_s > 0 ? (double)(a.sgate.expert_bytes + a.sgate.scale_expert_bytes +
                                            a.sup.expert_bytes + a.sup.scale_expert_bytes)
                                 : 0.0);
    const double ticks = gu / 6e12 * 1e8;
    a.d_defer_ticks = ticks < 50.0 ? 0u : (unsigned)(ticks < 1000.0 ? ticks : 1000.0);
  }

  char* base = static_cast<char*>(workspace);
  moe_cfg cc = *cfg;
  cc.accum_mode = a.atomic ? MOE_ACCUM_ATOMIC_F32 : MOE_ACCUM_SLOT;
  const Layout L = layout(&cc, n_tokens, MOE_PATH_DECODE, false, universal);
  a.ctl = reinterpret_cast<moe::Ctl*>(base);
  a.blend_ctr = reinterpret_cast<unsigned*>(base + L.blend_ctr);
  a.acc = a.atomic ? reinterpret_cast<float*>(base + L.acc) : nullptr;
  a.a_routed = reinterpret_cast<unsigned long long*>(base + L.a_routed);
  a.a_shared = reinterpret_cast<unsigned long long*>(base + L.a_shared);
  a.dbuf = a.atomic ? nullptr : reinterpret_cast<unsigned long long*>(base + L.dbuf);
  if (topk) {
    a.out_idx = topk->idx;
    a.out_w = topk->weights;
    a.out_logits = topk->logits;
  }
  const size_t lds = moe::decode_lds_bytes(a.H, a.I, a.I_s);
  hipError_t err = moe::launch_decode(a, fr, fs, rpl, lds, hs, ev ? ev[0] : nullptr,
                                      ev ? ev[1] : nullptr);
  if (err != hipSuccess)
    return fail(MOE_ERR_HIP, "launch failed: %s", hipGetErrorString(err));
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point (moe_forward_no_alloc): a device
// global, so the library never allocates it at call time. Each device that
// runs the library holds one copy, from module load until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];      // device address of `scratch` per device
bool g_scratch_cleared[kMaxDevices];   // the first-use clear was enqueued

// Zero n16 16-byte units from p (grid-stride).
__global__ void k_zero16(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's scratch address (looked up on the device's first
// call). On that first call, unless the stream is being captured into a
// graph, a fill kernel on the caller's stream also zeroes the head and the
// decode region ahead of the call's own kernels: the head must start at zero
// (its counters, error word and accumulator) and a decode word must not carry
// a tag by chance. The code object loader zero-fills the array already; the
// clear makes that explicit. It is not enqueued under capture, where a graph
// replay would clear the call counter again and let words of an earlier
// replay pass for the current call's.
moe_status static_scratch(const moe_cfg* cfg, hipStream_t hs, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  if (!g_scratch_cleared[dev]) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(hs, &cs);
    if (e != hipSuccess)
      return fail(MOE_ERR_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
    if (cs == hipStreamCaptureStatusNone) {
      // the head and the decode region of the universal layout (both of
      // fixed size); the grouped buffers need no clearing
      const size_t bytes = layout(cfg, 1, MOE_PATH_DECODE, false, true).total;
      const size_t n16 = (bytes + 15) / 16;
      hipLaunchKernelGGL(k_zero16, dim3(256), dim3(256), 0, hs,
                         static_cast<uint4*>(g_scratch_ptr[dev]), n16);
      e = hipGetLastError();
      if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "clearing the static scratch: %s", hipGetErrorString(e));
    }
    g_scratch_cleared[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
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
  // the most any call with 1..max_tokens tokens needs (the router's K split
  // makes the grouped size not quite monotone in N)
  size_t most = 0;
  for (int32_t n = 1; n <= max_tokens; ++n) {
    const size_t b = need_bytes(cfg, n);
    most = b > most ? b : most;
  }
  g_err[0] = 0;
  return most;
}

moe_status moe_group_layout(const moe_cfg* cfg, int32_t n_tokens, moe_group_view* view) {
  g_err[0] = 0;
  moe_status st = check_cfg(cfg);
  if (st) return st;
  if (!view) return fail(MOE_ERR_INVALID_ARG, "null view");
  int path;
  st = resolve_path(cfg, n_tokens, &path);
  if (st) return st;
  if (path != MOE_PATH_GROUPED)
    return fail(MOE_ERR_UNSUPPORTED, "a call with n_tokens=%d takes the decode path", n_tokens);
  const Layout L = layout(cfg, n_tokens, path, false);
  view->info = L.g_info;
  view->perm_tok = L.g_ptok;
  view->perm_slot = L.g_pslot;
  view->inv = L.g_inv;
  view->rows = (int32_t)gplan(cfg, n_tokens, false).mcap;
  return MOE_OK;
}

int32_t moe_num_launches(const moe_cfg* cfg, int32_t n_tokens) {
  if (check_cfg(cfg)) return -1;
  int path;
  if (resolve_path(cfg, n_tokens, &path)) return -1;
  return path == MOE_PATH_DECODE ? 1 : moe::kGLaunches;
}

moe_status moe_validate(const moe_cfg* cfg, const moe_router* router, const moe_experts* experts,
                        const moe_experts* shared, int32_t n_tokens, size_t workspace_bytes) {
  Share sh;
  sh.hi = cfg ? cfg->num_experts : 0;
  return validate_impl(cfg, router, experts, shared, n_tokens, workspace_bytes, sh);
}

moe_status moe_forward(const moe_cfg* cfg, const moe_router* router, const moe_experts* experts,
                       const moe_experts* shared, const void* x, int32_t n_tokens, void* out,
                       const moe_topk_out* topk, void* workspace, size_t workspace_bytes,
                       void* stream, const moe_trace* trace) {
  Share sh;
  sh.hi = cfg ? cfg->num_experts : 0;
  return forward_impl(cfg, router, experts, shared, x, n_tokens, out, topk, workspace,
                      workspace_bytes, stream, trace, sh);
}

moe_status moe_forward_no_alloc(const moe_cfg* cfg, const moe_router* router,
                                const moe_experts* experts, const moe_experts* shared,
                                const void* x, int32_t n_tokens, void* out,
                                const moe_topk_out* topk, void* stream,
                                const moe_trace* trace) {
  Share sh;
  sh.hi = cfg ? cfg->num_experts : 0;
  g_err[0] = 0;
  // refuse what does not fit before touching the device
  moe_status st = validate_impl(cfg, router, experts, shared, n_tokens, kStaticScratchBytes, sh,
                                true);
  if (st) return st;
  void* ws = nullptr;
  st = static_scratch(cfg, static_cast<hipStream_t>(stream), &ws);
  if (st) return st;
  return forward_impl(cfg, router, experts, shared, x, n_tokens, out, topk, ws,
                      kStaticScratchBytes, stream, trace, sh, true);
}

moe_status moe_forward_ep_partial(const moe_cfg* cfg, const moe_router* router,
                                  const moe_experts* local_experts, int32_t expert_begin,
                                  int32_t expert_end, const moe_experts* shared, const void* x,
                                  int32_t n_tokens, float* partial, const moe_topk_out* topk,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  const moe_trace* trace) {
  Share sh;
  sh.lo = expert_begin;
  sh.hi = expert_end;
  sh.partial = true;
  return forward_impl(cfg, router, local_experts, shared, x, n_tokens, partial, topk, workspace,
                      workspace_bytes, stream, trace, sh);
}

}  // extern "C"
