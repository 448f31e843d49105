// gfx950 kernels of the routed MoE layer forward, decode path (N <= 4).
//
// Five launches, in stream order:
//   1. k_router     z[N,E] = x Wr^T. One wave per router row; the row is read
//                   once for all N tokens (the batched router GEMV of
//                   "forward_k3.rs", MoeLayer::forward_k3, step 1).
//   2. k_topk_plan  one wave per token: top-k over E <= 256 scores, lowest
//                   index first on ties; softmax or sigmoid+bias weights,
//                   renorm, routed scaling factor ("forward_k3.rs" step 2).
//                   Then the batch's distinct experts ("units") are listed in
//                   ascending expert order with, per token, the slot t*k+j
//                   that routed to them, so every expert is streamed once.
//   3. k_gate_up    one workgroup per (unit, row tile): g = Wg x, u = Wu x for
//                   the unit's tokens (x staged in LDS), a = silu(g) * u.
//                   The shared expert runs as one more unit with all tokens.
//   4. k_down       one workgroup per (unit, row tile): d = Wd a for the
//                   unit's tokens (a staged in LDS); either stores w*d per slot
//                   (slot mode) or atomically adds w*d into an FP32 [N,H]
//                   accumulator ("forward_atomic_c4.rs").
//   5. k_blend / k_finalize  y = sum_j w*d + shared, cast to BF16 (RNE).
//
// Weights are read with 128-bit loads, `lpr` lanes per row, and dequantised
// in registers: FP4/FP8 pairs go to BF16 pairs with the gfx950 scaled
// converts, then into v_dot2_f32_bf16 against BF16 activations, FP32
// accumulation throughout.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int IT = 4;  // 16-byte chunks per lane per row held in flight

// ---------------------------------------------------------------------------
// Streaming core: RPL rows of NM matrices (same shape and format) against the
// staged activations of up to NT tokens. Lane group (lpr lanes) g of the wave
// owns rows row_base .. row_base+RPL-1; lane li of the group owns chunks
// li, li+lpr, ... of each row. acc[m][r][t] gets the lane's partial sums.
// ---------------------------------------------------------------------------
template <int F, int NM, int RPL, int NT>
__device__ __forceinline__ void stream_rows(const MatView (&mv)[NM], int row_base, int nrows,
                                            int cpr, int lpr, const uint32_t* xs,
                                            int xs_tok_words, uint32_t tokmask,
                                            float (&acc)[NM][RPL][NT]) {
  constexpr int XW = Fmt<F>::VPC / 2;  // 32-bit activation words per chunk
  const int li = (threadIdx.x & 63) & (lpr - 1);
  for (int c0 = 0; c0 < cpr; c0 += lpr * IT) {
    uint4 wq[IT][NM][RPL];
    uint32_t sc[IT][NM][RPL];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int c = c0 + it * lpr + li;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
          const int row = row_base + r;
          if (c < cpr && row < nrows) {
            wq[it][m][r] = ldg16(mv[m].data + (size_t)row * mv[m].row_bytes + (size_t)c * 16);
            sc[it][m][r] =
                load_chunk_scale<F>(mv[m].scales + (size_t)row * mv[m].scale_row_bytes, c);
          } else {
            wq[it][m][r] = make_uint4(0u, 0u, 0u, 0u);
            sc[it][m][r] = 0u;
          }
        }
      }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int c = c0 + it * lpr + li;
      if (c >= cpr) continue;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (!((tokmask >> t) & 1u)) continue;
        uint32_t xv[XW];
        const uint4* xp = reinterpret_cast<const uint4*>(xs + t * xs_tok_words + c * XW);
#pragma unroll
        for (int q = 0; q < XW / 4; ++q) {
          const uint4 v = xp[q];
          xv[4 * q + 0] = v.x;
          xv[4 * q + 1] = v.y;
          xv[4 * q + 2] = v.z;
          xv[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int r = 0; r < RPL; ++r) acc[m][r][t] += chunk_dot<F>(wq[it][m][r], sc[it][m][r], xv);
      }
    }
  }
}

// Copy the BF16 rows of the tokens in `mask` (row length `cols`) into LDS;
// token t lands at LDS word t * cols/2.
__device__ __forceinline__ void stage_rows(uint4* lds, const uint16_t* const* src, uint32_t mask,
                                           int cols) {
  const int per = cols / 8;  // uint4 per row
  for (int i = threadIdx.x; i < kNmax * per; i += kThreads) {
    const int t = i / per;
    const int q = i - t * per;
    if ((mask >> t) & 1u)
      lds[t * per + q] = *reinterpret_cast<const uint4*>(src[t] + (size_t)q * 8);
  }
}

__device__ __forceinline__ MatView view_of(const DevProj& p, int e) {
  MatView v;
  v.data = p.data + (size_t)e * p.expert_bytes;
  v.scales = p.scales ? p.scales + (size_t)e * p.scale_expert_bytes : nullptr;
  v.row_bytes = p.row_bytes;
  v.scale_row_bytes = p.scale_row_bytes;
  v.tensor_scale = p.tensor_scale ? p.tensor_scale[e] : 1.0f;
  return v;
}

// ---------------------------------------------------------------------------
// 1. Router projection.
// ---------------------------------------------------------------------------
struct RouterArgs {
  const uint16_t* x;
  const uint16_t* w;
  float* logits;
  int N, H, E;
};

__global__ __launch_bounds__(kThreads) void k_router(RouterArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (kThreads / 64) + wave;
  if (e >= a.E) return;
  const int t0 = blockIdx.y * kNmax;
  const int nt = min(kNmax, a.N - t0);
  const int cpr = a.H / 8;
  const uint8_t* wrow = reinterpret_cast<const uint8_t*>(a.w) + (size_t)e * a.H * 2;
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.x) + (size_t)t0 * a.H * 2;
  float acc[kNmax] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < cpr; c0 += 64 * IT) {
    uint4 wq[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int c = c0 + it * 64 + lane;
      wq[it] = c < cpr ? ldg16(wrow + (size_t)c * 16) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int c = c0 + it * 64 + lane;
      if (c >= cpr) continue;
#pragma unroll
      for (int t = 0; t < kNmax; ++t) {
        if (t >= nt) continue;
        const uint4 xq = ldg16(xb + (size_t)t * a.H * 2 + (size_t)c * 16);
        const uint32_t xv[4] = {xq.x, xq.y, xq.z, xq.w};
        acc[t] += chunk_dot<FMT_BF16>(wq[it], 0u, xv);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kNmax; ++t) {
    const float s = wave_sum(acc[t]);
    if (lane == 0 && t < nt) a.logits[(size_t)(t0 + t) * a.E + e] = s;
  }
}

// ---------------------------------------------------------------------------
// 2. Top-k routing and the expert plan (one workgroup, one wave per token).
// ---------------------------------------------------------------------------
struct TopkArgs {
  const float* logits;   // [N, E]
  const float* bias;     // [E] or null
  int N, E, k, scoring, renorm, maxu;
  float rsf;
  uint32_t* idx;         // [N, k]
  float* wts;            // [N, k]
  uint32_t* out_idx;     // optional copies
  float* out_w;
  float* out_logits;
  int32_t* num_units;
  int32_t* unit_expert;  // [maxu]
  int32_t* unit_slot;    // [maxu, kNmax]
  float* unit_w;         // [maxu, kNmax]
};

__global__ __launch_bounds__(kThreads) void k_topk_plan(TopkArgs a) {
  __shared__ int s_idx[kNmax * 16];
  __shared__ float s_w[kNmax * 16];
  __shared__ int s_present[256];
  __shared__ int s_unit_of[256];
  __shared__ int s_slot[256 * kNmax];
  __shared__ float s_uw[256 * kNmax];
  __shared__ int s_uexp[256];
  __shared__ int s_nunits;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  s_present[tid] = 0;
  for (int i = tid; i < 256 * kNmax; i += kThreads) {
    s_slot[i] = -1;
    s_uw[i] = 0.f;
  }

  for (int t = wave; t < a.N; t += kThreads / 64) {
    const float* z = a.logits + (size_t)t * a.E;
    float zv[4];
    uint32_t khi[4], klo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < a.E) {
        const float zz = z[e];
        float s = zz;
        if (a.scoring == 1) {
          s = 1.0f / (1.0f + expf(-zz));
          if (a.bias) s += a.bias[e];
        }
        zv[i] = zz;
        khi[i] = ordered_bits(s);
        klo[i] = 0xffffffffu - (uint32_t)e;
        if (a.out_logits) a.out_logits[(size_t)t * a.E + e] = zz;
      } else {
        zv[i] = -INFINITY;
        khi[i] = 0u;
        klo[i] = 0u;
      }
    }
    float zmax = 0.f, zsum = 1.f;
    if (a.scoring == 0) {
      zmax = wave_max(fmaxf(fmaxf(zv[0], zv[1]), fmaxf(zv[2], zv[3])));
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < a.E) p += expf(zv[i] - zmax);
      zsum = wave_sum(p);
    }
    int my_e = 0;
    float my_z = 0.f;
    for (int j = 0; j < a.k; ++j) {
      // lane-local best
      uint32_t bh = khi[0], bl = klo[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        if (khi[i] > bh || (khi[i] == bh && klo[i] > bl)) {
          bh = khi[i];
          bl = klo[i];
        }
      }
      // wave argmax on (score, -index)
#pragma unroll
      for (int m = 32; m > 0; m >>= 1) {
        const uint32_t oh = __shfl_xor(bh, m, 64);
        const uint32_t ol = __shfl_xor(bl, m, 64);
        if (oh > bh || (oh == bh && ol > bl)) {
          bh = oh;
          bl = ol;
        }
      }
      const int e = (int)(0xffffffffu - bl);
      const int slot = e >> 6;
      float zloc = zv[0];
#pragma unroll
      for (int i = 1; i < 4; ++i)
        if (slot == i) zloc = zv[i];
      const float zsel = __shfl(zloc, e & 63, 64);
      if (lane == (e & 63)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (slot == i) {
            khi[i] = 0u;
            klo[i] = 0u;
          }
      }
      if (lane == j) {
        my_e = e;
        my_z = zsel;
      }
    }
    float w = 0.f;
    if (lane < a.k) w = (a.scoring == 0) ? expf(my_z - zmax) / zsum : 1.0f / (1.0f + expf(-my_z));
    if (a.renorm) {
      const float tot = wave_sum(w);
      w = w / tot;
    }
    w *= a.rsf;
    if (lane < a.k) {
      const int s = t * a.k + lane;
      a.idx[s] = (uint32_t)my_e;
      a.wts[s] = w;
      if (a.out_idx) a.out_idx[s] = (uint32_t)my_e;
      if (a.out_w) a.out_w[s] = w;
      s_idx[s] = my_e;
      s_w[s] = w;
    }
  }
  __syncthreads();
  const int nslots = a.N * a.k;
  if (tid < nslots) s_present[s_idx[tid]] = 1;
  __syncthreads();
  if (wave == 0) {
    // ascending expert order: exclusive scan of the presence flags
    int cnt = 0;
    int loc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      loc[q] = cnt;
      cnt += s_present[lane * 4 + q];
    }
    int incl = cnt;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(incl, m, 64);
      if (lane >= m) incl += o;
    }
    const int base = incl - cnt;
#pragma unroll
    for (int q = 0; q < 4; ++q) s_unit_of[lane * 4 + q] = base + loc[q];
    if (lane == 63) s_nunits = incl;
  }
  __syncthreads();
  if (tid < nslots) {
    const int e = s_idx[tid];
    const int u = s_unit_of[e];
    const int t = tid / a.k;
    s_uexp[u] = e;
    s_slot[u * kNmax + t] = tid;
    s_uw[u * kNmax + t] = s_w[tid];
  }
  __syncthreads();
  const int nu = s_nunits;
  if (tid == 0) *a.num_units = nu;
  for (int i = tid; i < a.maxu * kNmax; i += kThreads) {
    a.unit_slot[i] = s_slot[i];
    a.unit_w[i] = s_uw[i];
  }
  for (int i = tid; i < a.maxu; i += kThreads) a.unit_expert[i] = (i < nu) ? s_uexp[i] : 0;
}

// ---------------------------------------------------------------------------
// 3. Expert gate + up projections and SiLU(gate) * up.
// ---------------------------------------------------------------------------
struct GateUpArgs {
  DevProj gate, up, sgate, sup;
  const uint16_t* x;
  int N, H, k, I, I_s;
  StageGeom gr, gs;
  const int32_t* num_units;
  const int32_t* unit_expert;
  const int32_t* unit_slot;
  uint16_t* a_routed;  // [N*k, I]
  uint16_t* a_shared;  // [N, I_s]
  float* zero_buf;     // atomic mode: accumulator cleared here
  int zero_count;
};

template <int F, int RPL>
__device__ __forceinline__ void gate_up_tile(const GateUpArgs& a, const DevProj& pg,
                                             const DevProj& pu, int e, int tile,
                                             const StageGeom& g, int nrows, const uint32_t* xs,
                                             uint32_t mask, const int (&slots)[kNmax],
                                             uint16_t* dst) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpr = g.lpr;
  const int groups = 64 / lpr;
  const int row_base = tile * g.rows_per_wg + (wave * groups + lane / lpr) * RPL;
  const MatView mv[2] = {view_of(pg, e), view_of(pu, e)};
  float acc[2][RPL][kNmax];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int t = 0; t < kNmax; ++t) acc[m][r][t] = 0.f;
  stream_rows<F, 2, RPL, kNmax>(mv, row_base, nrows, a.H / Fmt<F>::VPC, lpr, xs, a.H / 2, mask,
                                acc);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int t = 0; t < kNmax; ++t)
        if ((mask >> t) & 1u) acc[m][r][t] = group_sum(acc[m][r][t], lpr);
  if ((lane & (lpr - 1)) == 0) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int row = row_base + r;
      if (row >= nrows) continue;
      const float sg = row_scale<F>(mv[0], row);
      const float su = row_scale<F>(mv[1], row);
#pragma unroll
      for (int t = 0; t < kNmax; ++t) {
        if (!((mask >> t) & 1u)) continue;
        const float gv = acc[0][r][t] * sg;
        const float uv = acc[1][r][t] * su;
        dst[(size_t)slots[t] * nrows + row] = f32_to_bf16_rne(silu_f32(gv) * uv);
      }
    }
  }
}

template <int FR, int FS, int RPL>
__global__ __launch_bounds__(kThreads) void k_gate_up(GateUpArgs a) {
  extern __shared__ uint4 smem[];
  const int bid = blockIdx.x;
  if (a.zero_buf) {
    const int per = (a.zero_count + gridDim.x - 1) / gridDim.x;
    const int lo = bid * per;
    const int hi = min(a.zero_count, lo + per);
    for (int i = lo + threadIdx.x; i < hi; i += kThreads) a.zero_buf[i] = 0.f;
  }
  const bool is_shared = bid < a.gs.tiles;
  int e = 0, tile = 0;
  uint32_t mask = 0;
  int slots[kNmax];
  const uint16_t* src[kNmax];
  if (is_shared) {
    tile = bid;
#pragma unroll
    for (int t = 0; t < kNmax; ++t) {
      slots[t] = t;
      src[t] = a.x + (size_t)t * a.H;
      if (t < a.N) mask |= 1u << t;
    }
  } else {
    const int r = bid - a.gs.tiles;
    const int unit = r / a.gr.tiles;
    tile = r - unit * a.gr.tiles;
    if (unit >= *a.num_units) return;
    e = a.unit_expert[unit];
#pragma unroll
    for (int t = 0; t < kNmax; ++t) {
      const int s = a.unit_slot[unit * kNmax + t];
      slots[t] = s;
      src[t] = a.x + (size_t)t * a.H;
      if (s >= 0) mask |= 1u << t;
    }
  }
  stage_rows(smem, src, mask, a.H);
  __syncthreads();
  const uint32_t* xs = reinterpret_cast<const uint32_t*>(smem);
  if (is_shared) {
    if constexpr (FS != FMT_NONE)
      gate_up_tile<FS, RPL>(a, a.sgate, a.sup, 0, tile, a.gs, a.I_s, xs, mask, slots, a.a_shared);
  } else {
    gate_up_tile<FR, RPL>(a, a.gate, a.up, e, tile, a.gr, a.I, xs, mask, slots, a.a_routed);
  }
}

// ---------------------------------------------------------------------------
// 4. Down projections.
// ---------------------------------------------------------------------------
struct DownArgs {
  DevProj down, sdown;
  const uint16_t* a_routed;
  const uint16_t* a_shared;
  int N, H, k, I, I_s;
  StageGeom gr, gs;
  const int32_t* num_units;
  const int32_t* unit_expert;
  const int32_t* unit_slot;
  const float* unit_w;
  float* dbuf;  // slot mode: [N*k + N, H]
  float* acc;   // atomic mode: [N, H]
};

template <int F, int RPL>
__device__ __forceinline__ void down_tile(const DownArgs& a, const DevProj& pd, int e, int tile,
                                          const StageGeom& g, int cols, const uint32_t* xs,
                                          uint32_t mask, const int (&slots)[kNmax],
                                          const float (&wt)[kNmax], bool shared) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpr = g.lpr;
  const int groups = 64 / lpr;
  const int row_base = tile * g.rows_per_wg + (wave * groups + lane / lpr) * RPL;
  const MatView mv[1] = {view_of(pd, e)};
  float acc[1][RPL][kNmax];
#pragma unroll
  for (int r = 0; r < RPL; ++r)
#pragma unroll
    for (int t = 0; t < kNmax; ++t) acc[0][r][t] = 0.f;
  stream_rows<F, 1, RPL, kNmax>(mv, row_base, a.H, cols / Fmt<F>::VPC, lpr, xs, cols / 2, mask,
                                acc);
#pragma unroll
  for (int r = 0; r < RPL; ++r)
#pragma unroll
    for (int t = 0; t < kNmax; ++t)
      if ((mask >> t) & 1u) acc[0][r][t] = group_sum(acc[0][r][t], lpr);
  if ((lane & (lpr - 1)) == 0) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int row = row_base + r;
      if (row >= a.H) continue;
      const float rs = row_scale<F>(mv[0], row);
#pragma unroll
      for (int t = 0; t < kNmax; ++t) {
        if (!((mask >> t) & 1u)) continue;
        const float v = acc[0][r][t] * rs * wt[t];
        if (a.acc) {
          unsafeAtomicAdd(a.acc + (size_t)t * a.H + row, v);
        } else {
          const int s = shared ? a.N * a.k + t : slots[t];
          a.dbuf[(size_t)s * a.H + row] = v;
        }
      }
    }
  }
}

template <int FR, int FS, int RPL>
__global__ __launch_bounds__(kThreads) void k_down(DownArgs a) {
  extern __shared__ uint4 smem[];
  const int bid = blockIdx.x;
  const bool is_shared = bid < a.gs.tiles;
  int e = 0, tile = 0, cols = 0;
  uint32_t mask = 0;
  int slots[kNmax];
  float wt[kNmax];
  const uint16_t* src[kNmax];
  if (is_shared) {
    tile = bid;
    cols = a.I_s;
#pragma unroll
    for (int t = 0; t < kNmax; ++t) {
      slots[t] = t;
      wt[t] = 1.0f;
      src[t] = a.a_shared + (size_t)t * a.I_s;
      if (t < a.N) mask |= 1u << t;
    }
  } else {
    const int r = bid - a.gs.tiles;
    const int unit = r / a.gr.tiles;
    tile = r - unit * a.gr.tiles;
    if (unit >= *a.num_units) return;
    e = a.unit_expert[unit];
    cols = a.I;
#pragma unroll
    for (int t = 0; t < kNmax; ++t) {
      const int s = a.unit_slot[unit * kNmax + t];
      slots[t] = s;
      wt[t] = a.unit_w[unit * kNmax + t];
      src[t] = a.a_routed + (size_t)(s < 0 ? 0 : s) * a.I;
      if (s >= 0) mask |= 1u << t;
    }
  }
  stage_rows(smem, src, mask, cols);
  __syncthreads();
  const uint32_t* xs = reinterpret_cast<const uint32_t*>(smem);
  if (is_shared) {
    if constexpr (FS != FMT_NONE)
      down_tile<FS, RPL>(a, a.sdown, 0, tile, a.gs, cols, xs, mask, slots, wt, true);
  } else {
    down_tile<FR, RPL>(a, a.down, e, tile, a.gr, cols, xs, mask, slots, wt, false);
  }
}

// ---------------------------------------------------------------------------
// 5. Weighted sum + shared blend (slot mode) or accumulator cast (atomic).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_blend(const float* dbuf, uint16_t* out, int N, int H,
                                                   int k, int has_shared) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= N * H) return;
  const int t = i / H;
  const int r = i - t * H;
  float y = 0.f;
  for (int j = 0; j < k; ++j) y += dbuf[(size_t)(t * k + j) * H + r];
  if (has_shared) y += dbuf[(size_t)(N * k + t) * H + r];
  out[i] = f32_to_bf16_rne(y);
}

__global__ __launch_bounds__(kThreads) void k_finalize(const float* acc, uint16_t* out, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) out[i] = f32_to_bf16_rne(acc[i]);
}

// ---------------------------------------------------------------------------
// Host-side launch planning and dispatch.
// ---------------------------------------------------------------------------
static int vpc_of(int fmt) {
  switch (fmt) {
    case FMT_BF16: return 8;
    case FMT_FP8: return 16;
    default: return 32;
  }
}

StageGeom plan_stage(int fmt, int cols, int rows, int units, bool /*two_mats*/) {
  StageGeom g;
  const int cpr = cols / vpc_of(fmt);
  int want = (cpr + IT - 1) / IT;
  int lpr = 8;
  while (lpr < want && lpr < 64) lpr <<= 1;
  g.lpr = lpr;
  const int groups = 64 / lpr;
  // two rows per lane group when that still leaves at least two workgroups
  // per compute unit
  const int rows_wg2 = (kThreads / 64) * groups * 2;
  const long wgs2 = (long)units * ((rows + rows_wg2 - 1) / rows_wg2);
  g.rpl = (wgs2 >= 512) ? 2 : 1;
  g.rows_per_wg = (kThreads / 64) * groups * g.rpl;
  g.tiles = (rows + g.rows_per_wg - 1) / g.rows_per_wg;
  return g;
}

int decode_num_launches() { return 5; }

template <int FR, int FS>
static hipError_t launch_experts(const Call& c, hipStream_t st, hipEvent_t* ev) {
  // gate + up
  GateUpArgs ga;
  ga.gate = c.gate;
  ga.up = c.up;
  ga.sgate = c.sgate;
  ga.sup = c.sup;
  ga.x = c.x;
  ga.N = c.N;
  ga.H = c.H;
  ga.k = c.k;
  ga.I = c.I;
  ga.I_s = c.I_s;
  ga.gr = c.gu_r;
  ga.gs = c.gu_s;
  ga.num_units = c.ws.num_units;
  ga.unit_expert = c.ws.unit_expert;
  ga.unit_slot = c.ws.unit_slot;
  ga.a_routed = c.ws.a_routed;
  ga.a_shared = c.ws.a_shared;
  ga.zero_buf = c.atomic ? c.ws.acc : nullptr;
  ga.zero_count = c.N * c.H;
  const int gu_blocks = c.gu_s.tiles + c.maxu * c.gu_r.tiles;
  const size_t gu_lds = (size_t)kNmax * c.H * 2;
  if (ev) hipEventRecord(ev[2], st);
  if (c.gu_r.rpl == 2)
    hipLaunchKernelGGL((k_gate_up<FR, FS, 2>), dim3(gu_blocks), dim3(kThreads), gu_lds, st, ga);
  else
    hipLaunchKernelGGL((k_gate_up<FR, FS, 1>), dim3(gu_blocks), dim3(kThreads), gu_lds, st, ga);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // down
  DownArgs da;
  da.down = c.down;
  da.sdown = c.sdown;
  da.a_routed = c.ws.a_routed;
  da.a_shared = c.ws.a_shared;
  da.N = c.N;
  da.H = c.H;
  da.k = c.k;
  da.I = c.I;
  da.I_s = c.I_s;
  da.gr = c.dn_r;
  da.gs = c.dn_s;
  da.num_units = c.ws.num_units;
  da.unit_expert = c.ws.unit_expert;
  da.unit_slot = c.ws.unit_slot;
  da.unit_w = c.ws.unit_w;
  da.dbuf = c.atomic ? nullptr : c.ws.dbuf;
  da.acc = c.atomic ? c.ws.acc : nullptr;
  const int dn_blocks = c.dn_s.tiles + c.maxu * c.dn_r.tiles;
  const int max_cols = c.I > c.I_s ? c.I : c.I_s;
  const size_t dn_lds = (size_t)kNmax * max_cols * 2;
  if (ev) hipEventRecord(ev[3], st);
  if (c.dn_r.rpl == 2)
    hipLaunchKernelGGL((k_down<FR, FS, 2>), dim3(dn_blocks), dim3(kThreads), dn_lds, st, da);
  else
    hipLaunchKernelGGL((k_down<FR, FS, 1>), dim3(dn_blocks), dim3(kThreads), dn_lds, st, da);
  return hipGetLastError();
}

// The shared expert (if any) uses the routed format or BF16.
template <int FR>
static hipError_t dispatch_shared(const Call& c, hipStream_t st, hipEvent_t* ev) {
  switch (c.sgate.fmt) {
    case FMT_NONE: return launch_experts<FR, FMT_NONE>(c, st, ev);
    case FMT_BF16: return launch_experts<FR, FMT_BF16>(c, st, ev);
    default: break;
  }
  if (c.sgate.fmt == FR) return launch_experts<FR, FR>(c, st, ev);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const Call& c, hipStream_t st, hipEvent_t* ev) {
  // 1. router
  RouterArgs ra{c.x, c.router_w, c.ws.logits, c.N, c.H, c.E};
  dim3 rgrid((c.E + 3) / 4, (c.N + kNmax - 1) / kNmax);
  if (ev) hipEventRecord(ev[0], st);
  hipLaunchKernelGGL(k_router, rgrid, dim3(kThreads), 0, st, ra);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // 2. top-k + plan
  TopkArgs ta;
  ta.logits = c.ws.logits;
  ta.bias = c.router_bias;
  ta.N = c.N;
  ta.E = c.E;
  ta.k = c.k;
  ta.scoring = c.scoring;
  ta.renorm = c.renorm;
  ta.maxu = c.maxu;
  ta.rsf = c.rsf;
  ta.idx = c.ws.idx;
  ta.wts = c.ws.wts;
  ta.out_idx = c.out_idx;
  ta.out_w = c.out_w;
  ta.out_logits = c.out_logits;
  ta.num_units = c.ws.num_units;
  ta.unit_expert = c.ws.unit_expert;
  ta.unit_slot = c.ws.unit_slot;
  ta.unit_w = c.ws.unit_w;
  if (ev) hipEventRecord(ev[1], st);
  hipLaunchKernelGGL(k_topk_plan, dim3(1), dim3(kThreads), 0, st, ta);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  // 3-4. experts
  switch (c.gate.fmt) {
    case FMT_BF16: err = dispatch_shared<FMT_BF16>(c, st, ev); break;
    case FMT_FP8: err = dispatch_shared<FMT_FP8>(c, st, ev); break;
    case FMT_MXFP4: err = dispatch_shared<FMT_MXFP4>(c, st, ev); break;
    case FMT_NVFP4: err = dispatch_shared<FMT_NVFP4>(c, st, ev); break;
    default: err = hipErrorInvalidValue; break;
  }
  if (err != hipSuccess) return err;

  // 5. epilogue
  const int n = c.N * c.H;
  if (ev) hipEventRecord(ev[4], st);
  if (c.atomic)
    hipLaunchKernelGGL(k_finalize, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, st,
                       c.ws.acc, c.out, n);
  else
    hipLaunchKernelGGL(k_blend, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, st,
                       c.ws.dbuf, c.out, c.N, c.H, c.k, c.I_s > 0 ? 1 : 0);
  err = hipGetLastError();
  if (ev) hipEventRecord(ev[5], st);
  return err;
}

}  // namespace moe
