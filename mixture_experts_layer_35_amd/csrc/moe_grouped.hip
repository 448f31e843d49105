// gfx950 kernels of the routed MoE layer forward, grouped path (any N).
//
// The batch is sorted by expert so that each selected expert's weights are
// streamed once for all of the rows routed to it ("forward_batched.rs",
// MoeLayer::forward_batched: one router GEMM over the batch, then per-expert
// grouped work). Five stream-ordered launches:
//
//   router   z = x Wr^T as an MFMA GEMM, H split into ranges whose partial
//            logits are summed in a fixed order by the next kernel; also
//            clears the token masks
//   top-k    one wave per token: logits, top-k (shared with the decode path),
//            routing weights; sets bit t of mask[e] for each chosen e. The
//            last workgroup to finish then groups: tokens per expert from
//            the masks, counts padded to 16 rows, exclusive scan, and the
//            stable permutation of the N*k slots by (expert, token); each
//            slot's rank is the number of earlier tokens of the same expert
//            (a token picks an expert at most once), read off the mask words
//            with popcounts
//   gate+up  one workgroup per (unit, 64 output features): g and u for the
//            unit's rows as two 16x16 tiles per wave, a = silu(g) * u in BF16
//            into the permuted activation buffer; the shared expert is one
//            more unit holding every token
//   down     one workgroup per (unit, 64 or 128 output rows): d = Wd a; slot mode
//            stores d per permuted row, atomic mode adds w * d into an FP32
//            [N,H] accumulator
//   combine  y[t] = sum_j w[t,j] d[row(t,j)] + shared[t] in slot order, BF16
//            round to nearest even
//
// The MFMA streaming GEMM and the expert kernels are in moe_grouped.h; the
// expert kernels are instantiated per routed format in moe_grouped_*.hip.
#include "moe_grouped.h"
#include "moe_topk.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router: z partials. Workgroup = (row block of 128 experts, token group,
// K range); wave w owns expert rows rb*128 + 32w + [0, 32).
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(kGThreads) void k_g_router(GroupedArgs a) {
  extern __shared__ uint4 g_lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // clear the token masks (the top-k kernel, launched next, sets them) and,
  // with FP32 accumulation, the accumulator the down kernel adds into
  for (int i = blockIdx.x * kGThreads + tid; i < a.EL * a.WP + 1; i += gridDim.x * kGThreads)
    a.mask[i] = 0u;
  if (a.atomic) {
    float4* acc4 = reinterpret_cast<float4*>(a.acc);
    const int64_t n4 = (int64_t)a.N * a.H / 4;
    for (int64_t i = (int64_t)blockIdx.x * kGThreads + tid; i < n4;
         i += (int64_t)gridDim.x * kGThreads)
      acc4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (blockIdx.x == 0 && tid == 0) *a.ticket = 0u;
  const int s = blockIdx.x % a.ksplit;
  const int tg = (blockIdx.x / a.ksplit) % a.r_tg;
  const int rb = blockIdx.x / (a.ksplit * a.r_tg);
  const int c0 = s * a.kcps;
  const int nch = min(a.kcps, a.H / kGKC - c0);
  const int t0 = tg * 16 * NT;
  const int m = min(a.N - t0, 16 * NT);
  const XRows x{a.x + (int64_t)t0 * a.H + c0 * kGKC, a.H, nullptr, m};
  // Row blocks of 128 rows: rows 0..EW-1 are the router (E experts and the
  // zero experts, BF16 or NVFP4); with a shared-expert gate, the last block
  // holds only row EW, w_sg (BF16), since one block streams one format.
  const bool q_router = a.router_fmt == FMT_NVFP4;
  const bool gate_block = a.shared_gate && rb == a.r_rb - 1;
  auto store = [&](auto& acc, auto ntc, float scale) {
    constexpr int V = decltype(ntc)::value;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int n = 0; n < V; ++n) {
        const int j = n * 16 + (lane & 15);
        if (j < m) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int lr = 32 * wave + 16 * t + 4 * (lane >> 4) + r;  // row in the block
            int e;
            if (gate_block)
              e = lr == 0 ? a.EW : -1;
            else
              e = rb * kGRowsPerWG + lr;
            if (e >= 0 && (gate_block || e < a.EW))
              a.zpart[((int64_t)(t0 + j) * a.ksplit + s) * a.ER + e] = acc[t][n][r] * scale;
          }
        }
      }
  };
  ARow rows[2];
  if (q_router && !gate_block) {
    const MatView mq = gview(a.router_q, 0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int e = min(rb * kGRowsPerWG + 32 * wave + 16 * t + (lane & 15), a.EW - 1);
      rows[t] = arow(mq, e);
      rows[t].data += c0 * kGKC / 2;     // two E2M1 values per byte
      rows[t].scales += c0 * kGKC / 16;  // one E4M3 scale per 16 values
    }
    with_tiles<NT>((m + 15) >> 4, [&](auto ntc) {
      constexpr int V = decltype(ntc)::value;
      f32x4 acc[2][V];
      stream_gemm<FMT_NVFP4, 2, V>(acc, rows, x, nch, g_lds);
      store(acc, ntc, mq.tensor_scale);
    });
    return;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int e = min(rb * kGRowsPerWG + 32 * wave + 16 * t + (lane & 15), a.EW - 1);
    const uint16_t* wr = gate_block ? a.shared_gate : a.router_w + (int64_t)e * a.H;
    rows[t].data = reinterpret_cast<const uint8_t*>(wr + c0 * kGKC);
    rows[t].scales = nullptr;
  }
  with_tiles<NT>((m + 15) >> 4, [&](auto ntc) {
    constexpr int V = decltype(ntc)::value;
    f32x4 acc[2][V];
    stream_gemm<FMT_BF16, 2, V>(acc, rows, x, nch, g_lds);
    store(acc, ntc, 1.0f);
  });
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token; the last workgroup to finish then groups the
// slots by expert (group_slots below).
// ---------------------------------------------------------------------------
__device__ void group_slots(const GroupedArgs& a, uint4* lds);

// Device-coherent (agent-scope, relaxed) accesses for what the grouping
// workgroup reads from the other top-k workgroups of the same launch.
__device__ __forceinline__ int ld_dev(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kGThreads) void k_g_topk(GroupedArgs a) {
  extern __shared__ uint4 g_lds[];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kGThreads / 64) + (threadIdx.x >> 6);
  float zv[4] = {0.f, 0.f, 0.f, 0.f};
  int my_e = 0;
  float my_w = 0.f, gate_logit = 0.f;
  if (t < a.N) {
    const int id = a.tid2eid ? a.token_ids[t] : 0;  // hash routing: the token's id
    float bv[4];
    load_bias4(a.tid2eid ? nullptr : a.router_bias, a.EW, lane, bv);
    // sum the K-range partials of the lane's four logits in ascending range
    // order; lanes read consecutive experts, 16 ranges at a time
    const int ks = a.ksplit;
    for (int s0 = 0; s0 < ks; s0 += 16) {
      float v[4][16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float* p = a.zpart + ((int64_t)t * ks + s0 + q) * a.ER;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = lane + 64 * i;
          v[i][q] = (e < a.EW && s0 + q < ks) ? p[e] : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) zv[i] += v[i][q];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i >= a.EW) zv[i] = -INFINITY;
    float g = 0.f;
    if (a.shared_gate && lane == 0) {
      // the shared-expert weight sigmoid(x . w_sg), from router row EW
      for (int q = 0; q < ks; ++q) g += a.zpart[((int64_t)t * ks + q) * a.ER + a.EW];
    }
    if (!route_token(zv, bv, a.router_bias != nullptr, a.tid2eid, a.vocab, id, a.EW, a.k,
                     a.scoring, a.renorm, a.rsf, lane, my_e, my_w) &&
        lane == 0)
      __hip_atomic_fetch_or(a.err, kErrHashInput, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane < a.k) {
      st_dev(a.idx + t * a.k + lane, my_e);
      const int el = my_e - a.e_lo;  // only this call's experts are grouped
      if (el >= 0 && el < a.EL) atomicOr(a.mask + (int64_t)el * a.WP + (t >> 5), 1u << (t & 31));
    }
    gate_logit = g;
  }
  // the last workgroup to arrive groups the slots. idx is written with
  // device-coherent stores and mask with device atomics; each workgroup waits
  // for those to complete before taking its ticket (the only stores issued
  // so far), and the last one reads them with device-coherent loads (no
  // cache-wide fence either way)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(a.ticket, 1u) == gridDim.x - 1;
  __syncthreads();
  // the routing's other results (read by later launches or the caller only)
  if (t < a.N) {
    if (a.out_logits) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < a.EW) a.out_logits[(int64_t)t * a.EW + lane + 64 * i] = zv[i];
    }
    if (a.shared_gate && lane == 0) a.gamma[t] = 1.0f / (1.0f + expf(-gate_logit));
    if (lane < a.k) {
      const int sl = t * a.k + lane;
      a.wts[sl] = my_w;
      if (a.out_idx) a.out_idx[sl] = (uint32_t)my_e;
      if (a.out_w) a.out_w[sl] = my_w;
    }
  }
  if (!s_last) return;
  group_slots(a, g_lds);
}

// ---------------------------------------------------------------------------
// Grouping, by one workgroup (the last top-k workgroup).
// ---------------------------------------------------------------------------
// (The layout of the grouping's LDS, group_lds_layout, is in moe_internal.h.)
size_t grouped_group_lds(int E, int W) { return group_lds_layout(E, W).bytes; }

__device__ __forceinline__ uint64_t ld_dev64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// This code runs once per call, in one workgroup, with a cold instruction
// cache: the loops exit as soon as the call's sizes are covered (uniform
// conditions), so that small calls run little code.
__device__ void group_slots(const GroupedArgs& a, uint4* g_lds) {
  constexpr int kT = kGThreads;  // one thread per expert (E <= 256)
  constexpr int kSL = 32;        // slots per thread per pass, in groups of four
  constexpr int kML = 32;        // 8-byte mask loads per thread per batch
  const int E = a.EL, W = a.W, WP = a.WP;  // the experts this call computes
  const GroupLds L = group_lds_layout(E, W);
  char* lb = reinterpret_cast<char*>(g_lds);
  int* cnt = reinterpret_cast<int*>(lb);  // [256]
  int* base = cnt + 256;                  // [257]
  uint16_t* pre = reinterpret_cast<uint16_t*>(lb + L.pre_off);
  uint32_t* mlds = reinterpret_cast<uint32_t*>(lb + L.m_off);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nslots = a.N * a.k;
  // the first pass's experts, requested together with the masks
  int ev[kSL];
#pragma unroll
  for (int q = 0; q < kSL; ++q) ev[q] = -1;
#pragma unroll
  for (int q = 0; q < kSL; ++q) {
    if (q * kT >= nslots) break;
    const int sl = q * kT + tid;
    if (sl < nslots) ev[q] = ld_dev(a.idx + sl);
  }
  // the masks to LDS, a plain copy: kML loads in flight per thread, then
  // their stores
  {
    const int n2 = (E * WP + 1) / 2;
    const uint64_t* src = reinterpret_cast<const uint64_t*>(a.mask);
    uint64_t* dst = reinterpret_cast<uint64_t*>(mlds);
    for (int b0 = 0; b0 < n2; b0 += kML * kT) {
      uint64_t v[kML];
#pragma unroll
      for (int q = 0; q < kML; ++q) {
        if (b0 + q * kT >= n2) break;
        const int i = b0 + q * kT + tid;
        v[q] = i < n2 ? ld_dev64(src + i) : 0ull;
      }
#pragma unroll
      for (int q = 0; q < kML; ++q) {
        if (b0 + q * kT >= n2) break;
        const int i = b0 + q * kT + tid;
        if (i < n2) dst[i] = v[q];
      }
    }
  }
  lds_barrier();
  // tokens per expert, and the prefix before every fourth word: thread e
  // walks its words in order
  if (tid < E) {
    const uint32_t* m = mlds + tid * WP;
    int run = 0;
    for (int w = 0; w < W; ++w) {
      if ((w & 3) == 0) pre[tid * L.pw + (w >> 2)] = (uint16_t)run;
      run += __popc(m[w]);
    }
    cnt[tid] = run;
  }
  lds_barrier();
  // padded exclusive scan, the unit list and the work items (wave 0, four
  // experts per lane): a unit of c rows has ceil(c / T) items, T = 16 * nt
  // rows per pass of the expert kernels
  if (wave == 0) {
    const int T = 16 * a.nt;
    int pc[4], fl[4], ni[4], ps = 0, fs = 0, is = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      const int c = e < E ? cnt[e] : 0;
      pc[q] = (c + 15) & ~15;
      fl[q] = c > 0;
      ni[q] = (c + T - 1) / T;
      ps += pc[q];
      fs += fl[q];
      is += ni[q];
    }
    int ip = ps, ifl = fs, ii = is;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o1 = __shfl_up(ip, d, 64);
      const int o2 = __shfl_up(ifl, d, 64);
      const int o3 = __shfl_up(ii, d, 64);
      if (lane >= d) {
        ip += o1;
        ifl += o2;
        ii += o3;
      }
    }
    int b = ip - ps, u = ifl - fs, it = ii - is;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) {
        base[e] = b;
        if (fl[q]) {
          a.info->uexp[u] = e;
          a.info->ubase[u] = b;
          a.info->ucount[u] = cnt[e];
          for (int p = 0; p < ni[q]; ++p) a.info->item[it + p] = (u << 16) | p;
        }
      }
      b += pc[q];
      u += fl[q];
      it += ni[q];
    }
    if (lane == 63) {
      a.info->U = ifl;
      a.info->M = ip;
      a.info->nitems = ii;
      base[E] = ip;
    }
  }
  lds_barrier();
  // padding rows
  if (tid < E) {
    for (int r = base[tid] + cnt[tid]; r < base[tid + 1]; ++r) {
      a.perm_tok[r] = -1;
      a.perm_slot[r] = -1;
    }
  }
  // the slots, kSL per thread per pass (the first pass's experts were
  // requested above); slot sl belongs to token sl / k, stepped along with sl.
  // A slot's row is its expert's base plus the expert's tokens before the
  // slot's token (the stable order by token): the prefix of its four-word
  // group, the whole words before its word in the group and the bits below
  // the token in its word. A group of slots finds its rows from LDS with no
  // branch (every read is used, selected), then stores them, so that no
  // store stands between a load and the use of its value; lanes without a
  // slot of this share read row 0.
  const int k = a.k, dq = kT / k, dr = kT % k;
  for (int s0 = 0; s0 < nslots; s0 += kSL * kT) {
    if (s0 > 0) {
#pragma unroll
      for (int q = 0; q < kSL; ++q) {
        if (s0 + q * kT >= nslots) break;
        const int sl = s0 + q * kT + tid;
        ev[q] = sl < nslots ? ld_dev(a.idx + sl) : -1;
      }
    }
    int t = (int)((unsigned)(s0 + tid) / (unsigned)k), r = s0 + tid - t * k;
#pragma unroll
    for (int g = 0; g < kSL; g += 4) {
      if (s0 + g * kT >= nslots) break;
      int pos[4], tk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = ev[g + j] - a.e_lo;  // local expert index
        const bool ok = (unsigned)e < (unsigned)E;  // else another share's or none
        const int ec = ok ? e : 0, te = ok ? t : 0;
        const int wq = te >> 5, jm = wq & 3;
        const uint32_t* m = mlds + ec * WP;
        const int w0 = wq & ~3;
        const uint32_t m0 = m[w0], m1 = m[w0 + 1], m2 = m[w0 + 2], mw = m[wq];
        int rank = pre[ec * L.pw + (wq >> 2)] + base[ec];
        rank += __popc(m0 & (0u - (uint32_t)(jm > 0))) + __popc(m1 & (0u - (uint32_t)(jm > 1))) +
                __popc(m2 & (0u - (uint32_t)(jm > 2)));
        rank += __popc(mw & ((1u << (te & 31)) - 1u));
        pos[j] = ok ? rank : -1;
        tk[j] = t;
        t += dq;
        r += dr;
        if (r >= k) {
          r -= k;
          ++t;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sl = s0 + (g + j) * kT + tid;
        if (sl < nslots) {
          a.inv[sl] = pos[j];
          if (pos[j] >= 0) {
            a.perm_tok[pos[j]] = tk[j];
            a.perm_slot[pos[j]] = sl;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: four output columns per thread.
constexpr int kMaxTopk = 16;
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGThreads) void k_g_combine(GroupedArgs a) {
  const int64_t q = (int64_t)blockIdx.x * kGThreads + threadIdx.x;
  const int qpr = a.H / 4;
  if (q >= (int64_t)a.N * qpr) return;
  const int t = (int)(q / qpr);
  const int h = (int)(q - (int64_t)t * qpr) * 4;
  float4 y;
  if (a.atomic) {
    y = *reinterpret_cast<const float4*>(a.acc + (int64_t)t * a.H + h);
  } else {
    y = make_float4(0.f, 0.f, 0.f, 0.f);
    // the token's slot rows and weights first, then every slot's row of d,
    // all requested before any is added (k <= 16), added in slot order
    int row[kMaxTopk];
    float w[kMaxTopk];
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      row[j] = j < a.k ? a.inv[t * a.k + j] : -1;
      w[j] = j < a.k ? a.wts[t * a.k + j] : 0.f;
    }
    float4 d[kMaxTopk];
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j)  // row < 0: another share's expert, or no slot
      d[j] = row[j] >= 0 ? *reinterpret_cast<const float4*>(a.d_perm + (int64_t)row[j] * a.H + h)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      if (row[j] < 0) continue;
      y.x += w[j] * d[j].x;
      y.y += w[j] * d[j].y;
      y.z += w[j] * d[j].z;
      y.w += w[j] * d[j].w;
    }
    if (a.I_s > 0) {
      const float4 d = *reinterpret_cast<const float4*>(a.d_shared + (int64_t)t * a.H + h);
      const float g = a.shared_gate ? a.gamma[t] : 1.0f;
      y.x += g * d.x;
      y.y += g * d.y;
      y.z += g * d.z;
      y.w += g * d.w;
    }
  }
  if (a.out_f32)  // an expert-parallel share's FP32 partial
    *reinterpret_cast<float4*>(a.out_f32 + (int64_t)t * a.H + h) = y;
  else
    *reinterpret_cast<uint2*>(a.out + (int64_t)t * a.H + h) =
        make_uint2(pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w));
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
hipError_t launch_one(const void* fn, int blocks, int threads, size_t lds, hipStream_t st,
                      const GroupedArgs& a, hipEvent_t* ev, int i) {
  GroupedArgs copy = a;
  void* args[] = {&copy};
  if (blocks <= 0) {
    if (!ev) return hipSuccess;
    hipError_t e = hipEventRecord(ev[2 * i], st);
    return e != hipSuccess ? e : hipEventRecord(ev[2 * i + 1], st);
  }
  if (ev) return hipExtLaunchKernel(fn, dim3(blocks), dim3(threads), args, lds, st, ev[2 * i],
                                    ev[2 * i + 1], 0);
  return hipLaunchKernel(fn, dim3(blocks), dim3(threads), args, lds, st);
}

static const void* router_fn(int nt) {
  switch (nt) {
    case 1: return reinterpret_cast<const void*>(&k_g_router<1>);
    case 2: return reinterpret_cast<const void*>(&k_g_router<2>);
    case 4: return reinterpret_cast<const void*>(&k_g_router<4>);
    default: return reinterpret_cast<const void*>(&k_g_router<8>);
  }
}

hipError_t launch_grouped(const GroupedArgs& a, int fr, int fs, hipStream_t st, hipEvent_t* ev) {
  if (a.nt != 1 && a.nt != 2 && a.nt != 4 && a.nt != 8) return hipErrorInvalidValue;
  hipError_t err = launch_one(router_fn(a.nt), a.r_rb * a.r_tg * a.ksplit, kGThreads,
                              gemm_lds(a.nt), st, a, ev, 0);
  if (err != hipSuccess) return err;
  err = launch_one(reinterpret_cast<const void*>(&k_g_topk), (a.N + 3) / 4, kGThreads,
                   grouped_group_lds(a.EL, a.W), st, a, ev, 1);
  if (err != hipSuccess) return err;
  switch (fr) {
    case FMT_BF16: err = launch_experts<FMT_BF16>(a, fs, st, ev); break;
    case FMT_FP8: err = launch_experts<FMT_FP8>(a, fs, st, ev); break;
    case FMT_MXFP4: err = launch_experts<FMT_MXFP4>(a, fs, st, ev); break;
    case FMT_NVFP4: err = launch_experts<FMT_NVFP4>(a, fs, st, ev); break;
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess) return err;
  const int64_t quads = (int64_t)a.N * (a.H / 4);
  return launch_one(reinterpret_cast<const void*>(&k_g_combine),
                    (int)((quads + kGThreads - 1) / kGThreads), kGThreads, 0, st, a, ev, 4);
}

}  // namespace moe
