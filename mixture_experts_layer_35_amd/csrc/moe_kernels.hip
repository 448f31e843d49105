// gfx950 kernel of the routed MoE layer forward, decode path (N <= 4).
//
// One launch runs the whole layer. Its workgroups fall into phases by id, and
// a workgroup only ever waits for work of lower ids, so every wait ends:
// workgroups are dispatched in id order, and producers never wait for their
// consumers. Every wait is also bounded; on expiry a sticky error word is set
// instead of hanging.
//
//   R   router  z[N,E] = x Wr^T, one wave per router row, the row read once
//               for all N tokens ("forward_k3.rs", MoeLayer::forward_k3,
//               step 1). The last router workgroup runs top-k for every token
//               (one wave per token, a (score, -index) argmax per round with
//               DPP reductions; softmax or sigmoid+bias weights, renorm,
//               routed scaling factor: step 2), lists the batch's distinct
//               experts ("units") in ascending expert order and publishes,
//               per (unit, token), the top-k position and routing weight.
//   GU  gate+up one workgroup per (unit, row tile): g = Wg x and u = Wu x for
//               the unit's tokens (x staged in LDS); a = silu(g) * u. The
//               shared expert is one more unit that takes every token and
//               needs no plan, so it streams while the router runs.
//   D   down    one workgroup per (unit, row tile): loads its weights first,
//               then reads the unit's activations as they land, d = Wd a. Slot mode
//               stores w*d per (slot, row); atomic mode adds w*d into an FP32
//               [N,H] accumulator ("forward_atomic_c4.rs"). The last
//               contributor to a block of output rows sums it (slot mode: in
//               slot order, then the shared expert) and writes BF16 (round
//               to nearest even).
//
// Hand-offs between workgroups. The 8 XCDs have separate L2 caches and an
// agent-scope fence writes back or invalidates a whole L2, so there are no
// fences: a word handed to another workgroup is written and read with
// relaxed agent-scope atomics (coherent per access, sc1). Data words are
// 64-bit, value in the high half and the call's tag in the low half; a reader
// accepts a word only with the current tag, so nothing has to be cleared
// between calls and a producer never waits for its stores to complete. A
// consumer reads the words it needs until they carry the tag (bounded); the
// only counters are the blend tickets of the atomic mode and the done count.
// The tag is the workspace's call counter plus one; the last workgroup to
// finish bumps the counter and clears the done count.
//
// Weights are read with 128-bit loads, `lpr` lanes per row, and dequantised
// in registers: FP4/FP8 pairs go to BF16 pairs with the gfx950 scaled
// converts, then into v_dot2_f32_bf16 against BF16 activations; block scales
// multiply per-chunk partial sums, row and tensor scales the row result; FP32
// accumulation throughout.
#include <mutex>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {

constexpr int IT = 4;  // 16-byte chunks per lane per row in flight per pass
// rows of one row block: 4 waves x (64 / lanes per row >= 8) x 2 rows per lane group
constexpr int kBlockRowsMax = 64;

typedef unsigned long long u64;

// ---------------------------------------------------------------------------
// Coherent (agent-scope relaxed atomic) loads and stores, tagged words.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned ld_coh(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_coh64(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh64(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 tagged(float v, unsigned tag) {
  return ((u64)__builtin_bit_cast(unsigned, v) << 32) | tag;
}
__device__ __forceinline__ u64 tagged_u(unsigned v, unsigned tag) { return ((u64)v << 32) | tag; }
__device__ __forceinline__ float tag_value(u64 w) {
  return __builtin_bit_cast(float, (unsigned)(w >> 32));
}

// This call's tag: the workspace call counter + 1 (never 0, the value of
// zero-filled memory); stable until the last workgroup has finished. Each
// phase reads it together with its own first loads, so that the read costs
// no round trip of its own.
__device__ __forceinline__ unsigned call_tag(const DecodeArgs& a) {
  return ld_coh(&a.ctl->epoch) + 1u;
}

__device__ __forceinline__ void set_error(const DecodeArgs& a, unsigned code) {
  __hip_atomic_fetch_or(&a.ctl->error, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Add 1 to *p once every wave of the workgroup got here; returns the old
// value to every thread. With `complete`, this thread's memory operations
// finish first (needed where the reader does not check tags).
__device__ __forceinline__ unsigned wg_signal(unsigned* p, unsigned* s_tmp, bool complete) {
  if (complete) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    *s_tmp = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *s_tmp;
}

// One workgroup's report to its done group, made by thread 0 after a
// barrier that followed every wave's read of the call's tag. Returns the
// count before it, which the workgroup looks at only when it ends.
__device__ __forceinline__ unsigned arrive_early(unsigned* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T sel4(int i, T v0, T v1, T v2, T v3) {
  return i == 0 ? v0 : (i == 1 ? v1 : (i == 2 ? v2 : v3));
}

// j-th set bit of a 4-bit mask (j < popcount)
__device__ __forceinline__ int nth_token(uint32_t mask, int j) {
  const int t0 = __builtin_ctz(mask | 16u);
  const uint32_t m1 = mask & (mask - 1);
  const int t1 = __builtin_ctz(m1 | 16u);
  const uint32_t m2 = m1 & (m1 - 1);
  const int t2 = __builtin_ctz(m2 | 16u);
  const uint32_t m3 = m2 & (m2 - 1);
  const int t3 = __builtin_ctz(m3 | 16u);
  return sel4(j, t0, t1, t2, t3);
}

// ---------------------------------------------------------------------------
// Streaming core: RPL rows of NM matrices (same shape and format) against the
// staged activations of up to kNmax tokens. Lane group (lpr lanes) of the
// wave owns rows row_base .. row_base+RPL-1; lane li of the group owns chunks
// li, li+lpr, ... of each row. One pass covers lpr*IT chunks of every row.
// ---------------------------------------------------------------------------
template <int F, int NM, int RPL>
struct Stream {
  // FP4 block scales: BPC bytes per 16-byte chunk. The scale bits of one
  // pass (lpr * IT chunks of a row) are contiguous, so lane li of a group
  // fetches 32-bit word li (and lpr + li when SW == 2) of them, one load per
  // row, and spread() deals each lane the bits of its own IT chunks.
  static constexpr bool kChunkScales = F == FMT_MXFP4 || F == FMT_NVFP4;
  static constexpr int BPC = F == FMT_NVFP4 ? 2 : 1;
  static constexpr int CPW = 4 / BPC;             // chunks per scale word
  static constexpr int SW = kChunkScales ? IT / CPW : 1;  // scale words per lane per row
  uint4 wq[IT][NM][RPL];
  uint32_t sc[IT][NM][RPL];
  uint32_t sw[NM][RPL][SW];
  float acc[NM][RPL][kNmax];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int t = 0; t < kNmax; ++t) acc[m][r][t] = 0.f;
  }

  // the scale words of the pass at chunk c0 (issued ahead of its weights).
  // Scale rows that are not 4-byte aligned take their bytes one by one.
  __device__ __forceinline__ void load_scales(const MatView (&mv)[NM], int row_base, int nrows,
                                              int cpr, int lpr, int li, int c0) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const bool whole = ((mv[m].scale_row_bytes | (int)(uintptr_t)mv[m].scales) & 3) == 0;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const int row = row_base + r;
#pragma unroll
        for (int w = 0; w < SW; ++w) {
          const int cw = c0 + (w * lpr + li) * CPW;  // first chunk of the word
          uint32_t v = 0u;
          if (row < nrows && cw < cpr) {
            const uint8_t* p = mv[m].scales + (size_t)row * mv[m].scale_row_bytes + cw * BPC;
            if (whole) {
              v = *reinterpret_cast<const uint32_t*>(p);
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (cw + j / BPC < cpr) v |= (uint32_t)p[j] << (8 * j);
            }
          }
          sw[m][r][w] = v;
        }
      }
    }
  }

  // sc[it] = the scale bits of chunk c0 + it*lpr + li: word
  // (it*lpr + li) / CPW of the pass, i.e. word it / CPW of lane
  // (it % CPW) * lpr / CPW + li / CPW of the group. Every lane of the wave
  // takes part (a permute reads zero from an inactive lane).
  __device__ __forceinline__ void spread(int lpr, int li) {
    const int lane = threadIdx.x & 63;
    const int base = lane - li + li / CPW;
    const int shift = (li % CPW) * 8 * BPC;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int addr = (base + (it % CPW) * (lpr / CPW)) * 4;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int r = 0; r < RPL; ++r)
          sc[it][m][r] =
              (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)sw[m][r][it / CPW]) >> shift;
    }
  }

  // chunk sets I0 .. I1-1 of one pass (the pipelined loops below fetch the
  // two halves of the next pass while computing the two halves of this one)
  template <int I0, int I1>
  __device__ __forceinline__ void load_its(const MatView (&mv)[NM], int row_base, int nrows,
                                           int cpr, int lpr, int li, int c0) {
    if constexpr (kChunkScales && I0 == 0) load_scales(mv, row_base, nrows, cpr, lpr, li, c0);
#pragma unroll
    for (int it = I0; it < I1; ++it) {
      const int c = c0 + it * lpr + li;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
          const int row = row_base + r;
          if (c < cpr && row < nrows)
            wq[it][m][r] = ldg16(mv[m].data + (size_t)row * mv[m].row_bytes + (size_t)c * 16);
          else
            wq[it][m][r] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
  }

  __device__ __forceinline__ void load(const MatView (&mv)[NM], int row_base, int nrows, int cpr,
                                       int lpr, int li, int c0) {
    load_its<0, IT>(mv, row_base, nrows, cpr, lpr, li, c0);
  }

  template <int I0, int I1>
  __device__ __forceinline__ void compute_its(int cpr, int lpr, int li, int c0, const uint32_t* xs,
                                              int xs_tok_words, uint32_t mask) {
    constexpr int XW = Fmt<F>::VPC / 2;  // 32-bit activation words per chunk
    if constexpr (kChunkScales && I0 == 0) spread(lpr, li);
#pragma unroll
    for (int it = I0; it < I1; ++it) {
      const int c = c0 + it * lpr + li;
      if (c >= cpr) continue;
#pragma unroll
      for (int t = 0; t < kNmax; ++t) {
        if (!((mask >> t) & 1u)) continue;
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
          for (int r = 0; r < RPL; ++r)
            acc[m][r][t] += chunk_dot<F>(wq[it][m][r], sc[it][m][r], xv);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  __device__ __forceinline__ void compute(int cpr, int lpr, int li, int c0, const uint32_t* xs,
                                          int xs_tok_words, uint32_t mask) {
    compute_its<0, IT>(cpr, lpr, li, c0, xs, xs_tok_words, mask);
  }

  // One step of a software-pipelined stream: compute this pass (column
  // offset c0) half by half, and after each half issue the same half of the
  // next pass (rows nrow_base, offset nc0) into the registers it freed, so
  // that the next pass's weights are in flight while this one is computed.
  __device__ __forceinline__ void step(const MatView (&mv)[NM], bool more, int nrow_base,
                                       int nrows, int nc0, int cpr, int lpr, int li, int c0,
                                       const uint32_t* xs, int xs_tok_words, uint32_t mask) {
    compute_its<0, IT / 2>(cpr, lpr, li, c0, xs, xs_tok_words, mask);
    if (more) load_its<0, IT / 2>(mv, nrow_base, nrows, cpr, lpr, li, nc0);
    compute_its<IT / 2, IT>(cpr, lpr, li, c0, xs, xs_tok_words, mask);
    if (more) load_its<IT / 2, IT>(mv, nrow_base, nrows, cpr, lpr, li, nc0);
  }

  // row sums land in the last lane of each lane group
  __device__ __forceinline__ void reduce(int lpr, uint32_t mask) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int t = 0; t < kNmax; ++t)
          if ((mask >> t) & 1u) acc[m][r][t] = group_sum_last(acc[m][r][t], lpr);
  }
};

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
// Staging of activation rows into LDS (token t's row at LDS word
// t * cols/2). Only tokens in `mask` are copied; each thread issues up to SB
// loads before it stores any.
// ---------------------------------------------------------------------------
// BF16 input rows: token t at x + t * cols
// All n rows of x ([n, cols] BF16, contiguous) into LDS bytes [0, n*cols*2)
// with direct global-to-LDS loads: each wave instruction moves 1 KiB (16
// bytes per lane, lane i to LDS offset 16 i) and no registers hold the data,
// so the whole block is in flight at once. The caller waits (vmcnt) and
// synchronises before reading it.
__device__ __forceinline__ void stage_x_async(uint4* lds, const uint16_t* x, int n, int cols) {
  const int bytes = n * cols * 2;  // a multiple of 16
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(x);
  uint8_t* dst = reinterpret_cast<uint8_t*>(lds);
  for (int off = wave * 1024; off < bytes; off += (kThreads / 64) * 1024) {
    const int my = off + lane * 16;
    if (my < bytes)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + my),
                                       (__attribute__((address_space(3))) void*)(dst + off), 16,
                                       0, 0);
  }
}


// Tagged BF16 activation pairs from other workgroups: token t's row of cols
// values is cols/2 words at base + row_t * cols/2, each word a BF16 pair
// (high half) and the call's tag (low half). Words without the current tag
// are read again (bounded). The pairs go to LDS as they are.
__device__ __forceinline__ void stage_tagged(const DecodeArgs& a, uint4* lds, const u64* base,
                                             int r0, int r1, int r2, int r3, uint32_t mask,
                                             int cols, unsigned tag) {
  constexpr int Q = 4;  // loads in flight per thread
  const int m = __builtin_popcount(mask);
  uint32_t* w = reinterpret_cast<uint32_t*>(lds);
  const int per = cols / 2;  // pairs per row
  const int total = m * per;
  auto src = [&](int i) {
    const int j = i / per;
    const int row = sel4(nth_token(mask, j), r0, r1, r2, r3);
    return base + (size_t)row * per + (i - j * per);
  };
  for (int i0 = threadIdx.x; i0 < total; i0 += kThreads * Q) {
    u64 v[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = i0 + q * kThreads;
      v[q] = i < total ? ld_coh64(src(i)) : (u64)tag;
    }
    unsigned spins = 0;
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int q = 0; q < Q; ++q) ok = ok && (unsigned)v[q] == tag;
      if (ok) break;
      __builtin_amdgcn_s_sleep(2);
      if (++spins > a.spin_limit) {
        set_error(a, 2u);
        break;
      }
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if ((unsigned)v[q] != tag) v[q] = ld_coh64(src(i0 + q * kThreads));
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = i0 + q * kThreads;
      if (i < total) {
        const int j = i / per;
        w[nth_token(mask, j) * per + (i - j * per)] = (uint32_t)(v[q] >> 32);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Phase R: router rows, then (last router workgroup) top-k and the plan.
// ---------------------------------------------------------------------------
struct TopkScratch {
  unsigned bits[8];  // the selected experts of [e_lo, e_hi), one bit each
  int uexp[256];
  int jpos[256 * kNmax];
  float uw[256 * kNmax];
};

__device__ __forceinline__ void topk_and_plan(const DecodeArgs& a, TopkScratch* s, unsigned tag) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  if (tid < 8) s->bits[tid] = 0u;
  for (int i = tid; i < 256 * kNmax; i += kThreads) {
    s->jpos[i] = -1;
    s->uw[i] = 0.f;
  }
  __syncthreads();  // (before the logits arrive)
  // routing is on the critical path of every later workgroup: issue first
  // on this compute unit
  __builtin_amdgcn_s_setprio(3);
  // the bias does not depend on the logits: read it before waiting for them
  float bv[4];
  load_bias4(a.tid2eid ? nullptr : a.router_bias, a.EW, lane, bv);
  // wave t routes token t (N <= kNmax waves); lane j < k holds slot (t, j).
  // The routing's global outputs (logits, indices, weights, slot flags) are
  // written after the plan is published: the barriers below then wait for
  // LDS only, not for those stores.
  static_assert(kThreads / 64 >= kNmax, "one routing wave per token");
  const int rt = wave;  // the token this wave routes
  const bool routes = rt < a.N;
  int slot_e = -1;
  float slot_w = 0.f;
  float zv[4];
  if (routes) {
    const int id = a.tid2eid ? a.token_ids[rt] : 0;  // hash routing: the token's id
    const u64* zrow = a.ctl->zlog + rt * 256;
    u64 zw[4] = {(u64)tag, (u64)tag, (u64)tag, (u64)tag};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < a.EW) zw[i] = ld_coh64(zrow + lane + 64 * i);
    unsigned spins = 0;
    while (!__all((unsigned)zw[0] == tag && (unsigned)zw[1] == tag && (unsigned)zw[2] == tag &&
                  (unsigned)zw[3] == tag)) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > a.spin_limit) {
        if (lane == 0) set_error(a, 4u);
        break;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((unsigned)zw[i] != tag) zw[i] = ld_coh64(zrow + lane + 64 * i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) zv[i] = lane + 64 * i < a.EW ? tag_value(zw[i]) : -INFINITY;
    int my_e;
    float w;
    if (!route_token(zv, bv, a.router_bias != nullptr, a.tid2eid, a.vocab, id, a.EW, a.k,
                     a.scoring, a.renorm, a.rsf, lane, my_e, w) &&
        lane == 0)
      set_error(a, kErrHashInput);
    if (lane < a.k) {
      const bool real = my_e >= a.e_lo && my_e < a.e_hi;
      if (real) atomicOr(&s->bits[my_e >> 5], 1u << (my_e & 31));
      slot_e = my_e;
      slot_w = w;
    }
  }
  __syncthreads();
  // units: the distinct selected experts this call computes (those in
  // [e_lo, e_hi): all of them, or one expert-parallel share's range), in
  // ascending order; a slot's unit is the number of selected experts below
  // its own
  unsigned bw[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) bw[q] = s->bits[q];
  int nu = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) nu += __popc(bw[q]);
  if (slot_e >= a.e_lo && slot_e < a.e_hi) {
    const int wq = slot_e >> 5;
    int u = 0;
    unsigned word = 0u;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      u += q < wq ? __popc(bw[q]) : 0;
      word = q == wq ? bw[q] : word;
    }
    u += __popc(word & ((1u << (slot_e & 31)) - 1u));
    const int t = rt, j = lane;
    s->uexp[u] = slot_e;
    s->jpos[u * kNmax + t] = j;
    s->uw[u * kNmax + t] = slot_w;
  }
  __syncthreads();
  // publish two tagged words per (unit, token): the plan info and the weight
  for (int ut = tid; ut < a.maxu * kNmax; ut += kThreads) {
    const int u = ut / kNmax;
    const int t = ut - u * kNmax;
    unsigned info = 0u;
    float wt = 0.f;
    if (u >= nu) {
      info = kPlanAbsent;
    } else {
      info = (unsigned)s->uexp[u] << 16;
      const int j = s->jpos[ut];
      if (j >= 0) {
        info |= kPlanPresent | (unsigned)j;
        wt = s->uw[ut];
      }
    }
    u64* p = a.ctl->plan + u * kPlanStride + 2 * t;
    st_coh64(p, tagged_u(info, tag));
    st_coh64(p + 1, tagged(wt, tag));
  }
  // the routing's outputs
  if (routes) {
    if (a.out_logits) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < a.EW) a.out_logits[(size_t)rt * a.EW + lane + 64 * i] = zv[i];
    }
    if (lane < a.k) {
      const int sl = rt * a.k + lane;
      if (a.out_idx) a.out_idx[sl] = (uint32_t)slot_e;
      if (a.out_w) a.out_w[sl] = slot_w;
      if (a.slot_flags)
        st_coh64(&a.ctl->slot_real[sl],
                 tagged_u(slot_e >= a.e_lo && slot_e < a.e_hi ? 1u : 0u, tag));
    }
  }
}

// This wave's part of one router row's dot products with the N tokens,
// format RF: BF16 (8 values per 16-byte chunk) or NVFP4 (32 values per chunk
// with two E4M3 block scales). The row's chunks are dealt to the wpr waves of
// the row and their 64 lanes in turn (lane l of wave q takes chunks
// q * 64 + l + j * wpr * 64), RPR chunks per lane per round, all of a round's
// row and token loads in flight together; x is read from global memory
// (L2). Only the N real tokens are loaded and multiplied. The call's tag is
// read into `tag` right after the first round's loads are issued, so that
// both are in flight together; returns false if this wave had no chunk of the
// row (and so did not read the tag).
template <int RF>
__device__ __forceinline__ bool router_row(const DecodeArgs& a, const uint8_t* wrow,
                                           const uint8_t* srow, int q, int wpr, int lane,
                                           float (&acc)[kNmax], unsigned& tag) {
  bool have_tag = false;
  constexpr int VPC = Fmt<RF>::VPC;
  constexpr int XU = VPC / 8;  // 16-byte x loads per token and chunk
  constexpr int RPR = RF == FMT_BF16 ? 4 : 1;
  const int cpr = a.H / VPC;
  const int stride = wpr * 64;
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.x);
  for (int c0 = q * 64 + lane; c0 - lane < cpr; c0 += stride * RPR) {
    uint4 wq[RPR], xq[RPR][kNmax][XU];
    uint32_t sc[RPR];
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int r = 0; r < RPR; ++r) {
      const int c = c0 + r * stride;
      const bool in = c < cpr;
      wq[r] = in ? ldg16(wrow + (size_t)c * 16) : z;
      sc[r] = (RF != FMT_BF16 && in) ? load_chunk_scale<RF>(srow, c) : 0u;
#pragma unroll
      for (int t = 0; t < kNmax; ++t)
#pragma unroll
        for (int u = 0; u < XU; ++u)
          xq[r][t][u] = (in && t < a.N)
                            ? ldg16(xb + (size_t)t * a.H * 2 + (size_t)c * VPC * 2 + u * 16)
                            : z;
    }
    if (!have_tag) {  // the first round: the call's tag joins its loads
      tag = call_tag(a);
      have_tag = true;
    }
#pragma unroll
    for (int r = 0; r < RPR; ++r) {
#pragma unroll
      for (int t = 0; t < kNmax; ++t) {
        if (t >= a.N) continue;
        uint32_t xv[VPC / 2];
#pragma unroll
        for (int u = 0; u < XU; ++u) {
          xv[4 * u + 0] = xq[r][t][u].x;
          xv[4 * u + 1] = xq[r][t][u].y;
          xv[4 * u + 2] = xq[r][t][u].z;
          xv[4 * u + 3] = xq[r][t][u].w;
        }
        acc[t] += chunk_dot<RF>(wq[r], sc[r], xv);
      }
    }
  }
  return have_tag;
}

__device__ __forceinline__ void router_phase(const DecodeArgs& a, int wg, uint4* smem,
                                             float* s_part, unsigned& tag) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  // a.r_wpr waves share one router row (K split), so that a long row is one
  // round of loads per wave
  const int wpr = a.r_wpr;
  const int q = wave & (wpr - 1);
  const int e = wg * ((kThreads / 64) / wpr) + wave / wpr;
  // rows 0..EW-1: the router (BF16 or NVFP4); row EW (with a shared-expert
  // gate): w_sg, BF16
  const bool has_row = e < a.EW + (a.shared_gate ? 1 : 0);
  float acc[kNmax] = {0.f, 0.f, 0.f, 0.f};
  // the call's tag, read after the row's first loads, while they are in
  // flight (router_row reads it; a wave without a chunk of a row, here)
  bool have_tag = false;
  if (has_row) {
    if (e < a.EW && a.router_fmt == FMT_NVFP4) {
      const MatView m = view_of(a.router_q, 0);
      have_tag = router_row<FMT_NVFP4>(a, m.data + (size_t)e * m.row_bytes,
                                       m.scales + (size_t)e * m.scale_row_bytes, q, wpr, lane,
                                       acc, tag);
#pragma unroll
      for (int t = 0; t < kNmax; ++t) acc[t] *= m.tensor_scale;
    } else {
      const uint8_t* wrow = e < a.EW
                                ? reinterpret_cast<const uint8_t*>(a.router_w) + (size_t)e * a.H * 2
                                : reinterpret_cast<const uint8_t*>(a.shared_gate);
      have_tag = router_row<FMT_BF16>(a, wrow, nullptr, q, wpr, lane, acc, tag);
    }
#pragma unroll
    for (int t = 0; t < kNmax; ++t)
      if (t < a.N) acc[t] = wave_sum_dpp(acc[t]);
  }
  if (!have_tag) tag = call_tag(a);
  if (wpr > 1) {
    // the row's partial sums meet in LDS; the row's first wave adds them in
    // a fixed order
    if (lane == 0)
#pragma unroll
      for (int t = 0; t < kNmax; ++t) s_part[wave * kNmax + t] = acc[t];
    __syncthreads();
    if (q == 0) {
#pragma unroll
      for (int t = 0; t < kNmax; ++t) {
        float v = s_part[wave * kNmax + t];
        for (int i = 1; i < wpr; ++i) v += s_part[(wave + i) * kNmax + t];
        acc[t] = v;
      }
    }
  }
  if (has_row && q == 0 && lane == 0) {
#pragma unroll
    for (int t = 0; t < kNmax; ++t)
      if (t < a.N)
        st_coh64(e < a.EW ? a.ctl->zlog + t * 256 + e : a.ctl->glog + t, tagged(acc[t], tag));
  }
  // the last router workgroup (it waits only on lower ids) routes
  if (wg != a.nR - 1) return;
  topk_and_plan(a, reinterpret_cast<TopkScratch*>(smem), tag);
}

// Unit u's plan (polling its tagged words); also reads the call's tag, in
// flight together with the first plan load. Returns false if the unit is
// absent. slots[t] = t*k + j for tokens routed to the unit, else -1.
__device__ __forceinline__ bool read_plan(const DecodeArgs& a, int u, unsigned& tag, int& expert,
                                          int (&slots)[kNmax], float (&wt)[kNmax],
                                          uint32_t& mask, u64* s_words) {
  const u64* p = a.ctl->plan + u * kPlanStride + (threadIdx.x & (2 * kNmax - 1));
  // first a plain load, which a workgroup starting after the plan was
  // published usually serves from its XCD's L2 (another workgroup of the
  // unit brought the line in); a word with another call's tag is read again
  // coherently, from memory. A word carries its tag, so a line cached before
  // the plan was written is never taken for it.
  // every lane loads a word (lanes past the plan's words repeat them), so the
  // loads and the tag's need no branch and share one wait
  u64 v = *p;
  tag = call_tag(a);
  if (threadIdx.x < 2 * kNmax) {
    unsigned spins = 0;
    while ((unsigned)v != tag) {
      v = ld_coh64(p);
      if ((unsigned)v == tag) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > a.spin_limit) {
        set_error(a, 1u);
        break;
      }
    }
    s_words[threadIdx.x] = v;
  }
  __syncthreads();
  const unsigned info0 = (unsigned)(s_words[0] >> 32);
  if (info0 & kPlanAbsent) return false;
  expert = (int)((info0 >> 16) & 0xffu);
  mask = 0;
#pragma unroll
  for (int t = 0; t < kNmax; ++t) {
    const unsigned info = (unsigned)(s_words[2 * t] >> 32);
    const bool present = t < a.N && (info & kPlanPresent);
    slots[t] = present ? t * a.k + (int)(info & 31u) : -1;
    wt[t] = tag_value(s_words[2 * t + 1]);
    if (present) mask |= 1u << t;
  }
  return true;
}

// ---------------------------------------------------------------------------
// Phase GU: gate + up and SiLU(gate) * up. A workgroup covers g.sub row
// blocks with one staging of x.
// ---------------------------------------------------------------------------
// The end of one gate+up row block, once its row sums are in st: the
// reduction, SiLU(gate) * up, and the hand-off of the block's activations as
// tagged BF16 pairs of adjacent rows (they meet in LDS first).
template <int F, int RPL>
__device__ __forceinline__ void gate_up_emit(Stream<F, 2, RPL>& st, const MatView (&mv)[2],
                                             int row_base, int lane_row, int brow0,
                                             int block_rows, int nrows, int lpr, int li,
                                             float* s_rows, uint32_t mask,
                                             const int (&slots)[kNmax], u64* dst,
                                             unsigned tag) {
  st.reduce(lpr, mask);
  if (li == lpr - 1) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int row = row_base + r;
      const float sg = row < nrows ? row_scale<F>(mv[0], row) : 0.f;
      const float su = row < nrows ? row_scale<F>(mv[1], row) : 0.f;
#pragma unroll
      for (int t = 0; t < kNmax; ++t) {
        const float gv = st.acc[0][r][t] * sg;
        const float uv = st.acc[1][r][t] * su;
        s_rows[(lane_row + r) * kNmax + t] = silu_f32(gv) * uv;
      }
    }
  }
  __syncthreads();
  const int pairs = block_rows / 2;
  const int m = __builtin_popcount(mask);
  for (int i = threadIdx.x; i < m * pairs; i += kThreads) {
    const int j = i / pairs;
    const int p = i - j * pairs;
    const int row = brow0 + 2 * p;  // brow0 is even
    if (row >= nrows) continue;     // nrows is even: the pair is whole
    const int t = nth_token(mask, j);
    const uint32_t lo = f32_to_bf16_rne(s_rows[(2 * p) * kNmax + t]);
    const uint32_t hi = f32_to_bf16_rne(s_rows[(2 * p + 1) * kNmax + t]);
    const int slot = sel4(t, slots[0], slots[1], slots[2], slots[3]);
    st_coh64(dst + (size_t)slot * (nrows / 2) + row / 2, tagged_u(lo | (hi << 16), tag));
  }
  __syncthreads();  // s_rows is refilled by the next block
}

template <int F, int RPL>
__device__ __forceinline__ void gate_up_tile(const DecodeArgs& a, const DevProj& pg,
                                             const DevProj& pu, int e, int tile,
                                             const StageGeom& g, int nrows, uint4* smem,
                                             float* s_rows, uint32_t mask,
                                             const int (&slots)[kNmax], u64* dst, unsigned tag) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpr = g.lpr;
  const int li = lane & (lpr - 1);
  const int cpr = a.H / Fmt<F>::VPC;
  const int block_rows = g.rows_per_wg / g.sub;
  const int lane_row = (wave * (64 / lpr) + lane / lpr) * RPL;
  const MatView mv[2] = {view_of(pg, e), view_of(pu, e)};
  const uint32_t* xs = reinterpret_cast<const uint32_t*>(smem);
  const int row0 = tile * g.rows_per_wg;
  // row blocks that hold rows (uniform)
  const int nsub = min(g.sub, (nrows - row0 + block_rows - 1) / block_rows);
  // passes (lpr * IT chunks of every row) of all row blocks in order, each
  // pass's weights fetched while the previous pass is computed; a block's
  // activations leave after its last pass
  const int step_c = lpr * IT;
  const int npass = (cpr + step_c - 1) / step_c;
  const int nsteps = nsub * npass;
  Stream<F, 2, RPL> st;
  st.zero();
  st.load(mv, row0 + lane_row, nrows, cpr, lpr, li, 0);
  int b = 0, p = 0;
#pragma nounroll
  for (int s = 0; s < nsteps; ++s) {
    int nb = b, np = p + 1;
    if (np == npass) {
      np = 0;
      ++nb;
    }
    st.step(mv, s + 1 < nsteps, row0 + nb * block_rows + lane_row, nrows, np * step_c, cpr, lpr,
            li, p * step_c, xs, a.H / 2, mask);
    if (np == 0) {
      const int brow0 = row0 + b * block_rows;
      gate_up_emit<F, RPL>(st, mv, brow0 + lane_row, lane_row, brow0, block_rows, nrows, lpr,
                           li, s_rows, mask, slots, dst, tag);
      st.zero();
    }
    b = nb;
    p = np;
  }
}

template <int FR, int FS, int RPL>
__device__ __forceinline__ void gate_up_phase(const DecodeArgs& a, int wg, uint4* smem,
                                              float* s_rows, u64* s_words, unsigned& tag) {
  int slots[kNmax];
  uint32_t mask = 0;
  // x does not depend on the routing: stage every token now, while the
  // router and top-k still run
  const uint32_t all = (1u << a.N) - 1u;
  stage_x_async(smem, a.x, a.N, a.H);
  if (wg < a.nGs) {
    tag = call_tag(a);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (FS != FMT_NONE) {
#pragma unroll
      for (int t = 0; t < kNmax; ++t) slots[t] = t;
      gate_up_tile<FS, RPL>(a, a.sgate, a.sup, 0, wg, a.gs, a.I_s, smem, s_rows, all, slots,
                            a.a_shared, tag);
    }
    return;
  }
  const int r = wg - a.nGs;
  const int unit = r / a.gr.tiles;
  const int tile = r - unit * a.gr.tiles;
  int e;
  float wt[kNmax];
  // the plan is read while x is still landing in LDS (one memory round trip
  // for both)
  const bool present = read_plan(a, unit, tag, e, slots, wt, mask, s_words);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (!present) return;
  gate_up_tile<FR, RPL>(a, a.gate, a.up, e - a.e_lo, tile, a.gr, a.I, smem, s_rows, mask,
                        slots, a.a_routed, tag);
}

// ---------------------------------------------------------------------------
// Phase D: down projections and the blend of each finished row block.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void blend_block(const DecodeArgs& a, int bt, unsigned tag) {
  __shared__ unsigned s_real[kNmax * 16];
  const int r0 = bt * a.blend_rows;
  const int r1 = min(a.H, r0 + a.blend_rows);
  const int rows = r1 - r0;
  if (!a.atomic && a.slot_flags) {
    // which slots have words (published with the routing)
    if ((int)threadIdx.x < a.N * a.k) {
      const u64* p = &a.ctl->slot_real[threadIdx.x];
      u64 v = ld_coh64(p);
      unsigned spins = 0;
      while ((unsigned)v != tag) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > a.spin_limit) {
          set_error(a, 8u);
          break;
        }
        v = ld_coh64(p);
      }
      s_real[threadIdx.x] = (unsigned)(v >> 32);
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < a.N * rows; i += kThreads) {
    const int t = i / rows;
    const int r = r0 + (i - t * rows);
    float y = 0.f;
    if (a.atomic) {
      float* p = a.acc + (size_t)t * a.H + r;
      y = ld_coh(p);
      st_coh(p, 0.f);  // leave the accumulator zeroed for the next call
    } else {
      // slots in order, then the shared expert; a slot whose expert no
      // workgroup of this call computes (a zero expert, another share's
      // expert) has no words and adds nothing. The words are requested four
      // slots at a time before any of them is waited for (those without this
      // call's tag are read again), so the reads cost a round trip per four
      // slots, not per slot.
      constexpr int G = 4;
      const int ns = a.k + (a.I_s > 0 ? 1 : 0);
      for (int j0 = 0; j0 < ns; j0 += G) {
        u64 v[G];
        const u64* p[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int j = j0 + g;
          const int slot = j < a.k ? t * a.k + j : a.N * a.k + t;
          const bool need = j < ns && (j >= a.k || !a.slot_flags || s_real[slot]);
          p[g] = need ? a.dbuf + (size_t)slot * a.H + r : nullptr;
          v[g] = need ? ld_coh64(p[g]) : (u64)tag;
        }
        unsigned spins = 0;
        for (;;) {
          bool all = true;
#pragma unroll
          for (int g = 0; g < G; ++g) all = all && (unsigned)v[g] == tag;
          if (all) break;
          __builtin_amdgcn_s_sleep(1);
          if (++spins > a.spin_limit) {
            set_error(a, 8u);
            break;
          }
#pragma unroll
          for (int g = 0; g < G; ++g)
            if ((unsigned)v[g] != tag) v[g] = ld_coh64(p[g]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (p[g]) y += tag_value(v[g]);
      }
    }
    if (a.out_f32)
      a.out_f32[(size_t)t * a.H + r] = y;  // an expert-parallel share's FP32 partial
    else
      a.out[(size_t)t * a.H + r] = f32_to_bf16_rne(y);
  }
}

template <int F, int RPL>
__device__ __forceinline__ void down_tile(const DecodeArgs& a, const DevProj& pd, int e, int tile,
                                          const StageGeom& g, int cols, uint4* smem,
                                          uint32_t mask, const int (&slots)[kNmax],
                                          const float (&wt)[kNmax], const u64* src, bool shared,
                                          unsigned tag) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpr = g.lpr;
  const int li = lane & (lpr - 1);
  const int block_rows = g.rows_per_wg / g.sub;
  const int lane_row = (wave * (64 / lpr) + lane / lpr) * RPL;
  const int cpr = cols / Fmt<F>::VPC;
  const MatView mv[1] = {view_of(pd, e)};
  const uint32_t* xs = reinterpret_cast<const uint32_t*>(smem);
  // the activations are staged once for g.sub row blocks; the first pass's
  // weights are in flight while the workgroup waits for them (it reads the
  // tagged activation words until they carry this call's tag: no counter
  // sits between the two phases). Row blocks that hold rows (uniform, at
  // least one):
  const int row0 = tile * g.rows_per_wg;
  const int nsb = min(g.sub, (a.H - row0 + block_rows - 1) / block_rows);
  // passes of all row blocks in order, each pass's weights fetched while the
  // previous pass is computed (as in gate+up)
  const int step_c = lpr * IT;
  const int npass = (cpr + step_c - 1) / step_c;
  const int nsteps = nsb * npass;
  Stream<F, 1, RPL> st;
  st.zero();
  st.load(mv, row0 + lane_row, a.H, cpr, lpr, li, 0);
  stage_tagged(a, smem, src, slots[0] < 0 ? 0 : slots[0], slots[1] < 0 ? 0 : slots[1],
               slots[2] < 0 ? 0 : slots[2], slots[3] < 0 ? 0 : slots[3], mask, cols, tag);
  __syncthreads();
  int b = 0, p = 0;
#pragma nounroll
  for (int s = 0; s < nsteps; ++s) {
    int nb = b, np = p + 1;
    if (np == npass) {
      np = 0;
      ++nb;
    }
    st.step(mv, s + 1 < nsteps, row0 + nb * block_rows + lane_row, a.H, np * step_c, cpr, lpr,
            li, p * step_c, xs, cols / 2, mask);
    const int row_base = row0 + b * block_rows + lane_row;
    b = nb;
    p = np;
    if (np != 0) continue;  // the block has passes left
    st.reduce(lpr, mask);
    if (li == lpr - 1) {
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const int row = row_base + r;
        if (row >= a.H) continue;
        const float rs = row_scale<F>(mv[0], row);
#pragma unroll
        for (int t = 0; t < kNmax; ++t) {
          if (!((mask >> t) & 1u)) continue;
          const float v = st.acc[0][r][t] * rs * sel4(t, wt[0], wt[1], wt[2], wt[3]);
          if (a.atomic) {
            __hip_atomic_fetch_add(a.acc + (size_t)t * a.H + row, v, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          } else {
            const int sl =
                shared ? a.N * a.k + t : sel4(t, slots[0], slots[1], slots[2], slots[3]);
            st_coh64(a.dbuf + (size_t)sl * a.H + row, tagged(v, tag));
          }
        }
      }
    }
    st.zero();
  }
}

// Rows per lane group in the down phase: twice the gate+up count for the
// two-row (large layer) kernels, so that a down workgroup, which streams a
// short matrix, has as many weight bytes in flight as a gate+up workgroup.
template <int RPL>
constexpr int kDownRpl = RPL == 2 ? 4 : RPL;

template <int FR, int FS, int RPL>
__device__ __forceinline__ void down_phase(const DecodeArgs& a, int wg, uint4* smem, unsigned* s_tmp,
                           u64* s_words, unsigned& tag, unsigned* done_ctr, bool& arrived,
                           unsigned& done_old) {
  int slots[kNmax];
  float wt[kNmax];
  uint32_t mask = 0;
  int row0;
  if (wg < a.nDs) {
    if constexpr (FS == FMT_NONE) {
      return;
    } else {
#pragma unroll
      for (int t = 0; t < kNmax; ++t) {
        slots[t] = t;
        wt[t] = 1.0f;
        if (t < a.N) mask |= 1u << t;
      }
      if (a.shared_gate) {
        // the shared output's weight sigmoid(x . w_sg): the gate logits come
        // from the router phase (tagged)
        const u64* p = a.ctl->glog + (threadIdx.x & (kNmax - 1));
        u64 v = ld_coh64(p);  // every lane (past N: a repeat), no branch
        tag = call_tag(a);
        if (threadIdx.x < a.N) {
          unsigned spins = 0;
          while ((unsigned)v != tag) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > a.spin_limit) {
              set_error(a, 4u);
              break;
            }
            v = ld_coh64(p);
          }
          s_words[threadIdx.x] = v;
        }
        __syncthreads();
        arrived = true;
        if (threadIdx.x == 0) done_old = arrive_early(done_ctr);
#pragma unroll
        for (int t = 0; t < kNmax; ++t)
          if (t < a.N) wt[t] = 1.0f / (1.0f + expf(-tag_value(s_words[t])));
      } else {
        tag = call_tag(a);
      }
      row0 = wg * a.ds.rows_per_wg;
      down_tile<FS, kDownRpl<RPL>>(a, a.sdown, 0, wg, a.ds, a.I_s, smem, mask, slots, wt, a.a_shared, true,
                         tag);
    }
  } else {
    const int r = wg - a.nDs;
    const int unit = r / a.dr.tiles;
    const int tile = r - unit * a.dr.tiles;
    row0 = tile * a.dr.rows_per_wg;
    int e;
    const unsigned defer = a.d_defer_ticks;  // (read before the plan's loads)
    const bool present = read_plan(a, unit, tag, e, slots, wt, mask, s_words);
    arrived = true;
    if (threadIdx.x == 0) done_old = arrive_early(done_ctr);
    if (present) {
      if (defer) {
        // (a resident grid: let the gate+up weights stream first)
        const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
        while (__builtin_amdgcn_s_memrealtime() - t0 < defer) __builtin_amdgcn_s_sleep(2);
      }
      down_tile<FR, kDownRpl<RPL>>(a, a.down, e - a.e_lo, tile, a.dr, a.I, smem, mask, slots, wt, a.a_routed,
                         false, tag);
    }
  }
  const int bt = row0 / a.blend_rows;
  const int rows_bt = min(a.blend_rows, a.H - bt * a.blend_rows);
  if (!a.atomic) {
    // slot mode: the highest-id contributor to the row block (the last unit's
    // last tile in it) blends; it reads tagged words, so nobody signals
    const int last_tile = (bt * a.blend_rows + rows_bt + a.dr.rows_per_wg - 1) / a.dr.rows_per_wg - 1;
    const int r = wg - a.nDs;
    if (wg >= a.nDs && r / a.dr.tiles == a.maxu - 1 && r - (a.maxu - 1) * a.dr.tiles == last_tile)
      blend_block(a, bt, tag);
    return;
  }
  // atomic mode: every routed unit slot (absent ones too) and the shared
  // expert take a ticket; the last one casts the accumulator
  const unsigned expect =
      (unsigned)a.maxu * (unsigned)((rows_bt + a.dr.rows_per_wg - 1) / a.dr.rows_per_wg) +
      (a.I_s > 0 ? (unsigned)((rows_bt + a.ds.rows_per_wg - 1) / a.ds.rows_per_wg) : 0u);
  const unsigned old = wg_signal(&a.blend_ctr[bt * kLineWords], s_tmp, true);
  if (old + 1 != expect) return;
  if (threadIdx.x == 0) st_coh(&a.blend_ctr[bt * kLineWords], 0u);
  blend_block(a, bt, tag);
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int FR, int FS, int RPL>
__global__ __launch_bounds__(kThreads, RPL == 1 ? 4 : 2) void k_moe_decode(DecodeArgs a) {
  extern __shared__ uint4 smem[];
  __shared__ unsigned s_tmp;
  __shared__ u64 s_words[2 * kNmax];
  __shared__ float s_rows[kBlockRowsMax * kNmax];
  const int bid = blockIdx.x;
  unsigned tag;  // this call's tag, read by each phase with its first loads
  // The call counter (the epoch, from which the next call takes its tag)
  // advances once every workgroup has read this call's tag: each workgroup
  // reports once, after its tag has reached all of its waves, and whichever
  // reports last advances it. Reports are counted in two levels (per done
  // group, then groups) so that no single counter takes an atomic from every
  // workgroup.
  const unsigned total = (unsigned)(a.nR + a.nGs + a.nGr + a.nDs + a.nDr);
  const unsigned g = (unsigned)bid % kDoneGroups;
  const unsigned in_group = (total - g + kDoneGroups - 1) / kDoneGroups;
  const unsigned groups = total < (unsigned)kDoneGroups ? total : (unsigned)kDoneGroups;
  unsigned* done_ctr = &a.ctl->group_done[g * kLineWords];
  // down workgroups report as soon as they hold the tag (their atomic's
  // result is looked at only here at the end), so that the last workgroups
  // to finish, which are down workgroups, end without a counting round trip
  bool arrived = false;
  unsigned d = 0;  // thread 0: the group count this workgroup's report met
  if (bid < a.nR) {
    router_phase(a, bid, smem, s_rows, tag);
  } else if (bid < a.nR + a.nGs + a.nGr) {
    gate_up_phase<FR, FS, RPL>(a, bid - a.nR, smem, s_rows, s_words, tag);
  } else {
    down_phase<FR, FS, RPL>(a, bid - a.nR - a.nGs - a.nGr, smem, &s_tmp, s_words, tag, done_ctr,
                            arrived, d);
  }
  if (!arrived) {
    // (the barrier inside waits for every wave's loads, the tag's included)
    d = wg_signal(done_ctr, &s_tmp, false);
  } else if (threadIdx.x != 0) {
    return;
  }
  if (d + 1 != in_group) return;
  if (threadIdx.x == 0) {
    st_coh(&a.ctl->group_done[g * kLineWords], 0u);
    const unsigned top =
        __hip_atomic_fetch_add(&a.ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (top + 1 == groups) {
      st_coh(&a.ctl->done, 0u);
      const unsigned next = tag == 0xffffffffu ? 0u : tag;  // keep the next tag non-zero
      st_coh(&a.ctl->epoch, next);
    }
  }
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

int lanes_per_row(int fmt, int cols) {
  const int cpr = cols / vpc_of(fmt);
  const int want = (cpr + IT - 1) / IT;
  int lpr = 8;
  while (lpr < want && lpr < 64) lpr <<= 1;
  return lpr;
}

StageGeom stage_geom(int fmt, int cols, int rows, int rpl, int sub) {
  StageGeom g;
  g.lpr = lanes_per_row(fmt, cols);
  g.rpl = rpl;
  g.sub = sub;
  g.rows_per_wg = (kThreads / 64) * (64 / g.lpr) * rpl * sub;
  g.tiles = (rows + g.rows_per_wg - 1) / g.rows_per_wg;
  return g;
}

size_t decode_lds_bytes(int H, int I, int I_s) {
  int maxc = H > I ? H : I;
  maxc = maxc > I_s ? maxc : I_s;
  size_t b = (size_t)kNmax * maxc * 2;
  if (b < sizeof(TopkScratch)) b = sizeof(TopkScratch);
  return (b + 15) / 16 * 16;
}

// With trace events, the launch goes through hipExtLaunchKernel, which
// stamps the events at the kernel's own start and end (the same interval a
// kernel trace reports) rather than around the enqueue.
// Workgroups of kernel fn (kThreads threads, lds bytes of dynamic LDS) that
// the current device holds at once. Queried once per device, kernel and LDS
// size, into a fixed table (no allocation: the no-workspace entry point
// launches through here too).
static int resident_wgs(const void* fn, size_t lds) {
  struct Entry {
    int dev;
    const void* fn;
    size_t lds;
    int v;
  };
  static Entry table[128];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (table[i].dev == dev && table[i].fn == fn && table[i].lds == lds) return table[i].v;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, kThreads, lds) != hipSuccess) per = 0;
  const int v = cus * per;  // 0 when unknown: never taken for resident
  if (used < 128) table[used++] = Entry{dev, fn, lds, v};
  return v;
}

template <int FR, int FS>
static hipError_t launch(const DecodeArgs& a, int rpl, size_t lds, hipStream_t st, hipEvent_t e0,
                         hipEvent_t e1) {
  const int blocks = a.nR + a.nGs + a.nGr + a.nDs + a.nDr;
  const void* fn = rpl == 2 ? reinterpret_cast<const void*>(&k_moe_decode<FR, FS, 2>)
                            : reinterpret_cast<const void*>(&k_moe_decode<FR, FS, 1>);
  DecodeArgs copy = a;
  if (copy.d_defer_ticks && blocks > resident_wgs(fn, lds)) copy.d_defer_ticks = 0;
  void* args[] = {&copy};
  if (e0 || e1)
    return hipExtLaunchKernel(fn, dim3(blocks), dim3(kThreads), args, lds, st, e0, e1, 0);
  return hipLaunchKernel(fn, dim3(blocks), dim3(kThreads), args, lds, st);
}

template <int FR>
static hipError_t dispatch_shared(const DecodeArgs& a, int fs, int rpl, size_t lds,
                                  hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  if (fs == FMT_NONE) return launch<FR, FMT_NONE>(a, rpl, lds, st, e0, e1);
  if (fs == FMT_BF16) return launch<FR, FMT_BF16>(a, rpl, lds, st, e0, e1);
  if (fs == FR) return launch<FR, FR>(a, rpl, lds, st, e0, e1);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int fr, int fs, int rpl, size_t lds,
                         hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  switch (fr) {
    case FMT_BF16: return dispatch_shared<FMT_BF16>(a, fs, rpl, lds, st, e0, e1);
    case FMT_FP8: return dispatch_shared<FMT_FP8>(a, fs, rpl, lds, st, e0, e1);
    case FMT_MXFP4: return dispatch_shared<FMT_MXFP4>(a, fs, rpl, lds, st, e0, e1);
    case FMT_NVFP4: return dispatch_shared<FMT_NVFP4>(a, fs, rpl, lds, st, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
