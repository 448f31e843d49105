// Device building blocks of the grouped path: the streaming MFMA GEMM that
// multiplies weight rows (A operand, dequantised in registers) against the
// activations of a unit's tokens (B operand, staged in LDS), and the
// gate+up and down kernels built on it. Included by the per-format
// translation units, which instantiate the kernels for their routed format.
//
// Weight rows are the A operand of v_mfma_f32_16x16x32_bf16 (lane l holds
// row l % 16, eight consecutive K values of group l / 16), the unit's tokens
// the B operand, read from an LDS copy of the current 128-column chunk of
// their activations. Every lane fetches 16 bytes of its row per load, so the
// four lanes of a row read 64 contiguous bytes; FP8/FP4 are dequantised to
// BF16 exactly (FP8, FP4 times an E8M0 or E4M3 block scale all fit in BF16);
// FP8 row scales and the NVFP4 tensor scale multiply the FP32 accumulators.
// Loads of the next weight block are in flight while the current one is
// multiplied.
//
// The number of 16-token tiles of a pass is a compile-time constant inside
// the MFMA loop (a runtime choice among 1, 2, 4 and 8 tiles selects the
// loop): the loop body then has no branch around an MFMA, so every read of an
// accumulator sits in straight-line code after the MFMA that wrote it.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGThreads = 256;

// Per format: 16-byte loads per lane per 128-column chunk (LPC) and MFMA
// K-steps of 8 values per load (SPL); LPC * SPL = 4.
template <int F> struct GF;
template <> struct GF<FMT_BF16> { static constexpr int LPC = 4, SPL = 1; };
template <> struct GF<FMT_FP8> { static constexpr int LPC = 2, SPL = 2; };
template <> struct GF<FMT_MXFP4> { static constexpr int LPC = 1, SPL = 4; };
template <> struct GF<FMT_NVFP4> { static constexpr int LPC = 1, SPL = 4; };

// Four 16-byte loads of one weight row (a "block": 1, 2 or 4 chunks) plus,
// for FP4, the block-scale bits of each chunk.
struct WBlock {
  uint4 q[4];
  uint32_t sc[4];
};

// Row pointer and scales of one lane's A-operand row.
struct ARow {
  const uint8_t* data;    // start of the row
  const uint8_t* scales;  // FP4: start of the row's block scales
};

// 16 and 12 bytes read with one load from a 4-byte aligned address
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));

// FP4 block scales of block blk (chunks 4 blk .. 4 blk + 3) of a row. MXFP4
// keeps one E8M0 byte per 32 values, bytes 4c .. 4c+3 for the four K groups
// of chunk c; NVFP4 two E4M3 bytes per 32 values, bytes 8c + 2g, 8c + 2g + 1
// for group g. The block's 16 (MXFP4) or 32 (NVFP4) scale bytes are
// contiguous, so a "whole" block (all four chunks present, scales 4-byte
// aligned) is read with wide loads: MXFP4 one 16-byte load (sc[ql] = word
// ql, group g's byte at bit 8g), NVFP4 two 12-byte loads from word g/2 of
// each chunk pair (sc[ql] = the word that holds group g's half-word, at bit
// 16 (g&1)). Any other block is read chunk by chunk (sc[ql] = the bits
// themselves). Nothing here waits for a load; a_operand finds the bits.
template <int F>
__device__ __forceinline__ void load_block_scales(WBlock& b, const ARow& r, int blk, int g,
                                                  int nchunks, bool whole) {
  if constexpr (F == FMT_MXFP4) {
    if (whole) {
      const u32x4_a4 s = *reinterpret_cast<const u32x4_a4*>(r.scales + blk * 16);
      b.sc[0] = s.x;
      b.sc[1] = s.y;
      b.sc[2] = s.z;
      b.sc[3] = s.w;
    } else {
#pragma unroll
      for (int ql = 0; ql < 4; ++ql) {
        const int c = blk * 4 + ql;
        b.sc[ql] = c < nchunks ? (uint32_t)r.scales[c * 4 + g] : 0u;
      }
    }
  } else if constexpr (F == FMT_NVFP4) {
    if (whole) {
      const uint8_t* p = r.scales + blk * 32 + 4 * (g >> 1);
      const u32x3_a4 s0 = *reinterpret_cast<const u32x3_a4*>(p);
      const u32x3_a4 s1 = *reinterpret_cast<const u32x3_a4*>(p + 16);
      b.sc[0] = s0.x;
      b.sc[1] = s0.z;
      b.sc[2] = s1.x;
      b.sc[3] = s1.z;
    } else {
#pragma unroll
      for (int ql = 0; ql < 4; ++ql) {
        const int c = blk * 4 + ql;
        b.sc[ql] =
            c < nchunks ? (uint32_t)*reinterpret_cast<const uint16_t*>(r.scales + c * 8 + g * 2) : 0u;
      }
    }
  }
}

// Whether block blk of rows with these scales is read whole (see above).
__device__ __forceinline__ bool scales_whole(bool aligned4, int blk, int nchunks) {
  return aligned4 && blk * 4 + 4 <= nchunks;
}

template <int F>
__device__ __forceinline__ void load_block(WBlock& b, const ARow& r, int blk, int g, int nchunks,
                                           bool whole) {
  constexpr int LPC = GF<F>::LPC;
  constexpr int XPB = 4 / LPC;  // chunks per block
#pragma unroll
  for (int ql = 0; ql < 4; ++ql) {
    const int c = blk * XPB + ql / LPC;
    const int q = ql % LPC;
    if (XPB > 1 && c >= nchunks) break;  // a short last block
    // byte offset of columns c*128 + q*(128/LPC) + g*(32/LPC)
    int64_t off;
    if constexpr (F == FMT_BF16) off = (int64_t)(c * 128 + q * 32 + g * 8) * 2;
    else if constexpr (F == FMT_FP8) off = c * 128 + q * 64 + g * 16;
    else off = (c * 128 + g * 32) / 2;
    b.q[ql] = *reinterpret_cast<const uint4*>(r.data + off);
  }
  if constexpr (F == FMT_MXFP4 || F == FMT_NVFP4)
    load_block_scales<F>(b, r, blk, g, nchunks, whole);
}

// The eight BF16 A values of K-step h of load ql.
template <int F>
__device__ __forceinline__ bf16x8 a_operand(const WBlock& b, int ql, int h, int g, bool whole) {
  const uint4 v = b.q[ql];
  if constexpr (F == FMT_BF16) {
    return __builtin_bit_cast(bf16x8, v);
  } else if constexpr (F == FMT_FP8) {
    const uint32_t d0 = h ? v.z : v.x, d1 = h ? v.w : v.y;
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
    bf16x8 r = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    return r;
  } else if constexpr (F == FMT_MXFP4) {
    // the E8M0 block scale is a power of two: the scaled convert applies it
    const uint32_t d = h == 0 ? v.x : (h == 1 ? v.y : (h == 2 ? v.z : v.w));
    const float s = e8m0_to_f32((whole ? b.sc[ql] >> (8 * g) : b.sc[ql]) & 0xffu);
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 3);
    bf16x8 r = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    return r;
  } else {
    // the scaled converts take only the exponent of their scale operand, so
    // the E4M3 block scale (which has mantissa bits) multiplies in FP32; the
    // product has at most 6 significant bits and converts to BF16 exactly
    const uint32_t d = h == 0 ? v.x : (h == 1 ? v.y : (h == 2 ? v.z : v.w));
    const uint32_t bits = whole ? b.sc[ql] >> (16 * (g & 1)) : b.sc[ql];
    const f32x2 s2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bits, 1.0f, false);
    const float s = h < 2 ? s2.x : s2.y;
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    bf16x8 r = {(__bf16)(p0.x * s), (__bf16)(p0.y * s), (__bf16)(p1.x * s), (__bf16)(p1.y * s),
                (__bf16)(p2.x * s), (__bf16)(p2.y * s), (__bf16)(p3.x * s), (__bf16)(p3.y * s)};
    return r;
  }
}

// Activation chunk in LDS: [16*NT tokens][128 BF16] = 256 bytes per token;
// the 16-byte unit u of token row j sits at unit u ^ (j & 15), so the 16
// tokens one MFMA reads hit 16 different bank groups.
__device__ __forceinline__ uint4* lds_unit(uint4* buf, int row, int u) {
  return buf + row * 16 + (u ^ (row & 15));
}

// Source rows of the activations of one pass.
struct XRows {
  const uint16_t* base;  // row r of the matrix at base + r * ld
  int64_t ld;            // elements per row
  const int* map;        // optional: matrix row of pass row j is map[j]
  int count;             // pass rows with data; the rest are zero
};

__device__ __forceinline__ int x_row(const XRows& x, int j) {
  if (j >= x.count) return -1;
  return x.map ? x.map[j] : j;
}

// Global loads of chunk c of the pass's activations (NT loads per thread).
template <int NT>
__device__ __forceinline__ void x_fetch(uint4 (&v)[NT], const int (&rows)[NT], const XRows& x,
                                        int c) {
  const int u = threadIdx.x & 15;
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    v[p] = make_uint4(0u, 0u, 0u, 0u);
    if (rows[p] >= 0)
      v[p] = *reinterpret_cast<const uint4*>(x.base + rows[p] * x.ld + c * kGKC + u * 8);
  }
}

template <int NT>
__device__ __forceinline__ void x_store(uint4* buf, const uint4 (&v)[NT]) {
  const int u = threadIdx.x & 15;
#pragma unroll
  for (int p = 0; p < NT; ++p) *lds_unit(buf, (threadIdx.x >> 4) + 16 * p, u) = v[p];
}

// Multiply-accumulate one 128-column chunk: NA weight tiles (16 rows each)
// against NT token tiles.
template <int F, int NA, int NT>
__device__ __forceinline__ void mma_chunk(f32x4 (&acc)[NA][NT], const WBlock (&w)[NA], int xc,
                                          const uint4* buf, bool whole) {
  constexpr int LPC = GF<F>::LPC, SPL = GF<F>::SPL;
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < LPC; ++q) {
    const int ql = xc * LPC + q;
#pragma unroll
    for (int h = 0; h < SPL; ++h) {
      bf16x8 A[NA];
#pragma unroll
      for (int t = 0; t < NA; ++t) A[t] = a_operand<F>(w[t], ql, h, g, whole);
      const int u = 4 * SPL * q + SPL * g + h;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const bf16x8 B = __builtin_bit_cast(bf16x8, buf[(n * 16 + j) * 16 + (u ^ j)]);
#pragma unroll
        for (int t = 0; t < NA; ++t)
          acc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t], B, acc[t][n], 0, 0, 0);
      }
    }
  }
}

// acc[t][n] = sum over K of W_t[row] * X[token] for the wave's NA tiles and
// the pass's 16*NT tokens, K = 128 * nchunks. All 256 threads of the
// workgroup stage the activations; lds holds two chunk buffers of 16*NT token
// rows.
template <int F, int NA, int NT>
__device__ __forceinline__ void stream_gemm(f32x4 (&acc)[NA][NT], const ARow (&rows)[NA],
                                            const XRows& x, int nchunks, uint4* lds) {
  constexpr int XPB = 4 / GF<F>::LPC;
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int t = 0; t < NA; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  int xr[NT];
#pragma unroll
  for (int p = 0; p < NT; ++p) xr[p] = x_row(x, (threadIdx.x >> 4) + 16 * p);
  uint4* buf0 = lds;
  uint4* buf1 = lds + 16 * 16 * NT;
  uint4 xv[NT];
  x_fetch<NT>(xv, xr, x, 0);
  x_store<NT>(buf0, xv);
  const int nblk = (nchunks + XPB - 1) / XPB;
  WBlock cur[NA], nxt[NA];
  // FP4 scales of one matrix share their alignment (rows and experts are
  // multiples of 4 bytes apart)
  const bool al4 = ((uintptr_t)rows[0].scales & 3) == 0;
#pragma unroll
  for (int t = 0; t < NA; ++t)
    load_block<F>(cur[t], rows[t], 0, g, nchunks, scales_whole(al4, 0, nchunks));
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    // the next block's weights are in flight while this one is multiplied
    if (blk + 1 < nblk) {
#pragma unroll
      for (int t = 0; t < NA; ++t)
        load_block<F>(nxt[t], rows[t], blk + 1, g, nchunks, scales_whole(al4, blk + 1, nchunks));
    }
#pragma unroll
    for (int xc = 0; xc < XPB; ++xc) {
      const int c = blk * XPB + xc;
      if (XPB > 1 && c >= nchunks) break;
      const bool more = c + 1 < nchunks;
      if (more) x_fetch<NT>(xv, xr, x, c + 1);
      mma_chunk<F, NA, NT>(acc, cur, xc, (c & 1) ? buf1 : buf0, scales_whole(al4, blk, nchunks));
      if (more) x_store<NT>((c & 1) ? buf0 : buf1, xv);
      __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < NA; ++t) cur[t] = nxt[t];
  }
}

// Calls fn(std::integral_constant<int, T>) with T the smallest of 1, 2, 4, 8
// (up to NTMAX) that covers nt token tiles.
template <int NTMAX, typename Fn>
__device__ __forceinline__ void with_tiles(int nt, Fn&& fn) {
  if (NTMAX == 1 || nt <= 1) {
    fn(std::integral_constant<int, 1>{});
    return;
  }
  if constexpr (NTMAX >= 2) {
    if (NTMAX == 2 || nt <= 2) {
      fn(std::integral_constant<int, 2>{});
      return;
    }
  }
  if constexpr (NTMAX >= 4) {
    if (NTMAX == 4 || nt <= 4) {
      fn(std::integral_constant<int, 4>{});
      return;
    }
  }
  if constexpr (NTMAX >= 8) fn(std::integral_constant<int, 8>{});
}

// Work item and tile of routed workgroup b of the gate+up kernels of two or
// more token tiles (batches above 64 tokens).
// Workgroup b runs on XCD b mod 8 (counted from the routed part's start), so
// items go in groups of eight, the tiles of item 8g + x all on one XCD and
// interleaved with the group's other seven: the tiles of an item then share
// that XCD's L2 copy of the item's token rows instead of each XCD fetching
// them. (With up to 64 tokens the rows are few and the plain order, the
// tiles of one item next to each other, measured faster.)
__device__ __forceinline__ void xcd_item(int b, int tiles, int& item, int& tile) {
  const int G = 8 * tiles;
  const int g = b / G, r = b - g * G;
  tile = r >> 3;
  item = 8 * g + (r & 7);
}

__device__ __forceinline__ MatView gview(const DevProj& p, int e) {
  MatView m;
  m.data = p.data + (int64_t)e * p.expert_bytes;
  m.scales = p.scales ? p.scales + (int64_t)e * p.scale_expert_bytes : nullptr;
  m.row_bytes = p.row_bytes;
  m.scale_row_bytes = p.scale_row_bytes;
  m.tensor_scale = p.tensor_scale ? p.tensor_scale[e] : 1.0f;
  return m;
}

__device__ __forceinline__ ARow arow(const MatView& m, int row) {
  ARow r;
  r.data = m.data + (int64_t)row * m.row_bytes;
  r.scales = m.scales ? m.scales + (int64_t)row * m.scale_row_bytes : nullptr;
  return r;
}

// Scale of output row `row` after the reduction: FP8 row scale, NVFP4
// tensor scale, else 1.
template <int F>
__device__ __forceinline__ float out_scale(const MatView& m, int row) {
  if constexpr (F == FMT_FP8) return reinterpret_cast<const float*>(m.scales)[row];
  else if constexpr (F == FMT_NVFP4) return m.tensor_scale;
  else return 1.0f;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// ---------------------------------------------------------------------------
// Gate+up. Workgroup = (unit, 64 features [, token group for the shared
// expert]); wave w owns features f0 + 16w + [0,16): tile 0 gate rows, tile 1
// up rows, so a lane holds g and u of the same (feature, token).
// ---------------------------------------------------------------------------
template <int F, int NT>
__device__ __forceinline__ void gate_up_pass(const MatView& mg, const MatView& mu, int f0,
                                             const XRows& x, uint16_t* dst, int64_t dst_ld,
                                             int store_rows, int nchunks, uint4* lds) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int frow = f0 + 16 * wave + (lane & 15);
  ARow rows[2] = {arow(mg, frow), arow(mu, frow)};
  f32x4 acc[2][NT];
  stream_gemm<F, 2, NT>(acc, rows, x, nchunks, lds);
  const int fo = f0 + 16 * wave + 4 * (lane >> 4);
  float sg[4], su[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sg[r] = out_scale<F>(mg, fo + r);
    su[r] = out_scale<F>(mu, fo + r);
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int j = n * 16 + (lane & 15);
    if (j < store_rows) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = silu_f32(acc[0][n][r] * sg[r]) * (acc[1][n][r] * su[r]);
      const uint2 pk = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      *reinterpret_cast<uint2*>(dst + j * dst_ld + fo) = pk;
    }
  }
}

// With one token tile (units of at most 16 tokens) the kernel is held to 128
// registers, four workgroups per compute unit: the grid then fits in one
// round of workgroups at the batched-decode sizes instead of leaving a tail.
template <int FR, int FS, int NTMAX>
__global__ __launch_bounds__(kGThreads, NTMAX == 1 ? 4 : 1) void k_g_gate_up(GroupedArgs a) {
  extern __shared__ uint4 g_lds[];
  const int bid = blockIdx.x;
  constexpr int T = 16 * NTMAX;
  const int nch = a.H / kGKC;
  if (bid < a.gu_s) {
    if constexpr (FS != FMT_NONE) {
      const int tiles = a.I_s / 64;
      const int tile = bid % tiles, tg = bid / tiles;
      const int t0 = tg * T;
      const int m = min(a.N - t0, T);
      const XRows x{a.x + (int64_t)t0 * a.H, a.H, nullptr, m};
      const MatView mg = gview(a.sgate, 0), mu = gview(a.sup, 0);
      uint16_t* dst = a.a_shared + (int64_t)t0 * a.I_s;
      with_tiles<NTMAX>((m + 15) >> 4, [&](auto nt) {
        gate_up_pass<FS, decltype(nt)::value>(mg, mu, tile * 64, x, dst, a.I_s, m, nch, g_lds);
      });
    }
    return;
  }
  // one work item: T rows (a pass) of one unit
  const int b = bid - a.gu_s;
  int i, tile;
  if constexpr (NTMAX >= 2) {
    xcd_item(b, a.gu_r, i, tile);
  } else {
    i = b / a.gu_r;
    tile = b - i * a.gu_r;
  }
  if (i >= a.info->nitems) return;
  const int item = a.info->item[i];
  const int u = item >> 16, p0 = (item & 0xffff) * T;
  const int e = a.info->uexp[u], cnt = a.info->ucount[u], rb = a.info->ubase[u];
  const int mpad = (cnt + 15) & ~15;
  const MatView mg = gview(a.gate, e), mu = gview(a.up, e);
  const XRows x{a.x, a.H, a.perm_tok + rb + p0, min(cnt - p0, T)};
  const int rows = min(mpad - p0, T);  // padding rows get a = 0
  uint16_t* dst = a.a_perm + (int64_t)(rb + p0) * a.I;
  with_tiles<NTMAX>((rows + 15) >> 4, [&](auto nt) {
    gate_up_pass<FR, decltype(nt)::value>(mg, mu, tile * 64, x, dst, a.I, rows, nch, g_lds);
  });
}

// ---------------------------------------------------------------------------
// Down. Workgroup = (unit, DR output rows [, token group]), DR = 64 or 128
// (g_down_rows); wave w owns rows h0 + 16 NA w + [0, 16 NA) as NA = DR / 64
// tiles.
// ---------------------------------------------------------------------------
template <int F, int NT, int NA = 2>
__device__ __forceinline__ void down_pass(const GroupedArgs& a, const MatView& md, int h0,
                                          const XRows& x, int nchunks, int rows, bool shared,
                                          int row0, uint4* lds) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  ARow ar[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) ar[t] = arow(md, h0 + 16 * NA * wave + 16 * t + (lane & 15));
  f32x4 acc[NA][NT];
  stream_gemm<F, NA, NT>(acc, ar, x, nchunks, lds);
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    const int ho = h0 + 16 * NA * wave + 16 * t + 4 * (lane >> 4);
    float sd[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sd[r] = out_scale<F>(md, ho + r);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int j = n * 16 + (lane & 15);
      if (j < rows) {
        const float4 d = make_float4(acc[t][n][0] * sd[0], acc[t][n][1] * sd[1],
                                     acc[t][n][2] * sd[2], acc[t][n][3] * sd[3]);
        if (!a.atomic) {
          float* dst = shared ? a.d_shared : a.d_perm;
          *reinterpret_cast<float4*>(dst + (int64_t)(row0 + j) * a.H + ho) = d;
        } else {
          int tok = row0 + j;
          float w = a.shared_gate ? a.gamma[tok] : 1.0f;
          if (!shared) {
            tok = a.perm_tok[row0 + j];
            w = tok >= 0 ? a.wts[a.perm_slot[row0 + j]] : 0.f;
          }
          if (tok >= 0) {
            float* dst = a.acc + (int64_t)tok * a.H + ho;
            unsafeAtomicAdd(dst + 0, w * d.x);
            unsafeAtomicAdd(dst + 1, w * d.y);
            unsafeAtomicAdd(dst + 2, w * d.z);
            unsafeAtomicAdd(dst + 3, w * d.w);
          }
        }
      }
    }
  }
}

template <int FR, int FS, int NTMAX>
__global__ __launch_bounds__(kGThreads) void k_g_down(GroupedArgs a) {
  extern __shared__ uint4 g_lds[];
  const int bid = blockIdx.x;
  constexpr int T = 16 * NTMAX;
  constexpr int DR = g_down_rows(NTMAX);
  const int tiles = a.H / DR;
  if (bid < a.dn_s) {
    if constexpr (FS != FMT_NONE) {
      const int tile = bid % tiles, tg = bid / tiles;
      const int t0 = tg * T;
      const int m = min(a.N - t0, T);
      const XRows x{a.a_shared + (int64_t)t0 * a.I_s, a.I_s, nullptr, m};
      const MatView md = gview(a.sdown, 0);
      with_tiles<NTMAX>((m + 15) >> 4, [&](auto nt) {
        down_pass<FS, decltype(nt)::value, DR / 64>(a, md, tile * DR, x, a.I_s / kGKC, m, true,
                                           t0, g_lds);
      });
    }
    return;
  }
  // one work item: T rows (a pass) of one unit
  const int b = bid - a.dn_s;
  const int i = b / a.dn_r, tile = b % a.dn_r;
  if (i >= a.info->nitems) return;
  const int item = a.info->item[i];
  const int u = item >> 16, p0 = (item & 0xffff) * T;
  const int e = a.info->uexp[u], cnt = a.info->ucount[u], rb = a.info->ubase[u];
  const MatView md = gview(a.down, e);
  const int m = min(cnt - p0, T);
  const XRows x{a.a_perm + (int64_t)(rb + p0) * a.I, a.I, nullptr, m};
  with_tiles<NTMAX>((m + 15) >> 4, [&](auto nt) {
    down_pass<FR, decltype(nt)::value, DR / 64>(a, md, tile * DR, x, a.I / kGKC, m, false,
                                       rb + p0, g_lds);
  });
}

// Bytes of dynamic LDS of the expert kernels: two chunk buffers of 16*NT
// token rows of 256 bytes.
inline size_t gemm_lds(int nt) { return (size_t)2 * 16 * nt * 256; }

hipError_t launch_one(const void* fn, int blocks, int threads, size_t lds, hipStream_t st,
                      const GroupedArgs& a, hipEvent_t* ev, int i);

// Gate+up and down launches (launches 2 and 3 of the call) for routed
// format FR; defined in one translation unit per format.
template <int FR>
hipError_t launch_experts(const GroupedArgs& a, int fs, hipStream_t st, hipEvent_t* ev);
template <>
hipError_t launch_experts<FMT_BF16>(const GroupedArgs&, int, hipStream_t, hipEvent_t*);
template <>
hipError_t launch_experts<FMT_FP8>(const GroupedArgs&, int, hipStream_t, hipEvent_t*);
template <>
hipError_t launch_experts<FMT_MXFP4>(const GroupedArgs&, int, hipStream_t, hipEvent_t*);
template <>
hipError_t launch_experts<FMT_NVFP4>(const GroupedArgs&, int, hipStream_t, hipEvent_t*);

template <int FR, int FS, int NT>
hipError_t launch_experts_t(const GroupedArgs& a, hipStream_t st, hipEvent_t* ev) {
  // (the gate+up kernels of two or more tiles take their items in groups of
  // eight: xcd_item)
  const int gu_items = NT >= 2 ? (a.max_items + 7) / 8 * 8 : a.max_items;
  hipError_t err = launch_one(reinterpret_cast<const void*>(&k_g_gate_up<FR, FS, NT>),
                              a.gu_s + gu_items * a.gu_r, kGThreads, gemm_lds(NT), st, a, ev, 2);
  if (err != hipSuccess) return err;
  return launch_one(reinterpret_cast<const void*>(&k_g_down<FR, FS, NT>),
                    a.dn_s + a.max_items * a.dn_r, kGThreads, gemm_lds(NT), st, a, ev, 3);
}

template <int FR, int FS>
hipError_t launch_experts_nt(const GroupedArgs& a, hipStream_t st, hipEvent_t* ev) {
  switch (a.nt) {
    case 1: return launch_experts_t<FR, FS, 1>(a, st, ev);
    case 2: return launch_experts_t<FR, FS, 2>(a, st, ev);
    case 4: return launch_experts_t<FR, FS, 4>(a, st, ev);
    case 8: return launch_experts_t<FR, FS, 8>(a, st, ev);
    default: return hipErrorInvalidValue;
  }
}

// Shared-expert format: none, BF16 or the routed format.
template <int FR>
hipError_t launch_experts_fs(const GroupedArgs& a, int fs, hipStream_t st, hipEvent_t* ev) {
  if (fs == FMT_NONE) return launch_experts_nt<FR, FMT_NONE>(a, st, ev);
  if (fs == FMT_BF16) return launch_experts_nt<FR, FMT_BF16>(a, st, ev);
  if constexpr (FR != FMT_BF16) {
    if (fs == FR) return launch_experts_nt<FR, FR>(a, st, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
