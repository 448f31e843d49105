// Device-side building blocks for the gfx950 MoE kernels: weight-chunk
// decoding into BF16 pairs, packed dot products, wave reductions.
//
// A "chunk" is 16 bytes of one weight row, fetched with one 128-bit load:
// 32 FP4 values, 16 FP8 values or 8 BF16 values. Each FP4 chunk is exactly one
// MXFP4 group (32 values, one E8M0 scale) or two NVFP4 groups (16 values each,
// one E4M3 scale each), so block scales are applied once per partial sum,
// never per element. Row or tensor scales are applied after the row
// reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum { FMT_BF16 = 0, FMT_FP8 = 1, FMT_MXFP4 = 2, FMT_NVFP4 = 3, FMT_NONE = 7 };

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int F> struct Fmt;
template <> struct Fmt<FMT_BF16> { static constexpr int VPC = 8; };
template <> struct Fmt<FMT_FP8> { static constexpr int VPC = 16; };
template <> struct Fmt<FMT_MXFP4> { static constexpr int VPC = 32; };
template <> struct Fmt<FMT_NVFP4> { static constexpr int VPC = 32; };
template <> struct Fmt<FMT_NONE> { static constexpr int VPC = 8; };

// One projection of one expert, already offset to that expert.
struct MatView {
  const uint8_t* data;    // row-major, row_bytes per row
  const uint8_t* scales;  // block scales (FP4), row scales (FP8, as float), or null
  int32_t row_bytes;
  int32_t scale_row_bytes;
  float tensor_scale;     // NVFP4 per-expert scale, 1 otherwise
};

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) {
  return __builtin_bit_cast(bf16x2, v);
}

__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// E8M0 byte -> 2^(b-127) as float (b = 0 is the subnormal 2^-127, 255 is NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  uint32_t bits = b ? (b << 23) : 0x00400000u;
  bits = (b == 255u) ? 0x7fc00000u : bits;
  return __builtin_bit_cast(float, bits);
}

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Partial dot products of one weight chunk with one token's matching 16..64
// bytes of BF16 activations (xv: VPC/2 packed BF16 pairs). Returns the
// chunk's contribution with the block scale applied; sc holds the chunk's
// scale byte(s) (low byte first).
template <int F>
__device__ __forceinline__ float chunk_dot(const uint4& wq, uint32_t sc, const uint32_t* xv);

template <>
__device__ __forceinline__ float chunk_dot<FMT_BF16>(const uint4& wq, uint32_t, const uint32_t* xv) {
  float p = 0.f;
  p = dot2(as_bf16x2(wq.x), as_bf16x2(xv[0]), p);
  p = dot2(as_bf16x2(wq.y), as_bf16x2(xv[1]), p);
  p = dot2(as_bf16x2(wq.z), as_bf16x2(xv[2]), p);
  p = dot2(as_bf16x2(wq.w), as_bf16x2(xv[3]), p);
  return p;
}

// FP8 E4M3 -> BF16 pairs is exact; the per-row scale is applied later.
template <>
__device__ __forceinline__ float chunk_dot<FMT_FP8>(const uint4& wq, uint32_t, const uint32_t* xv) {
  const uint32_t w[4] = {wq.x, wq.y, wq.z, wq.w};
  float p = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], 1.0f, false);
    bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], 1.0f, true);
    p = dot2(lo, as_bf16x2(xv[2 * q]), p);
    p = dot2(hi, as_bf16x2(xv[2 * q + 1]), p);
  }
  return p;
}

// Two E2M1 values per byte; E2M1 -> BF16 is exact. Byte b of word q holds
// columns 8q+2b (low nibble) and 8q+2b+1 (high nibble).
__device__ __forceinline__ float fp4_word_dot(uint32_t w, const uint32_t* xv, float p) {
  p = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0), as_bf16x2(xv[0]), p);
  p = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1), as_bf16x2(xv[1]), p);
  p = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2), as_bf16x2(xv[2]), p);
  p = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3), as_bf16x2(xv[3]), p);
  return p;
}

template <>
__device__ __forceinline__ float chunk_dot<FMT_MXFP4>(const uint4& wq, uint32_t sc, const uint32_t* xv) {
  float p = 0.f;
  p = fp4_word_dot(wq.x, xv + 0, p);
  p = fp4_word_dot(wq.y, xv + 4, p);
  p = fp4_word_dot(wq.z, xv + 8, p);
  p = fp4_word_dot(wq.w, xv + 12, p);
  return p * e8m0_to_f32(sc & 0xffu);
}

template <>
__device__ __forceinline__ float chunk_dot<FMT_NVFP4>(const uint4& wq, uint32_t sc, const uint32_t* xv) {
  float p0 = 0.f, p1 = 0.f;
  p0 = fp4_word_dot(wq.x, xv + 0, p0);
  p0 = fp4_word_dot(wq.y, xv + 4, p0);
  p1 = fp4_word_dot(wq.z, xv + 8, p1);
  p1 = fp4_word_dot(wq.w, xv + 12, p1);
  f32x2 s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc, 1.0f, false);
  return p0 * s.x + p1 * s.y;
}

// Scale bits of chunk c of a row (FP4 formats only).
template <int F>
__device__ __forceinline__ uint32_t load_chunk_scale(const uint8_t* srow, int c) {
  if constexpr (F == FMT_MXFP4) {
    return srow[c];
  } else if constexpr (F == FMT_NVFP4) {
    return *reinterpret_cast<const uint16_t*>(srow + 2 * c);
  } else {
    return 0u;
  }
}

// Per-row scale applied after the reduction.
template <int F>
__device__ __forceinline__ float row_scale(const MatView& m, int row) {
  if constexpr (F == FMT_FP8) {
    return reinterpret_cast<const float*>(m.scales)[row];
  } else if constexpr (F == FMT_NVFP4) {
    return m.tensor_scale;
  } else {
    return 1.0f;
  }
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// Workgroup barrier that orders LDS accesses only: it waits for this wave's
// LDS operations, not for its outstanding global stores (a __syncthreads
// waits for those too). For phases that exchange data through LDS while
// global results are still being written.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int m = width >> 1; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Float -> uint32 with the same order (larger float -> larger integer).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

}  // namespace moe
