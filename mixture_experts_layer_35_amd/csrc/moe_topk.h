// Wave-level reductions and the per-token top-k selection shared by the
// decode and grouped kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {

// DPP reductions over the 64 lanes of a wave (row shifts, then the row
// broadcasts 15 and 31); the full result is read from lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               ROW_MASK, 0xf, false));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<0x111, 0xf>(v);
  v += dpp_f32<0x112, 0xf>(v);
  v += dpp_f32<0x114, 0xf>(v);
  v += dpp_f32<0x118, 0xf>(v);
  v += dpp_f32<0x142, 0xa>(v);
  v += dpp_f32<0x143, 0xc>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sum over aligned groups of `width` lanes (8..64); the sum lands in the last
// lane of each group.
__device__ __forceinline__ float group_sum_last(float v, int width) {
  v += dpp_f32<0x111, 0xf>(v);
  v += dpp_f32<0x112, 0xf>(v);
  v += dpp_f32<0x114, 0xf>(v);
  if (width >= 16) v += dpp_f32<0x118, 0xf>(v);
  if (width >= 32) v += dpp_f32<0x142, 0xa>(v);
  if (width >= 64) v += dpp_f32<0x143, 0xc>(v);
  return v;
}

// max over finite-or--inf floats via their ordered integer images
__device__ __forceinline__ float wave_max_dpp(float v) {
  const uint32_t m = wave_max_u32(ordered_bits(v));
  const uint32_t b = (m & 0x80000000u) ? (m & 0x7fffffffu) : ~m;
  return __builtin_bit_cast(float, b);
}

// The correction bias of experts lane + 64 i (0 where there is none).
__device__ __forceinline__ void load_bias4(const float* bias, int E, int lane, float bv[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    bv[i] = (bias && e < E) ? bias[e] : 0.f;
  }
}

// Exact top-k of (score bits hi, expert) keys, one wave, k rounds: each lane
// sorts its four keys once (a five-exchange network); each round takes the
// wave maximum of the lanes' head scores, breaks a tie between heads by the
// lower expert, and pops the winner's head. Lane j < k returns the j-th
// expert. Used when the packed keys of topk_wave cannot decide.
__device__ __forceinline__ int topk_exact(const uint32_t hi_in[4], int E, int k, int lane) {
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    hi[i] = e < E ? hi_in[i] : 0u;
    lo[i] = e < E ? 0xffffffffu - (uint32_t)e : 0u;  // larger lo = lower expert
  }
  auto cx = [&](int x, int y) {
    const bool sw = hi[y] > hi[x] || (hi[y] == hi[x] && lo[y] > lo[x]);
    const uint32_t h0 = hi[x], l0 = lo[x];
    hi[x] = sw ? hi[y] : hi[x];
    lo[x] = sw ? lo[y] : lo[x];
    hi[y] = sw ? h0 : hi[y];
    lo[y] = sw ? l0 : lo[y];
  };
  cx(0, 1);
  cx(2, 3);
  cx(0, 2);
  cx(1, 3);
  cx(1, 2);
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t mh = wave_max_u32(hi[0]);
    const unsigned long long tied = __ballot(hi[0] == mh);
    int wl;
    uint32_t ml;
    if (__popcll(tied) == 1) {
      wl = __ffsll((long long)tied) - 1;
      ml = (uint32_t)__builtin_amdgcn_readlane((int)lo[0], wl);
    } else {
      ml = wave_max_u32(hi[0] == mh ? lo[0] : 0u);
      wl = __ffsll((long long)__ballot(hi[0] == mh && lo[0] == ml)) - 1;
    }
    if (lane == wl) {
      hi[0] = hi[1];
      lo[0] = lo[1];
      hi[1] = hi[2];
      lo[1] = lo[2];
      hi[2] = hi[3];
      lo[2] = lo[3];
      hi[3] = 0u;
      lo[3] = 0u;
    }
    if (lane == j) my_e = (int)(0xffffffffu - ml);
  }
  return my_e;
}

// e^x from the hardware base-2 exponential: t = x log2(e) rounded to FP32,
// 2^t, times 1 + (x log2(e) - t) ln 2 for the part the rounding of t lost (an
// FMA gives it exactly but for the tail of log2(e)), so the error is the
// hardware exponential's, a few ulp, at any |x|. And the logistic function
// with the hardware reciprocal. The routing needs no more: the selection
// margins of its inputs are orders of magnitude wider, and equal inputs still
// give equal outputs, so exact ties stay ties.
__device__ __forceinline__ float fast_exp(float x) {
  const float l2e_hi = 1.44269502162933350f;  // log2(e) to FP32
  const float l2e_lo = 1.92596299112661746e-08f;  // log2(e) - l2e_hi
  const float t = x * l2e_hi;
  const float lost = fmaf(x, l2e_hi, -t) + x * l2e_lo;
  return __builtin_amdgcn_exp2f(t) * fmaf(lost, 0.693147180559945f, 1.0f);
}
__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp(-x));
}

// Top-k routing of one token by one wave ("forward_k3.rs",
// MoeLayer::forward_k3, step 2; "forward_batched.rs", the routing step and
// its softmax+bias arm). The router logits sit four per lane: expert lane +
// 64 i in zv[i] (-inf past the router width E). Selection score: the logit
// (softmax, no bias), softmax(logit) + correction bias (softmax with a
// bias), or sigmoid(logit) + correction bias (sigmoid). Keys order by
// (score, -expert), so equal scores go to the lower expert index. bv holds
// the correction bias of the same four experts (read by the caller ahead of
// the logits; 0 without a bias).
//
// Selection packs each key into 32 bits: the score's top 24 ordered bits,
// then 255 - expert. These keys are distinct, so each of k + 1 rounds is one
// wave maximum, and the winner's lane (expert % 64) pops its head; the pops
// are selects, with no branch. The packed order equals the true order
// wherever two keys differ in their top 24 bits; if none of the k + 1
// largest packed keys shares its top 24 bits with the next one, the first k
// are exactly the true top k in order (any other key is below the (k+1)-th
// in its top bits). Otherwise the exact rounds of topk_exact decide.
//
// Weights: softmax over all E logits or the plain sigmoid of the chosen
// logits (no bias), optionally divided by their sum, then times the routed
// scaling factor. With renormalisation the softmax denominator cancels:
// w_j = exp(z_j - z_1) / sum over the chosen i of exp(z_i - z_1), z_1 the
// largest logit (the first choice), so the sum over all E is formed only to
// score with a bias or to weight without renormalisation. Lane j < k returns
// the j-th choice and its weight.
__device__ __forceinline__ void topk_wave(const float zv[4], const float bv[4], bool has_bias,
                                          int E, int k, int scoring, int renorm, float rsf,
                                          int lane, int& my_e, float& my_w) {
  const bool full_softmax = scoring == 0 && (has_bias || !renorm);
  float zmax = 0.f, rzsum = 1.f;
  if (full_softmax) {
    zmax = wave_max_dpp(fmaxf(fmaxf(zv[0], zv[1]), fmaxf(zv[2], zv[3])));
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < E) p += fast_exp(zv[i] - zmax);
    rzsum = __builtin_amdgcn_rcpf(wave_sum_dpp(p));
  }
  uint32_t hi[4], key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    const bool in = e < E;
    float sc = zv[i];
    if (scoring == 1)
      sc = fast_sigmoid(zv[i]) + bv[i];
    else if (has_bias)
      sc = fast_exp(zv[i] - zmax) * rzsum + bv[i];
    hi[i] = in ? ordered_bits(sc) : 0u;
    key[i] = in ? ((hi[i] & 0xffffff00u) | (255u - (uint32_t)e)) : 0u;
  }
  // the lane's four keys, largest first
  auto cx = [&](int x, int y) {
    const uint32_t a = key[x], b = key[y];
    key[x] = max(a, b);
    key[y] = min(a, b);
  };
  cx(0, 1);
  cx(2, 3);
  cx(0, 2);
  cx(1, 3);
  cx(1, 2);
  uint32_t mine = 0u;
  for (int j = 0; j <= k; ++j) {
    const uint32_t m = wave_max_u32(key[0]);
    const bool win = lane == ((int)(255u - (m & 255u)) & 63);  // the winner's lane
    key[0] = win ? key[1] : key[0];
    key[1] = win ? key[2] : key[1];
    key[2] = win ? key[3] : key[2];
    key[3] = win ? 0u : key[3];
    mine = lane == j ? m : mine;
  }
  const uint32_t next = (uint32_t)__shfl((int)mine, lane + 1 < 64 ? lane + 1 : lane, 64);
  const bool amb = lane < k && (mine >> 8) == (next >> 8);
  if (__ballot(amb) == 0ull)
    my_e = lane < k ? (int)(255u - (mine & 255u)) : 0;
  else
    my_e = topk_exact(hi, E, k, lane);
  // the chosen expert's logit: expert e sits in lane e % 64, register e / 64
  const int src = my_e & 63, reg = (my_e >> 6) & 3;
  const float z0 = __shfl(zv[0], src, 64), z1 = __shfl(zv[1], src, 64);
  const float z2 = __shfl(zv[2], src, 64), z3 = __shfl(zv[3], src, 64);
  const float my_z = reg == 0 ? z0 : (reg == 1 ? z1 : (reg == 2 ? z2 : z3));
  float w = 0.f;
  if (scoring == 1) {
    w = fast_sigmoid(my_z);
  } else if (full_softmax) {
    w = fast_exp(my_z - zmax) * rzsum;
  } else {
    // renormalised softmax: relative to the first choice's logit, the largest
    const float z_first = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, my_z)));
    w = fast_exp(my_z - z_first);
  }
  w = lane < k ? w : 0.f;
  if (renorm) w = w * __builtin_amdgcn_rcpf(wave_sum_dpp(w));
  my_w = w * rsf;
}

// Hash routing of one token by one wave ("forward_batched.rs", the
// hash-routing branch): lane j < k takes expert row[j] of the token's table
// row; the weights are the unbiased softmax (over all E logits) or sigmoid of
// those experts' logits, then renormalisation and the routed scaling factor
// as in topk_wave. Returns false (on every lane) if the row has an expert
// outside [0, E) or the same expert twice; such a slot gets expert E (past
// every expert, so it adds nothing) and weight 0.
__device__ __forceinline__ bool hash_wave(const float zv[4], const int32_t* row, int E, int k,
                                          int scoring, int renorm, float rsf, int lane,
                                          int& my_e, float& my_w) {
  int e = lane < k ? row[lane] : 0;
  const bool in = e >= 0 && e < E;
  // a repeat of an earlier lane's expert: compare with each lane i < k
  bool dup = false;
  for (int i = 0; i < k; ++i) {
    const int ei = __shfl(e, i, 64);
    dup = dup || (i < lane && ei == e);
  }
  const bool bad = lane < k && (!in || dup);
  const bool ok = __ballot(bad) == 0ull;
  e = in ? e : 0;
  // the chosen logit: expert e sits at lane e % 64, register e / 64
  const int src = e & 63, reg = e >> 6;
  const float z0 = __shfl(zv[0], src, 64), z1 = __shfl(zv[1], src, 64);
  const float z2 = __shfl(zv[2], src, 64), z3 = __shfl(zv[3], src, 64);
  const float z = reg == 0 ? z0 : (reg == 1 ? z1 : (reg == 2 ? z2 : z3));
  float zmax = 0.f, zsum = 1.f;
  if (scoring == 0) {
    zmax = wave_max_dpp(fmaxf(fmaxf(zv[0], zv[1]), fmaxf(zv[2], zv[3])));
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < E) p += expf(zv[i] - zmax);
    zsum = wave_sum_dpp(p);
  }
  float w = 0.f;
  if (lane < k && !bad) w = (scoring == 0) ? expf(z - zmax) / zsum : 1.0f / (1.0f + expf(-z));
  if (renorm) {
    const float sum = wave_sum_dpp(w);
    w = sum > 0.f ? w / sum : 0.f;
  }
  my_w = w * rsf;
  my_e = bad ? E : e;
  return ok;
}

// Route one token with one wave: hash routing when a table is given (id is
// the token's id, read by the caller), else top-k selection. Returns false
// for an invalid hash input (id outside [0, vocab), or a bad table row); the
// token's slots then get expert E (past every expert) and weight 0.
__device__ __forceinline__ bool route_token(const float zv[4], const float bv[4], bool has_bias,
                                            const int32_t* tid2eid, int vocab, int id, int E,
                                            int k, int scoring, int renorm, float rsf, int lane,
                                            int& my_e, float& my_w) {
  if (tid2eid) {
    if (id < 0 || id >= vocab) {
      my_e = E;
      my_w = 0.f;
      return false;
    }
    return hash_wave(zv, tid2eid + (size_t)id * k, E, k, scoring, renorm, rsf, lane, my_e, my_w);
  }
  topk_wave(zv, bv, has_bias, E, k, scoring, renorm, rsf, lane, my_e, my_w);
  return true;
}

}  // namespace moe
