// Internal interface between the host entry points (moe_api.cpp) and the
// kernel launchers (moe_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// One projection for all experts of a set, in the canonical layout.
struct DevProj {
  const uint8_t* data = nullptr;
  const uint8_t* scales = nullptr;
  const float* tensor_scale = nullptr;
  int64_t expert_bytes = 0;        // data bytes per expert
  int64_t scale_expert_bytes = 0;  // scale bytes per expert
  int32_t row_bytes = 0;
  int32_t scale_row_bytes = 0;
  int32_t rows = 0, cols = 0, fmt = 0;
};

// Per-call device pointers carved out of the workspace.
struct Workspace {
  float* logits = nullptr;      // [N, E]
  uint32_t* idx = nullptr;      // [N, k]
  float* wts = nullptr;         // [N, k]
  int32_t* num_units = nullptr; // [1]
  int32_t* unit_expert = nullptr;  // [maxu]
  int32_t* unit_slot = nullptr;    // [maxu, NMAX] slot t*k+j or -1
  float* unit_w = nullptr;         // [maxu, NMAX]
  uint16_t* a_routed = nullptr;    // [N*k, I] BF16
  uint16_t* a_shared = nullptr;    // [N, I_s] BF16
  float* dbuf = nullptr;           // [N*k + N, H] FP32 (slot mode)
  float* acc = nullptr;            // [N, H] FP32 (atomic mode)
  size_t total = 0;
};

constexpr int kNmax = 4;      // tokens per call on the decode path
constexpr int FMT_NONE_HOST = 7;  // no shared expert (same value as FMT_NONE)
constexpr int kThreads = 256; // threads per workgroup (4 waves)

struct StageGeom {
  int lpr = 64;          // lanes per row (power of two, 8..64)
  int rpl = 1;           // rows per lane group
  int rows_per_wg = 4;   // rows (gate/up: row pairs) per workgroup
  int tiles = 0;         // workgroups per unit
};

struct Call {
  int N = 0, H = 0, I = 0, E = 0, k = 0, I_s = 0;
  int scoring = 0, renorm = 1, atomic = 0;
  float rsf = 1.f;
  int maxu = 0;  // max distinct experts: min(E, N*k)
  const uint16_t* x = nullptr;
  uint16_t* out = nullptr;
  const uint16_t* router_w = nullptr;
  const float* router_bias = nullptr;
  DevProj gate, up, down;
  DevProj sgate, sup, sdown;  // fmt FMT_NONE (7) when absent
  StageGeom gu_r, gu_s, dn_r, dn_s;
  Workspace ws;
  uint32_t* out_idx = nullptr;
  float* out_w = nullptr;
  float* out_logits = nullptr;
};

// Lanes per row and rows per workgroup for a (format, cols, rows) stream.
StageGeom plan_stage(int fmt, int cols, int rows, int units, bool two_mats);

// Number of launches of the decode path.
int decode_num_launches();

// Enqueue the decode path. events (optional) are recorded before each launch
// and after the last. Returns hipSuccess or the first launch error.
hipError_t launch_decode(const Call& c, hipStream_t stream, hipEvent_t* events);

}  // namespace moe
