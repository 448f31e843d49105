// Internal interface between the host entry points (moe_api.cpp) and the
// kernel launcher (moe_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kNmax = 4;          // tokens per call on the decode path
constexpr int kThreads = 256;     // threads per workgroup (4 waves)
constexpr int FMT_NONE_HOST = 7;  // no shared expert (same value as FMT_NONE)
constexpr int FMT_BF16_HOST = 0;   // the values of moe_format / the device FMT_ codes
constexpr int FMT_NVFP4_HOST = 3;

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

// Per-call state at the start of the workspace. It starts zero-filled; the
// counters are zero again after every call, and the tagged words (logits,
// plan) carry the call's tag, so they never need clearing. Counters sit on
// their own 128-byte lines so pollers and atomics do not pile onto one line.
constexpr int kLineWords = 32;    // 128 bytes
constexpr int kDoneGroups = 64;   // workgroup i reports to done group i % 64
constexpr unsigned kErrHashInput = 1u << 16;  // sticky error bit: invalid hash-routing input
constexpr int kPlanStride = 16;   // 64-bit plan words per unit (one line)
struct Ctl {
  unsigned done;   // done groups finished
  unsigned pad0[kLineWords - 1];
  unsigned error;  // sticky: 1 plan wait, 2 activation wait, 4 logits wait, 8 blend wait expired
  unsigned pad1[kLineWords - 1];
  unsigned epoch;  // calls completed on this workspace; the call's tag is epoch + 1
  unsigned pad2[kLineWords - 1];
  unsigned group_done[kDoneGroups * kLineWords];  // per done group, one line each
  // router logits, tagged; token t, expert e at t * 256 + e
  unsigned long long zlog[kNmax * 256];
  // shared-expert gate logits x . w_sg, tagged, one per token
  unsigned long long glog[kNmax];
  // the plan: unit u, token t: words u * kPlanStride + 2t (info) and + 2t + 1
  // (routing weight), both tagged
  unsigned long long plan[256 * kPlanStride];
  // per routing slot t * k + j, tagged: 1 if the slot's expert is computed by
  // this call (not a zero expert, not another share's), else 0; the
  // slot-order blend skips the others
  unsigned long long slot_real[kNmax * 16];
};
// the error word is bytes 128..131
static_assert(sizeof(Ctl) == 384 + kDoneGroups * 128 + kNmax * 256 * 8 + kNmax * 8 +
                                 256 * kPlanStride * 8 + kNmax * 16 * 8,
              "Ctl layout");

// Plan info word (high half of the tagged word):
constexpr unsigned kPlanAbsent = 1u << 30;  // unit index >= number of distinct experts
constexpr unsigned kPlanPresent = 1u << 8;  // the token routes to this unit
// expert id in bits 16..23, top-k position j in bits 0..4

struct StageGeom {
  int lpr = 64;          // lanes per row (power of two, 8..64)
  int rpl = 1;           // rows per lane group
  int sub = 1;           // row blocks per workgroup (one activation staging)
  int rows_per_wg = 4;   // rows (gate/up: row pairs) per workgroup
  int tiles = 0;         // workgroups per unit
};

struct DecodeArgs {
  // inputs
  const uint16_t* x;
  const uint16_t* router_w;
  const float* router_bias;
  const uint16_t* shared_gate;  // [H] BF16 or null: shared output weighted by sigmoid(x . w_sg)
  DevProj router_q;             // the router as NVFP4 [EW, H] (router_fmt NVFP4), else unused
  int router_fmt;               // FMT_BF16 (router_w) or FMT_NVFP4 (router_q)
  DevProj gate, up, down, sgate, sup, sdown;
  int N, H, I, E, k, I_s, scoring, renorm, atomic, maxu;
  int EW;          // router width: E experts and the zero experts
  int e_lo, e_hi;  // experts computed: [e_lo, e_hi); weights hold these only
  // 1 when a slot's expert may not be computed by this call (zero experts,
  // an expert-parallel share, hash routing): the routing then publishes a
  // flag per slot, which the slot-order blend reads
  int slot_flags;
  const int32_t* tid2eid;    // hash routing table [vocab, k], or null
  const int32_t* token_ids;  // [N]
  int vocab;
  float rsf;
  // phases (workgroup id ranges, in this order): router, shared gate+up,
  // routed gate+up, shared down, routed down
  int nR, nGs, nGr, nDs, nDr;
  int r_wpr;  // waves per router row (1, 2 or 4)
  StageGeom gr, gs, dr, ds;
  int blend_rows;  // output rows per blend block
  unsigned spin_limit;
  // routed down workgroups wait this long (100 MHz realtime ticks) after
  // reading the plan before they request weights; zero unless the call's
  // whole grid is resident at once (set at launch)
  unsigned d_defer_ticks;
  // workspace
  Ctl* ctl;
  unsigned* blend_ctr;  // [ceil(H / blend_rows) * kLineWords]
  unsigned long long* a_routed;  // [N*k, I] tagged FP32 SiLU(gate)*up
  unsigned long long* a_shared;  // [N, I_s] tagged FP32
  unsigned long long* dbuf;      // slot mode [N*k + N, H] tagged FP32 w*down
  float* acc;                    // atomic mode [N, H], zero at rest
  // outputs
  uint16_t* out;
  float* out_f32;  // instead of out: an expert-parallel share's FP32 partial
  uint32_t* out_idx;
  float* out_w;
  float* out_logits;
};

// ---------------------------------------------------------------------------
// Grouped path (any N up to MOE_MAX_TOKENS): router GEMM, per-token top-k,
// grouping of the N*k slots by expert, gate+up and down as grouped BF16 MFMA
// GEMMs over the permuted rows, and a combine pass.
// ---------------------------------------------------------------------------
constexpr int kGKC = 128;         // K columns per staged activation chunk
constexpr int kGRowsPerWG = 128;  // weight rows per workgroup (4 waves x 2 tiles x 16)
// Output rows of a down workgroup: 64 (one tile per wave) for batches of up to
// 64 tokens, so that a grid just above one round of resident workgroups
// leaves a tail half as long; 128 above.
__host__ __device__ constexpr int g_down_rows(int nt) { return nt == 1 ? 64 : kGRowsPerWG; }
constexpr int kGLaunches = 5;     // router, top-k (+ grouping), gate+up, down, combine

// Result of the grouping step, read by the expert kernels.
// Upper bound on the grouped path's work items: maxu + ceil(N * k / (16 * nt))
// with nt = 1 up to 64 tokens and nt = 8 above (at most 256 + 64 and
// 256 + 512).
constexpr int kMaxItems = 1024;

struct GroupInfo {
  int U;         // distinct routed experts in the batch ("units")
  int M;         // rows of the permuted buffers in use (per-unit counts padded to 16)
  int pad[30];
  int uexp[256];    // expert of unit u (local index: expert - e_lo), ascending
  int ubase[256];   // first permuted row of unit u (a multiple of 16)
  int ucount[256];  // tokens routed to unit u
  // work items of the expert kernels: one per (unit, pass of 16 * nt of its
  // rows), unit in bits 16.., pass index in bits 0..15, units in order
  int nitems;
  int pad2[31];
  int item[kMaxItems];
};

struct GroupedArgs {
  const uint16_t* x;
  const uint16_t* router_w;
  const float* router_bias;
  const uint16_t* shared_gate;  // [H] BF16 or null: shared output weighted by sigmoid(x . w_sg)
  DevProj router_q;             // the router as NVFP4 [EW, H] (router_fmt NVFP4), else unused
  int router_fmt;               // FMT_BF16 (router_w) or FMT_NVFP4 (router_q)
  DevProj gate, up, down, sgate, sup, sdown;
  int N, H, I, E, k, I_s, scoring, renorm, atomic;
  int EW;  // router width: E experts and the zero experts
  int ER;  // router rows: EW, plus the shared gate's row
  const int32_t* tid2eid;    // hash routing table [vocab, k], or null
  const int32_t* token_ids;  // [N]
  int vocab;
  unsigned* err;  // the workspace's sticky error word
  int e_lo, EL;  // experts computed: e_lo .. e_lo + EL - 1; weights hold these only
  float rsf;
  int nt;      // 16-token MFMA tiles per pass (1, 2, 4 or 8)
  int W;       // token-mask words per expert, ceil(N / 32)
  int WP;      // token-mask row stride in words, W | 1 (odd)
  int maxu;    // min(E, N * k)
  int max_items;  // bound on the work items: maxu + ceil(N * k / (16 * nt))
  int ksplit;  // router: H split into ksplit ranges of kcps 128-column chunks
  int kcps;
  // grids
  int r_rb, r_tg;   // router row blocks, token groups
  int s_tg;         // token groups of the shared expert
  int gu_s, gu_r;   // gate+up: shared workgroups, workgroups per routed unit
  int dn_s, dn_r;   // down: same
  // workspace
  float* zpart;      // [N, ksplit, ER] partial router logits (row EW: the shared gate)
  float* gamma;      // [N] shared-expert weights sigmoid(x . w_sg) (with a gate)
  unsigned* ticket;  // top-k workgroups finished (zeroed by the router kernel)
  uint32_t* mask;    // [EL, W] bit t of word t/32: token t routes to expert e_lo + e
  int* idx;          // [N*k]
  float* wts;        // [N*k]
  GroupInfo* info;
  int* perm_tok;     // [Mcap] token of each permuted row, -1 on padding
  int* perm_slot;    // [Mcap] slot t*k+j of each permuted row, -1 on padding
  int* inv;          // [N*k] permuted row of each slot (-1: expert outside the range)
  uint16_t* a_perm;  // [Mcap, I] BF16 silu(g)*u
  uint16_t* a_shared;  // [N, I_s] BF16
  float* d_perm;     // slot mode [Mcap, H] FP32 down outputs
  float* d_shared;   // slot mode [N, H] FP32
  float* acc;        // atomic mode [N, H] FP32
  // outputs
  uint16_t* out;
  float* out_f32;  // instead of out: an expert-parallel share's FP32 partial
  uint32_t* out_idx;
  float* out_w;
  float* out_logits;
};

// Enqueue the grouped path. ev: null, or 2 events per launch (start, stop).
hipError_t launch_grouped(const GroupedArgs& a, int fr, int fs, hipStream_t stream,
                          hipEvent_t* ev);
// The token masks are kept with an odd row stride WP = W | 1 (words), in
// global memory and in LDS alike, so that threads walking the words of
// consecutive experts hit different LDS banks; the global buffer holds one
// word more than EL * WP, so it is copied in 8-byte words.
// LDS: counts [256] and bases [257]; one 16-bit prefix (the expert's tokens
// before it) per group of four mask words; the masks, plus four words of
// padding (a slot reads the first three words of its four-word group, which
// may end past its row). At the largest sizes (256 experts, 4096 tokens) this is 147 KB.
struct GroupLds {
  int pw;
  size_t pre_off, m_off, bytes;
};

constexpr __host__ __device__ GroupLds group_lds_layout(int E, int W) {
  GroupLds L{};
  L.pw = (W + 3) / 4;
  L.pre_off = (256 + 257) * 4;
  L.m_off = (L.pre_off + (size_t)E * L.pw * 2 + 15) / 16 * 16;
  L.bytes = L.m_off + ((size_t)(E * (W | 1) + 1) / 2 * 2 + 4) * 4;
  return L;
}

size_t grouped_group_lds(int E, int W);

int lanes_per_row(int fmt, int cols);
StageGeom stage_geom(int fmt, int cols, int rows, int rpl, int sub);
size_t decode_lds_bytes(int H, int I, int I_s);

// Enqueue the fused decode kernel (formats: routed fr, shared fs or FMT_NONE).
hipError_t launch_decode(const DecodeArgs& a, int fr, int fs, int rpl, size_t lds,
                         hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace moe
