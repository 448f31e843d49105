/*
 * moe_mi355x.h - C ABI of the routed mixture-of-experts layer forward for
 * small token batches on AMD Instinct MI355X (gfx950).
 *
 * One call computes, for N tokens x[N,H] (BF16):
 *   z      = x * Wr^T                 router projection, width E + Z
 *   idx, w = top-k of z (softmax), of softmax(z)+bias (softmax with a
 *            correction bias) or of sigmoid(z)+bias (sigmoid); or, with a
 *            hash table, the table's k experts for the token's id; the
 *            weights are the unbiased softmax(z) or sigmoid(z) of the chosen
 *            experts, optional renormalisation, times the routed scaling
 *            factor. A chosen zero expert (index >= E) adds nothing.
 *   a      = silu(Wg[e] x) * (Wu[e] x)  per routed (token, expert) pair
 *   y[t]   = sum_j w[t,j] * Wd[idx[t,j]] a  +  g[t] * shared expert(x[t]),
 *            g[t] = sigmoid(x[t] . w_sg) with a shared-expert gate, else 1
 *   out    = BF16(y) (round to nearest even)
 *
 * The stages and their arguments follow the reference pages:
 *   "spark_model/layers/moe/forward_k3.rs", MoeLayer::forward_k3 (the five
 *     stages of the fused forward; step 2 for sigmoid+bias vs softmax routing,
 *     norm_topk_prob and routed_scaling_factor; the E8M0 guard for GS32 E8M0
 *     against GS16 E4M3 scales; scale2 per expert for NVFP4; the plain
 *     residual add of the shared expert when there is no shared-expert gate);
 *   "spark_model/layers/moe/forward_atomic_c4.rs",
 *     MoeLayer::forward_atomic_c4_decode (FP32 accumulation of the weighted
 *     down projections into an [N,H] buffer, then the BF16 cast; the scratch
 *     size check that refuses with a need/have message);
 *   "metrale_model_layers/layers/moe/forward_batched.rs",
 *     MoeLayer::forward_batched (one router GEMM with M = N; the grouped FP8
 *     decode in which every expert streams its weights once for all rows and
 *     the result equals the per-token loop's).
 *
 * Memory ownership: the caller owns every buffer (weights, x, out, top-k
 * outputs, workspace). The library never allocates, frees or synchronises
 * and never reads device memory on the host. Pointers marked "device" must be
 * device memory of the current HIP device; results are valid once the stream
 * reaches them, and every input must stay alive until then.
 *
 * Errors: every argument is validated on the host before anything is
 * enqueued; an invalid call returns a non-zero moe_status and enqueues
 * nothing. moe_last_error() then gives a thread-local message. There are no
 * silent fallbacks: a combination the library does not implement is refused
 * with MOE_ERR_UNSUPPORTED.
 *
 * Concurrency: calls are re-entrant. Two calls that share a workspace must be
 * ordered (same stream, or synchronised); the workspace carries per-call
 * state.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a null, misaligned, mis-sized or out-of-range argument */
  MOE_ERR_UNSUPPORTED = 2, /* a valid request this library does not implement */
  MOE_ERR_WORKSPACE = 3,   /* workspace too small ("need X bytes, have Y") */
  MOE_ERR_HIP = 4          /* a HIP launch or runtime error */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_scoring;

/* How routed down projections are summed.
 * SLOT: each output row tile sums its experts in a fixed order (bitwise
 *       deterministic run to run).
 * ATOMIC_F32: FP32 atomic adds of w * down into an [N,H] accumulator in the
 *       workspace, then a BF16 cast ("forward_atomic_c4.rs"); summation order
 *       varies run to run. */
typedef enum { MOE_ACCUM_SLOT = 0, MOE_ACCUM_ATOMIC_F32 = 1 } moe_accum;

/* Which kernel family runs the experts. DECODE streams each selected expert
 * once for all of its tokens with VALU dot products (N <= 4). GROUPED sorts
 * the (token, expert) pairs by expert and runs them as per-expert tiles on
 * MFMA (N <= MOE_MAX_TOKENS). AUTO picks DECODE for N <= 4. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_GROUPED = 2 } moe_path;

/* Weight element formats (all little-endian, row-major):
 *   BF16          data [count, rows, cols] BF16; no scales.
 *   FP8_ROWSCALE  data [count, rows, cols] OCP E4M3FN bytes;
 *                 scales [count, rows] FP32, one per output row.
 *   MXFP4         data [count, rows, cols/2] E2M1 pairs, even column in the
 *                 low nibble; scales [count, rows, cols/32] E8M0 bytes.
 *   NVFP4         data as MXFP4; scales [count, rows, cols/16] E4M3FN bytes;
 *                 tensor_scale [count] FP32 (one per expert).
 * W[e,r,c] = value(data) * block or row scale (* tensor_scale[e] for NVFP4).
 * Scale groups run along the reduction axis (columns). */
typedef enum {
  MOE_FMT_BF16 = 0,
  MOE_FMT_FP8_ROWSCALE = 1,
  MOE_FMT_MXFP4 = 2,
  MOE_FMT_NVFP4 = 3
} moe_format;

#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 16
#define MOE_MAX_DECODE_TOKENS 4
#define MOE_MAX_TOKENS 4096

typedef struct {
  int32_t hidden;               /* H: model width (columns of gate/up, rows of down) */
  int32_t inter;                /* I: routed expert intermediate size */
  int32_t num_experts;          /* E: 1..MOE_MAX_EXPERTS */
  int32_t top_k;                /* k: 1..min(E, MOE_MAX_TOPK) */
  int32_t shared_inter;         /* I_s: shared expert intermediate size, 0 = none */
  int32_t scoring;              /* moe_scoring */
  int32_t norm_topk_prob;       /* 1: divide the k weights by their sum */
  float routed_scaling_factor;  /* multiplies the routed weights (after renorm) */
  int32_t accum_mode;           /* moe_accum */
  int32_t path;                 /* moe_path */
  /* Z: zero experts, 0 = none. The router has E + Z rows (E + Z <=
   * MOE_MAX_EXPERTS) and routing runs over all of them; experts E..E+Z-1
   * have no weights and a slot that chooses one adds nothing to the output,
   * while its weight still counts in the renormalisation ("forward_batched.rs",
   * the router width num_experts + zero_expert_num, which is also the row
   * stride of the logits; "forward_k3.rs", the zero-expert guard). */
  int32_t zero_experts;
} moe_cfg;


typedef struct {
  int32_t format;            /* moe_format */
  const void* data;          /* device, 16-byte aligned */
  size_t data_bytes;         /* must equal the size implied by format/count/rows/cols */
  const void* scales;        /* device; NULL for BF16 */
  size_t scale_bytes;        /* must equal the size implied by the format */
  const float* tensor_scale; /* device FP32 [count] for NVFP4, else NULL */
  int32_t rows, cols, count;
} moe_weight;

/* gate and up: rows = I (I_s), cols = H; down: rows = H, cols = I (I_s).
 * All three projections of one set share one format. */
typedef struct {
  moe_weight gate, up, down;
} moe_experts;

typedef struct {
  /* device, BF16 [E + Z, H], 16-byte aligned; NULL when weight_q is given */
  const void* weight;
  /* device, FP32 [E + Z] correction bias, or NULL. It steers selection only:
   * sigmoid scoring selects on sigmoid(z) + bias, softmax scoring on
   * softmax(z) + bias ("forward_batched.rs", the softmax+bias arm
   * router_bias_one that serves zero-expert routers); the weights stay the
   * unbiased probabilities. Ignored with a hash table. */
  const float* bias;
  /* device, BF16 [H], 16-byte aligned, or NULL: the shared-expert gate. With
   * it, token t's shared-expert output is added with weight
   * sigmoid(x[t] . shared_gate); without it, with weight 1 ("forward_k3.rs",
   * the EP all-reduce block: the batched blend with a sigmoid gate, or a
   * plain residual add when the layer has no gate). Needs shared_inter > 0. */
  const void* shared_gate;
  /* Hash routing ("forward_batched.rs", the hash-routing branch: expert ids
   * from a token-id to expert table, weights from the logits), or NULL:
   * tid2eid is device int32 [vocab, k]; token t takes experts
   * tid2eid[token_ids[t] * k + j], j = 0..k-1, in that order, each in
   * [0, E + Z) and distinct. token_ids is device int32 [n_tokens], per call.
   * The weights are softmax(z) (over all E + Z logits) or sigmoid(z) at
   * those experts, then renormalisation and the routed scaling factor as
   * above. A token id outside [0, vocab), or a table row with an expert out
   * of range or twice, sets the sticky device error word (bit 16) and that
   * token's output is not valid. */
  const int32_t* tid2eid;
  int32_t vocab;
  const int32_t* token_ids;
  /* A quantised router in place of weight, or NULL: NVFP4 only (rows E + Z,
   * cols H, count 1, the layout of moe_weight), the router weights
   * dequantised in registers against BF16 activations, FP32 logits
   * ("forward_k3.rs" and "forward_atomic_c4.rs", the NVFP4 router GEMV and
   * GEMM taken when the layer has an NVFP4 gate; "forward_ep.rs", the same
   * for one token). The shared-expert gate stays BF16. */
  const moe_weight* weight_q;
} moe_router;

/* Optional per-call outputs (each pointer may be NULL, device memory). */
typedef struct {
  uint32_t* idx;  /* [N, k] selected experts, descending score, lowest index on ties */
  float* weights; /* [N, k] routing weights (after renorm and scaling) */
  float* logits;  /* [N, E + Z] router logits (FP32) */
} moe_topk_out;

/* Optional timing hook: when non-NULL, launch i of the call (0 <=
 * i < moe_num_launches) is made with hipExtLaunchKernel so that events[2i]
 * and events[2i+1] record that kernel's own start and end; count must be
 * >= 2 * moe_num_launches. The events must be created by the caller. */
typedef struct {
  void** events; /* hipEvent_t[count] */
  int32_t count;
} moe_trace;

/* Bytes of workspace moe_forward needs for cfg and up to max_tokens tokens:
 * the caller-owned scratch whose size every call checks before it enqueues
 * anything ("forward_atomic_c4.rs", MoeLayer::forward_atomic_c4_decode: the
 * scratch arena size check that refuses with a need/have message). The
 * workspace has three regions: a head of counters and the decode FP32
 * accumulator, the decode path's hand-off region (sized for
 * MOE_MAX_DECODE_TOKENS tokens whatever max_tokens is) and, for
 * max_tokens above MOE_MAX_DECODE_TOKENS, the grouped path's per-call
 * buffers. The regions never overlap, so calls of either path may share one
 * workspace in any order. Host only. Returns 0 if cfg is invalid or
 * max_tokens is outside 1..MOE_MAX_TOKENS (moe_last_error() says why). */
size_t moe_workspace_bytes(const moe_cfg* cfg, int32_t max_tokens);

/* Validates a call exactly as moe_forward does, without enqueueing anything.
 * Host only; never touches device memory. */
moe_status moe_validate(const moe_cfg* cfg, const moe_router* router,
                        const moe_experts* experts, const moe_experts* shared,
                        int32_t n_tokens, size_t workspace_bytes);

/* Number of kernel launches moe_forward makes for this call (for moe_trace):
 * 1 on the decode path (one fused kernel); 5 on the grouped path (router,
 * top-k with the grouping, gate+up, down, combine). Returns -1 if the call
 * is invalid. */
int32_t moe_num_launches(const moe_cfg* cfg, int32_t n_tokens);

/* Where a grouped-path call keeps the result of its grouping step
 * ("forward_batched.rs", MoeLayer::forward_batched: tokens grouped by expert
 * so that each expert is streamed once for all of its rows). Byte offsets
 * into the workspace, valid after the call has run on its stream and until
 * the next call that uses the workspace. All arrays are int32:
 *   info       [2 + 30 + 3 * 256]: U (distinct experts), M (rows in use),
 *              30 unused, then uexp[256], ubase[256], ucount[256]: unit u's
 *              expert (ascending), first row (a multiple of 16) and count;
 *   perm_tok   [rows]: token of each grouped row, -1 on padding rows;
 *   perm_slot  [rows]: slot t*k + j of each grouped row, -1 on padding;
 *   inv        [n_tokens * k]: grouped row of each slot.
 * Rows of one expert keep ascending slot order; each expert's rows are
 * padded to a multiple of 16. */
typedef struct {
  size_t info, perm_tok, perm_slot, inv;
  int32_t rows; /* capacity of perm_tok and perm_slot */
} moe_group_view;

/* Fills *view for a grouped-path call with this cfg and n_tokens. Returns
 * MOE_ERR_UNSUPPORTED if such a call would take the decode path. Host only. */
moe_status moe_group_layout(const moe_cfg* cfg, int32_t n_tokens, moe_group_view* view);

/* The layer forward. x: device BF16 [n_tokens, H]; out: device BF16
 * [n_tokens, H] (every element is written); shared: NULL iff
 * cfg->shared_inter == 0; topk, trace: optional. workspace: device, 256-byte
 * aligned, at least moe_workspace_bytes(cfg, n_tokens) bytes, zero-filled
 * before the first call that uses it. Its head holds the decode path's
 * per-call counters and FP32 accumulator, which every decode call returns to
 * zero and the grouped path leaves alone; the decode path's hand-off words
 * (each tagged with its call's number) sit in a region of their own that no
 * grouped call writes. So a workspace sized for max_tokens serves any later
 * call with the same cfg and n_tokens <= max_tokens, on either path, in any
 * order. Bytes 128..131 are a sticky device error word
 * (either path may set bits; the caller clears it): bits 0..3 a decode
 * workgroup's bounded wait for another expired, bit 16 an invalid hash-routing
 * input. Results of a call that set it are not valid. stream: hipStream_t
 * (NULL = default stream). */
moe_status moe_forward(const moe_cfg* cfg, const moe_router* router,
                       const moe_experts* experts, const moe_experts* shared,
                       const void* x, int32_t n_tokens, void* out,
                       const moe_topk_out* topk, void* workspace,
                       size_t workspace_bytes, void* stream,
                       const moe_trace* trace);

/* One expert-parallel share of the layer forward, with no collective: the
 * experts are split over G devices, device g holding experts
 * [expert_begin, expert_end), and the layer output is the sum of the G
 * partials plus the shared expert's term, added once ("forward_k3.rs", the
 * EP all-reduce block: each device sums its own experts' weighted down
 * projections, the results are all-reduced, and the shared expert is blended
 * in once afterwards; "forward_atomic_c4.rs", the finalize call that leaves
 * the shared term out on an EP device; "forward_ep.rs", the local expert
 * range [local_start, local_end) of an EP rank).
 *
 * Every token is routed over all E experts as in moe_forward (the router
 * weight is the full [E, H] one, and topk reports the full routing); only
 * the (token, expert) pairs whose expert lies in [expert_begin, expert_end)
 * are computed. local_experts holds those experts' weights only: count =
 * expert_end - expert_begin, local index e - expert_begin. shared: the
 * shared expert when this share is to add its term (weighted by the
 * shared-expert gate when router->shared_gate is set), or NULL to leave it
 * out (router->shared_gate is then ignored); at most one share of a layer
 * should carry it. partial: device FP32 [n_tokens, H], 16-byte aligned,
 * every element written (zero for a token none of whose experts is local).
 * cfg->accum_mode applies as for moe_forward (the slot-order sum skips the
 * slots of other shares' experts). The workspace and the other arguments are
 * as for moe_forward, and one workspace sized by moe_workspace_bytes serves
 * both entry points. Errors:
 * MOE_ERR_INVALID_ARG for an empty range or one outside [0, E), and for
 * local_experts whose count is not the range's size. */
moe_status moe_forward_ep_partial(const moe_cfg* cfg, const moe_router* router,
                                  const moe_experts* local_experts, int32_t expert_begin,
                                  int32_t expert_end, const moe_experts* shared,
                                  const void* x, int32_t n_tokens, float* partial,
                                  const moe_topk_out* topk, void* workspace,
                                  size_t workspace_bytes, void* stream,
                                  const moe_trace* trace);

/* moe_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Its scratch is a static device array
 * inside the library, 16 MiB per device, held from the library's first use
 * on a device until the process ends; the call itself allocates nothing and
 * frees nothing. Arguments, results, ownership and errors are those of
 * moe_forward, with these differences:
 *   - a call whose scratch need exceeds 16 MiB is refused with
 *     MOE_ERR_WORKSPACE before anything is enqueued (every decode-path call
 *     fits, at most 7 MiB; grouped-path calls fit up to a few dozen tokens,
 *     depending on the layer);
 *   - every call on one device shares that device's array, whatever its
 *     layer: calls that overlap on one device (different streams or threads
 *     without ordering) race and give wrong results, and must be ordered;
 *   - the first call on a device looks the array up and, unless its stream
 *     is being captured into a graph, enqueues a fill kernel that zeroes it
 *     ahead of the call (the loader has zeroed it already);
 *   - the sticky device error word lives in the static array, so device-side
 *     errors (an expired wait, an invalid hash-routing input) are not visible
 *     to the caller; use moe_forward to observe them.
 * stream: hipStream_t of the current device (NULL = default stream). */
moe_status moe_forward_no_alloc(const moe_cfg* cfg, const moe_router* router,
                                const moe_experts* experts, const moe_experts* shared,
                                const void* x, int32_t n_tokens, void* out,
                                const moe_topk_out* topk, void* stream,
                                const moe_trace* trace);

/* The name of a status code ("MOE_OK", "MOE_ERR_WORKSPACE", ...; unknown
 * codes give "MOE_ERR_UNKNOWN"). A refused call is refused by name rather
 * than served by a silent fallback, as the pages' forward functions do
 * ("forward_k3.rs", MoeLayer::forward_k3: the zero-expert guard and the E8M0
 * guard each bail with a named error). Static storage; never NULL. */
const char* moe_status_str(moe_status status);

/* The detail of the last refusal on the calling thread (the need/have
 * figures of a workspace refusal, the argument and the limit of an invalid
 * one; "forward_atomic_c4.rs", the scratch size check, and "forward_k3.rs",
 * the E8M0 guard, name what they refuse and why). Thread-local storage valid
 * until the thread's next call into the library; "" after a call that
 * succeeded. Never NULL. */
const char* moe_last_error(void);

/* MOE_ABI_VERSION of the built library, so that a caller can refuse a
 * library whose structs differ from its header instead of calling it with
 * mismatched arguments (the same refuse-by-name habit as moe_status_str). */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
