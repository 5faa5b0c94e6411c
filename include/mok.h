/*
 * mok.h -- C ABI of libmok: the forward pass of a DeepSeek-V3-style mixture-of-experts layer
 * (or one expert-parallel rank's share of it) on one AMD MI355X (gfx950).
 *
 * The layer, after the Mixture-of-Kittens (MoK) write-up, section "Overlapping compute and
 * communication in MoE": a router projection picks the top-k routed experts of each token
 * and gives each a router weight; each picked expert runs a SwiGLU feed-forward network
 * (gate and up projections, SwiGLU, down projection); the layer combines the shared
 * experts' and the routed experts' outputs with the router weights:
 *
 *   logits[t,e] = x[t] . W_r[e]
 *   idx[t,0..k) = the k largest logits (ties -> lower expert index), in descending order
 *   w[t,j]      = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0)   (softmax renormalised over
 *                 the picks)
 *   FFN_e(a)    = W_down[e] (silu(W_gate[e] a) * (W_up[e] a)),  silu(z) = z / (1 + e^-z)
 *   P[t*k+j]    = w[t,j] * FFN_{idx[t,j]}(x[t])                  (route slot, source-indexed)
 *   S[t]        = sum_s FFN_shared_s(x[t])
 *   y[t]        = S[t] + sum_{j=0..k-1, ascending} P[t*k+j]      (fixed order: bit-stable)
 *
 * One rank's share (same section: with expert parallelism each rank holds E/EP routed
 * experts plus the shared expert) computes P only at the routes of its local experts
 * [e0, e0+E_l) over a pool of T_pool tokens from R = T_pool / tokens_per_rank source ranks,
 * and S for its own T_own tokens; the sum over j then belongs to each token's source rank.
 *
 * The dispatch plan is the pull schedule of the write-up's "Scheduling" section: routes to
 * local experts, grouped by expert, each group in ascending (source rank, source index),
 * found by counting and a prefix sum rather than a sort, with counts per local expert, per
 * (local expert, source rank) and region offsets.
 *
 * Conventions (all entry points):
 *  - Pointers are DEVICE pointers unless stated otherwise; the caller owns every buffer.
 *    The library never allocates device memory and never frees caller memory.
 *  - Matrices are row-major and dense. Weights use the [out, in] layout: the reduction
 *    dimension is contiguous.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only enqueues work on
 *    it and returns; no call waits for the GPU, and the host never reads routing counts.
 *  - Return value: a mok_status. On any status other than MOK_OK nothing was enqueued
 *    (validation happens before the first launch) except MOK_EHIP, which reports a failed
 *    launch. Calls on different streams are independent if they use separate workspaces.
 *  - bf16 is stored as uint16 bit patterns (the upper half of a float32).
 */
#ifndef MOK_H_
#define MOK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOK_OK = 0,
  MOK_EINVAL = 1,        /* a pointer, size or shape is invalid                      */
  MOK_EUNSUPPORTED = 2,  /* valid request this build does not implement              */
  MOK_EWORKSPACE = 3,    /* workspace missing or smaller than the size query says    */
  MOK_EHIP = 4           /* a HIP runtime call or kernel launch failed               */
} mok_status;

typedef enum {
  MOK_FP32 = 0,   /* float32 inputs, weights and outputs                                    */
  MOK_BF16 = 1,   /* bf16 inputs, weights and outputs; float32 accumulation                 */
  MOK_MXFP8 = 2   /* bf16 inputs/weights/outputs in memory; the expert GEMMs run on OCP
                     MXFP8 operands (E4M3 elements, one E8M0 scale per 32 along K) that
                     the library quantises on the device on every call                      */
} mok_dtype;

/* Human-readable name of a status code (static string; never NULL). */
const char* mok_status_string(int status);

/* Library version, e.g. "mok 0.1.0 gfx950". Static string. */
const char* mok_version(void);

/* ---------------------------------------------------------------- stage 1: routing
 * Router projection + top-k + weights (formulas above).
 *   x        [T, d]  FP32 or BF16 (io_dtype), w_router [E, d] same type.
 *   logits   [T, E]  float32 output (also the scratch the top-k reads).
 *   topk_idx [T, k]  int32 output, topk_w [T, k] float32 output.
 * The logit of (t, e) is ONE float32 fused multiply-add chain over i = 0..d-1 in ascending
 * order starting from +0 (so routing indices are reproducible bit for bit). Requires
 * 1 <= k <= E <= 1024, d >= 1, T >= 0 (T == 0 enqueues nothing). */
int mok_route(const void* x, const void* w_router, int64_t T, int32_t d, int32_t E, int32_t k,
              int32_t io_dtype, float* logits, int32_t* topk_idx, float* topk_w, void* stream);

/* Top-k + weights on given float32 logits [T, E] (same rules as mok_route). */
int mok_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx,
             float* topk_w, void* stream);

/* ---------------------------------------------------------------- stage 2: dispatch plan
 * Pull schedule of the local experts [e0, e0+E_l) over routes r = t*k + j of a pool of
 * T_pool tokens (topk_idx [T_pool, k] int32, device):
 *   counts      [E_l]        routes per local expert
 *   offsets     [E_l + 1]    exclusive prefix sum of counts (region offsets)
 *   rank_counts [E_l * R]    routes per (local expert, source rank), R = T_pool / tokens_per_rank
 *   route_ids   [T_pool * min(k, E_l)] capacity; entries [offsets[e], offsets[e+1]) are the
 *               routes r of local expert e in ascending r (= ascending source rank, then
 *               source index). Entries at and beyond offsets[E_l] are left untouched.
 * Deterministic: integer counting, scans and a stable scatter; no order-dependent atomics.
 * Requires T_pool % tokens_per_rank == 0, 0 <= e0, 1 <= E_l, e0 + E_l <= E, 1 <= k <= E,
 * E_l <= 1024. topk_idx entries outside [0, E) are ignored (never local).
 * ws: device scratch of at least mok_dispatch_plan_workspace_bytes(...) bytes. */
int mok_dispatch_plan_workspace_bytes(int64_t T_pool, int32_t k, int32_t E_l, size_t* bytes);
int mok_dispatch_plan(const int32_t* topk_idx, int64_t T_pool, int32_t k, int32_t E, int32_t e0,
                      int32_t E_l, int32_t tokens_per_rank, int32_t* counts, int32_t* offsets,
                      int32_t* rank_counts, int32_t* route_ids, void* ws, size_t ws_bytes,
                      void* stream);

/* ---------------------------------------------------------------- stages 1-5: the layer */
typedef struct mok_moe_args {
  int32_t dtype;           /* mok_dtype                                                     */
  int32_t d;               /* model dim (multiple of 64; FP32: multiple of 32)              */
  int32_t E;               /* routed experts in the layer                                   */
  int32_t k;               /* top-k                                                         */
  int32_t I;               /* routed expert intermediate (multiple of 64)                   */
  int32_t e0, E_l;         /* local experts [e0, e0+E_l)                                    */
  int32_t tokens_per_rank; /* pool rows per source rank (T_pool % tokens_per_rank == 0)     */
  int64_t T_pool;          /* rows of the token pool x                                      */
  int64_t own_begin;       /* first pool row of this rank's own tokens                      */
  int32_t T_own;           /* own tokens (rows of the shared experts)                       */
  int32_t n_shared;        /* shared experts (0 allowed)                                    */
  int32_t I_shared;        /* shared expert intermediate (multiple of 64)                   */
  int32_t minibatch_rows;  /* rows per minibatch of the work loop: 128, 256, 512 or 1024    */
  int32_t ring_rows;       /* capacity of the macrobatch ring, multiple of minibatch_rows   */
  uint32_t flags;          /* MOK_FLAG_* below; 0 = defaults                                */
  /* inputs (device) */
  const void* x;           /* [T_pool, d] (FP32: float32, else bf16)                        */
  const void* w_router;    /* [E, d] same type as x; NULL when topk_idx_in is given         */
  const int32_t* topk_idx_in; /* optional [T_pool, k] routing (then topk_w_in is required)  */
  const float* topk_w_in;     /* optional [T_pool, k]                                       */
  const void* w_gate;      /* [E_l, I, d]                                                   */
  const void* w_up;        /* [E_l, I, d]                                                   */
  const void* w_down;      /* [E_l, d, I]                                                   */
  const void* ws_gate;     /* [n_shared, I_shared, d]  (NULL iff n_shared == 0)             */
  const void* ws_up;       /* [n_shared, I_shared, d]                                       */
  const void* ws_down;     /* [n_shared, d, I_shared]                                       */
  /* scratch */
  void* workspace;         /* device, >= mok_moe_workspace_bytes(args)                      */
  size_t workspace_bytes;
  /* outputs (device); FP32: float32, else bf16 */
  void* y_slots;           /* [T_pool * k, d]: row t*k+j = P[t*k+j] for local routes only;
                              other rows are not written                                    */
  void* y_shared;          /* [T_own, d] = S (NULL iff n_shared == 0)                       */
  void* y;                 /* [T_pool, d] combined output; required iff E_l == E (then
                              own_begin == 0 and T_own == T_pool), else must be NULL        */
  /* optional outputs (device, may be NULL): when given they are used as the forward's own
     storage for these intermediates, so the caller can inspect them afterwards */
  float* logits_out;       /* [T_pool, E]  (router runs only)                               */
  int32_t* topk_idx_out;   /* [T_pool, k]  (router runs only)                               */
  float* topk_w_out;       /* [T_pool, k]  (router runs only)                               */
  int32_t* counts_out;     /* [E_l]                                                         */
  int32_t* offsets_out;    /* [E_l + 1]                                                     */
  int32_t* rank_counts_out;/* [E_l * R]                                                     */
  int32_t* route_ids_out;  /* [T_pool * min(k, E_l)]                                        */
  /* optional measurement hook (host array, may be NULL): 2 * MOK_N_STAGES hipEvent_t created
     by the caller with timing enabled. Event 2s takes the time stage s's first kernel starts
     and event 2s+1 the time its last kernel ends: they are attached to those kernels' own
     dispatches (hipExtLaunchKernel), so no marker is queued between kernels. A stage that
     launches nothing records both as markers, back to back. NULL entries are skipped. With
     the ring work loop both GEMM stages run in one launch, timed as MOK_STAGE_UP. */
  void* const* stage_events;
} mok_moe_args;

/* stages of mok_moe_forward, for stage_events */
#define MOK_STAGE_ROUTE 0    /* router logits + top-k (router runs only)          */
#define MOK_STAGE_PLAN 1     /* dispatch plan                                      */
#define MOK_STAGE_QUANT 2    /* MXFP8 weight quantisation (MXFP8 only)             */
#define MOK_STAGE_UP 3       /* gate/up GEMM with SwiGLU (fused bf16/fp32 gather)  */
#define MOK_STAGE_DOWN 4     /* down GEMM with routing-weight scale                */
#define MOK_STAGE_COMBINE 5  /* fixed-order combine (full layer only)              */
#define MOK_STAGE_GATHER 6   /* device work list; MXFP8 stage order: + pull gather and
                                quantisation of the A rows (MOK_STAGE_UP is then the
                                gate/up GEMM launch alone)                         */
#define MOK_N_STAGES 7

/* flags */
#define MOK_FLAG_NO_RING 1u  /* stage-ordered launches over all routes (ring sized to every
                                possible route) instead of the persistent ring work loop;
                                same results                                                */

int mok_moe_workspace_bytes(const mok_moe_args* args, size_t* bytes);
int mok_moe_forward(const mok_moe_args* args, void* stream);

/* ---------------------------------------------------------------- MXFP8 quantiser
 * OCP MX v1.0 MXFP8 along rows: src [rows, K] bf16 (device), K % 32 == 0.
 *   codes  [rows, K]      E4M3 ("FN": bias 7, max 448, no infinities) bytes
 *   scales [rows, K / 32] E8M0 bytes (2^(byte-127))
 * Per block of 32: s = floor(log2(amax)) - 8 clamped to [-127, 127] (amax == 0 -> -127);
 * element = round-to-nearest-even(|v| * 2^-s) on the E4M3 grid, saturated to 448, sign kept.
 * The layer's MXFP8 path quantises its operands with this same device code. */
int mok_quantize_mxfp8(const void* src_bf16, int64_t rows, int32_t K, uint8_t* codes,
                       uint8_t* scales, void* stream);

/* ---------------------------------------------------------------- device error word
 * The persistent work loop bounds every wait; a wait that runs out sets a nonzero error word
 * in the workspace and the loop exits. This SYNCHRONOUS call waits for `stream`, then reads
 * the word (0 = no error) of a workspace last used by mok_moe_forward. Opt-in: the forward
 * itself never synchronises. */
int mok_get_device_error(const void* workspace, uint32_t* err, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOK_H_ */
