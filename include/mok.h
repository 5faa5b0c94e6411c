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
  MOK_MXFP8 = 2,  /* bf16 inputs/weights/outputs in memory; the expert GEMMs run on OCP
                     MXFP8 operands (E4M3 elements, one E8M0 scale per 32 along K) that
                     the library quantises on the device on every call                      */
  MOK_MXFP4 = 3   /* as MOK_MXFP8 with OCP MXFP4 operands (E2M1 elements: 0, 0.5, 1, 1.5,
                     2, 3, 4, 6 and sign; one E8M0 scale per 32 along K)                    */
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
 * E_l <= 1024. topk_idx entries outside [0, E) are ignored (never local). A token's k ids are
 * expected to be distinct, as top-k output is; if a token names a local expert twice, counts
 * and offsets still count every route, route_ids keeps only the entries below its capacity
 * (nothing is written past it), and offsets[E_l] > T_pool * min(k, E_l) flags the case.
 * ws: device scratch of at least mok_dispatch_plan_workspace_bytes(...) bytes. */
int mok_dispatch_plan_workspace_bytes(int64_t T_pool, int32_t k, int32_t E_l, size_t* bytes);
int mok_dispatch_plan(const int32_t* topk_idx, int64_t T_pool, int32_t k, int32_t E, int32_t e0,
                      int32_t E_l, int32_t tokens_per_rank, int32_t* counts, int32_t* offsets,
                      int32_t* rank_counts, int32_t* route_ids, void* ws, size_t ws_bytes,
                      void* stream);

/* The same plan for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): same arguments and results
 * as mok_dispatch_plan without `ws`. Its scratch is a fixed 256 KiB device array inside the
 * library (one per GPU, kept until the process ends) that holds the plan's per-chunk expert
 * histograms: chunks x E_l int32, at most 2^16 for any valid arguments (the plan cuts the
 * routes into at most 256 chunks, with chunks^2 x E_l <= 2^23); a request needing more would
 * return MOK_EWORKSPACE before any launch. Calls no allocator. Every call on one GPU shares
 * that GPU's array, so calls that overlap on one GPU (unordered streams) race. */
int mok_dispatch_plan_noalloc(const int32_t* topk_idx, int64_t T_pool, int32_t k, int32_t E,
                              int32_t e0, int32_t E_l, int32_t tokens_per_rank, int32_t* counts,
                              int32_t* offsets, int32_t* rank_counts, int32_t* route_ids,
                              void* stream);

/* ---------------------------------------------------------------- stages 1-5: the layer */
typedef struct mok_moe_args {
  int32_t dtype;           /* mok_dtype                                                     */
  int32_t d;               /* model dim (multiple of 128)                                   */
  int32_t E;               /* routed experts in the layer                                   */
  int32_t k;               /* top-k                                                         */
  int32_t I;               /* routed expert intermediate (multiple of 64; MXFP8: of 128;
                              MXFP4: of 256; d likewise a multiple of 256 for MXFP4)         */
  int32_t e0, E_l;         /* local experts [e0, e0+E_l)                                    */
  int32_t tokens_per_rank; /* pool rows per source rank (T_pool % tokens_per_rank == 0)     */
  int64_t T_pool;          /* rows of the token pool x                                      */
  int64_t own_begin;       /* first pool row of this rank's own tokens                      */
  int32_t T_own;           /* own tokens (rows of the shared experts)                       */
  int32_t n_shared;        /* shared experts (0 allowed)                                    */
  int32_t I_shared;        /* shared expert intermediate (as I)                             */
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
  int32_t* route_ids_out;  /* [T_pool * min(k, E_l)]. If the given routing repeats a local
                              expert within a token so that the local routes exceed this,
                              the forward computes nothing past the plan and sets the device
                              error word (MOK_DEVERR_OVERFLOW)                              */
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
#define MOK_FLAG_STAGE_LOOP 2u /* the stage order (every minibatch in its own slot, as with
                                MOK_FLAG_NO_RING) run by one persistent launch: per-XCD
                                queues of gate/up tiles then down tiles, a down tile waiting
                                only for its own minibatch's gate/up tiles, so the two stages
                                overlap at their boundary; same results. Takes precedence
                                over MOK_FLAG_NO_RING.                                      */

int mok_moe_workspace_bytes(const mok_moe_args* args, size_t* bytes);
int mok_moe_forward(const mok_moe_args* args, void* stream);

/* ---------------------------------------------------------------- workspace regions
 * Where a forward keeps an intermediate inside its workspace, so that a caller can read it
 * back after the forward (parity checks, debugging). Pure host call: validates `args` like
 * mok_moe_workspace_bytes and returns, for region `region`, the byte offset into the
 * workspace, its size in bytes and `rows` (below). MOK_EINVAL if the region does not exist
 * for this configuration (e.g. an MXFP8 region of a BF16 forward).
 *
 * MXFP8 codes are E4M3 bytes, row-major [rows, K] like the bf16 source; MXFP4 codes are E2M1
 * nibbles, row-major [rows, K/2] bytes, element 2i in the low nibble of byte i. Scales are E8M0
 * bytes kept "K-step major": a source of `rows` rows splits into matrices of R rows (R is
 * returned in *rows); in matrix g the scale of (row r, 32-element block b) sits at byte
 *     g * R * (K / 32) + ((b / 4) * R + r) * 4 + (b % 4)
 * so the 4 scales of 128-element K step b/4 of consecutive rows are contiguous.
 *   region                  K      source rows          R
 *   MOK_REGION_WG/WU/WD_*   d/d/I  E_l*I, E_l*I, E_l*d  I, I, d      (routed gate, up, down)
 *   MOK_REGION_SG/SU/SD_*   d/d/Is n_s*Is (gate, up)    n_s*Is       (shared: the experts
 *                                  n_s*d (down)         d             concatenated along I)
 *   MOK_REGION_A_*          d      ring rows            ring rows    (gathered x rows)
 *   MOK_REGION_H_*          Hld    ring rows            ring rows    (hidden activations)
 * Ring rows = n_slots * minibatch_rows, Hld = max(I, n_shared * I_shared); with
 * MOK_FLAG_NO_RING every minibatch keeps its own slot (the m-th minibatch -- routed experts
 * ascending, each region cut into minibatch_rows pieces, then the own tokens -- uses ring
 * rows [m * minibatch_rows, ...)). MOK_REGION_H of a BF16 / FP32 forward holds H itself
 * ([ring rows, Hld] bf16 / float32). MOK_REGION_WORKLIST is the device work list (int32;
 * layout internal), whose word 4 is the device error word. */
#define MOK_REGION_WORKLIST 0
#define MOK_REGION_H 1
#define MOK_REGION_H_SCALES 2
#define MOK_REGION_A_CODES 3
#define MOK_REGION_A_SCALES 4
#define MOK_REGION_WG_CODES 5
#define MOK_REGION_WG_SCALES 6
#define MOK_REGION_WU_CODES 7
#define MOK_REGION_WU_SCALES 8
#define MOK_REGION_WD_CODES 9
#define MOK_REGION_WD_SCALES 10
#define MOK_REGION_SG_CODES 11
#define MOK_REGION_SG_SCALES 12
#define MOK_REGION_SU_CODES 13
#define MOK_REGION_SU_SCALES 14
#define MOK_REGION_SD_CODES 15
#define MOK_REGION_SD_SCALES 16
#define MOK_N_REGIONS 17
int mok_moe_workspace_region(const mok_moe_args* args, int32_t region, size_t* offset,
                             size_t* bytes, int64_t* rows);

/* ---------------------------------------------------------------- backward
 * Gradients of the layer (or share) of mok_moe_forward with the routing held fixed (the routing
 * itself -- router projection, top-k -- is not differentiated here: its weights' gradient
 * arrives through dtopk_w). The MoK write-up presents MoK as a training kernel (introduction);
 * the Telegram post reports its forward and backward speed-ups ("Method and experiments").
 * Through the same pull plan as the forward, per local route r = t*k + j of expert e with
 * a = x[t], g = Wg a, u = Wu a, h = silu(g) u, and slot gradient dP_r:
 *   dtopk_w[r]   = <dP_r, Wd h>                        (routing-weight gradient)
 *   dh = w_r Wd^T dP_r;  dg = dh u silu'(g);  du = dh silu(g)
 *   dx_slots[r]  = Wg^T dg + Wu^T du                   (source-indexed, like y_slots)
 *   dw_gate[e] += dg a^T,  dw_up[e] += du a^T,  dw_down[e] += w_r dP_r h^T
 * and the same, unweighted, for the shared experts on the own tokens (dx_shared sums them).
 * Whole layer (E_l == E): dP_r = dy[t] and the shared gradient is dy[own]; dx = dx_shared +
 * sum_{j ascending} dx_slots[t*k + j] (the forward's fixed-order combine). Share: dy_slots
 * [T_pool*k, d] (read at local routes) and dy_shared [T_own, d].
 * BF16 only (MOK_EUNSUPPORTED otherwise): bf16 inputs and dx, float32 weight gradients
 * (overwritten, not accumulated), float32 accumulation throughout. Deterministic: no atomics;
 * every sum has a fixed order. route_rows_cap bounds the routed rows the workspace holds
 * (0: the worst case T_pool * min(k, E_l)); a plan with more local routes computes nothing
 * past the plan and sets MOK_DEVERR_OVERFLOW (mok_moe_backward_error). */
typedef struct mok_moe_bwd_args {
  int32_t dtype;           /* MOK_BF16                                                      */
  int32_t d, E, k, I, e0, E_l, tokens_per_rank;   /* as mok_moe_args (d % 128, I % 64)     */
  int64_t T_pool, own_begin;
  int32_t T_own, n_shared, I_shared;              /* n_shared <= 64, I_shared % 64         */
  int64_t route_rows_cap;  /* 0 = worst case                                                */
  /* forward inputs (device) */
  const void* x;           /* [T_pool, d] bf16                                              */
  const int32_t* topk_idx; /* [T_pool, k] the forward's routing                             */
  const float* topk_w;     /* [T_pool, k]                                                   */
  const void *w_gate, *w_up, *w_down;     /* [E_l, I, d], [E_l, I, d], [E_l, d, I] bf16     */
  const void *ws_gate, *ws_up, *ws_down;  /* shared: [n_s, I_s, d], .., [n_s, d, I_s]       */
  /* upstream gradient (device, bf16): dy for a whole layer, else dy_slots and dy_shared */
  const void* dy;          /* [T_pool, d]                                                   */
  const void* dy_slots;    /* [T_pool * k, d]                                               */
  const void* dy_shared;   /* [T_own, d]                                                    */
  void* workspace;         /* device, >= mok_moe_backward_workspace_bytes                   */
  size_t workspace_bytes;
  /* outputs (device) */
  void* dx_slots;          /* [T_pool * k, d] bf16, written at local routes only            */
  void* dx_shared;         /* [T_own, d] bf16 (n_shared > 0 and T_own > 0)                  */
  void* dx;                /* [T_pool, d] bf16, whole layer only (else NULL)                */
  float* dtopk_w;          /* [T_pool, k], written at local routes only; may be NULL        */
  float *dw_gate, *dw_up, *dw_down;       /* float32, the weights' shapes                   */
  float *dws_gate, *dws_up, *dws_down;    /* float32 (n_shared > 0)                         */
} mok_moe_bwd_args;
int mok_moe_backward_workspace_bytes(const mok_moe_bwd_args* args, size_t* bytes);
int mok_moe_backward(const mok_moe_bwd_args* args, void* stream);
/* SYNCHRONOUS (opt-in): waits for `stream`, then reads the backward's device error word. */
int mok_moe_backward_error(const void* workspace, const mok_moe_bwd_args* args, uint32_t* err,
                           void* stream);

/* ---------------------------------------------------------------- pull vs push dispatch
 * Two ways to bring each local expert its token rows, measured side by side (the Telegram post
 * on MoK, "Method and experiments": pushing needs a contended slot counter per expert and
 * scattered writes; pulling lets each expert read its tokens in large contiguous pieces; the
 * MoK write-up, "Choosing the right communication direction", pulls for dispatch). The layer
 * itself pulls inside its gate/up GEMM; these entry points copy the rows on their own.
 *
 * mok_pull_gather: buf row i = x[route_ids[i] / k] for i < offsets[E_l], the plan of
 *   mok_dispatch_plan (route_ids, offsets: device). x [T_pool, d] FP32 or BF16 (io_dtype);
 *   buf [T_pool * min(k, E_l), d] capacity, rows past offsets[E_l] untouched. Deterministic.
 * mok_push_dispatch: no plan. Every route r = t*k + j whose expert e = topk_idx[r] is local
 *   (e0 <= e < e0 + E_l) takes the next slot s of its expert with an atomic add on fill[e - e0]
 *   and writes buf[(e - e0) * capacity + s] = x[t] and src_route[(e - e0) * capacity + s] = r.
 *   fill [E_l] int32 is cleared by the call (no memset: a kernel) and ends as the number of
 *   local routes of each expert; slots >= capacity are not written (fill > capacity tells the
 *   caller routes were dropped). buf [E_l, capacity, d], src_route [E_l, capacity]. The set of
 *   rows per expert is determined; their order within an expert is not (it follows atomic
 *   arrival). Requires d * element size % 16 == 0. */
int mok_pull_gather(const void* x, int64_t T_pool, int32_t d, int32_t k, int32_t io_dtype,
                    const int32_t* route_ids, const int32_t* offsets, int32_t E_l, void* buf,
                    void* stream);
int mok_push_dispatch(const void* x, int64_t T_pool, int32_t d, int32_t k, int32_t io_dtype,
                      const int32_t* topk_idx, int32_t e0, int32_t E_l, int64_t capacity,
                      int32_t* fill, void* buf, int32_t* src_route, void* stream);

/* ---------------------------------------------------------------- MXFP8 quantiser
 * OCP MX v1.0 MXFP8 along rows: src [rows, K] bf16 (device), K % 32 == 0.
 *   codes  [rows, K]      E4M3 ("FN": bias 7, max 448, no infinities) bytes
 *   scales [rows, K / 32] E8M0 bytes (2^(byte-127))
 * Per block of 32: s = floor(log2(amax)) - 8 clamped to [-127, 127] (amax == 0 -> -127);
 * element = round-to-nearest-even(|v| * 2^-s) on the E4M3 grid, saturated to 448, sign kept.
 * The forward's own MXFP8 quantisers apply the same rules with other device code (K-step-
 * major scales, the row gather fused in); mok_moe_workspace_region exposes what they wrote. */
int mok_quantize_mxfp8(const void* src_bf16, int64_t rows, int32_t K, uint8_t* codes,
                       uint8_t* scales, void* stream);

/* OCP MX v1.0 MXFP4 along rows, the same conventions: codes [rows, K/2] bytes of E2M1 codes
 * (sign bit 3; element 2i in the low nibble of byte i), scales [rows, K/32] E8M0. Per block of
 * 32: s = floor(log2(amax)) - 2 clamped to [-127, 127] (amax == 0 -> -127); element = the
 * nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 to |v| * 2^-s (ties to the even code), saturated to 6,
 * sign kept. The forward's MXFP4 quantisers apply the same rules (K-step-major scales). */
int mok_quantize_mxfp4(const void* src_bf16, int64_t rows, int32_t K, uint8_t* codes,
                       uint8_t* scales, void* stream);

/* The same two quantisers for float32 rows (src [rows, K] float32, device; K % 32 == 0),
 * through the device code the gate/up epilogue uses to encode H from its float32 values: the
 * MX forward's H codes follow exactly these rules. Same outputs, layouts and errors. */
int mok_quantize_mxfp8_f32(const float* src, int64_t rows, int32_t K, uint8_t* codes,
                           uint8_t* scales, void* stream);
int mok_quantize_mxfp4_f32(const float* src, int64_t rows, int32_t K, uint8_t* codes,
                           uint8_t* scales, void* stream);

/* ---------------------------------------------------------------- device error word
 * The persistent work loop bounds every wait; a wait that runs out sets a nonzero error word
 * in the workspace and the loop exits. This SYNCHRONOUS call waits for `stream`, then reads
 * the word (0 = no error) of a workspace last used by mok_moe_forward. Opt-in: the forward
 * itself never synchronises. Bits: */
#define MOK_DEVERR_OVERFLOW 1u  /* the plan did not fit the work list / route_ids capacity
                                   (only possible with given routing that repeats an expert
                                   within a token): no expert tile ran                       */
#define MOK_DEVERR_WAIT 2u      /* a bounded wait of the ring work loop ran out              */
int mok_get_device_error(const void* workspace, uint32_t* err, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOK_H_ */
