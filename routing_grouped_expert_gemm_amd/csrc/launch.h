// Internal launchers of libmok (host side). Not part of the C ABI.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mok {

// Kernel launch with optional timing events (either may be NULL): e0 takes the time the kernel
// starts and e1 the time it ends. hipExtLaunchKernel ties them to the kernel's own dispatch, so
// no marker packet is queued on the stream, which would leave it idle for a few microseconds.
// A stage of several kernels passes e0 to its first launch and e1 to its last.
template <class... KArgs, class... Args>
inline void launch_k(void (*k)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                     hipEvent_t e0, hipEvent_t e1, Args... args) {
  hipExtLaunchKernelGGL(k, grid, block, shmem, s, e0, e1, 0u, args...);
}
// The events of a launch that is skipped (nothing to do): recorded as markers instead.
inline void mark_empty(hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (e0) (void)hipEventRecord(e0, s);
  if (e1) (void)hipEventRecord(e1, s);
}

hipError_t launch_router_logits(const void* x, const void* wr, int64_t n_tok, int d, int E,
                                bool bf16, float* logits, hipStream_t s,
                                hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
hipError_t launch_topk(const float* logits, int64_t n_tok, int E, int k, int32_t* idx,
                       float* w, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// Router logits + top-k: for E of 16, 32 or 64 and d a multiple of 16 one fused launch
// (route_fused_blocks > 0: its workgroup count), otherwise the two launches above.
int64_t route_fused_blocks(int64_t n_tok, int d, int E, int k);
hipError_t launch_route(const void* x, const void* wr, int64_t n_tok, int d, int E, int k,
                        bool bf16, float* logits, int32_t* idx, float* w, hipStream_t s,
                        hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// The plan: chunk histograms (blk_counts: plan_n_blocks * E_l ints of workspace), then the
// stable scatter; with wb (the expert stages' work list to build) one more workgroup of the
// scatter launch builds it from the same sums.
struct WlBuild;
int64_t plan_chunk(int64_t n_routes, int E_l);
int64_t plan_n_blocks(int64_t n_routes, int E_l);
hipError_t launch_plan(const int32_t* idx, int64_t n_tok, int k, int e0, int E_l,
                       int64_t tokens_per_rank, int32_t* counts, int32_t* offsets,
                       int32_t* rank_counts, int32_t* route_ids, int32_t* blk_counts,
                       int64_t route_cap, hipStream_t s, hipEvent_t ev0 = nullptr,
                       hipEvent_t ev1 = nullptr, const WlBuild* wb = nullptr);

// MX scales of the operands the expert GEMMs read are stored K-step major: a matrix of R rows
// and K columns keeps the 4 scales of K step j (128 elements) of row r as the 4-byte word
// j * R + r, so one K step's scales of consecutive rows are contiguous. Byte offset of the
// scale of (row r, 32-element block b):
__host__ __device__ inline int64_t mx_kmajor_scale(int64_t r, int b, int64_t R) {
  return ((int64_t)(b >> 2) * R + r) * 4 + (b & 3);
}
// MX quantiser: MXFP8 (E4M3 codes [rows, K]) or, fp4, MXFP4 (E2M1 codes [rows, K/2], element
// 2i in the low nibble of byte i). scales_kmajor == 0: scales row-major [rows, K/32] (the
// mok_quantize_mx* layout); R > 0: the rows form rows / R matrices of R rows, each with
// K-step-major scales (mx_kmajor_scale).
hipError_t launch_quantize_mx(const void* src_bf16, int64_t rows, int K, uint8_t* codes,
                              uint8_t* scales, bool fp4, hipStream_t s, hipEvent_t e0 = nullptr,
                              hipEvent_t e1 = nullptr, int64_t scales_kmajor = 0);
// The same rules for float32 rows (row-major scales), with the H epilogue's encoders.
hipError_t launch_quantize_mx_f32(const float* src, int64_t rows, int K, uint8_t* codes,
                                  uint8_t* scales, bool fp4, hipStream_t s);

// Operand element type of the expert GEMMs.
enum class Elem : int { F32 = 0, BF16 = 1, FP8 = 2, FP4 = 3 };

// Everything the expert-GEMM stages of one forward need (device pointers unless noted).
struct ExpertPass {
  Elem elem;             // GEMM operand type
  bool out_f32;          // outputs (H for non-MX, P, S, y) in float32 (else bf16)
  int d, k, I, E_l;
  int e0;                // first local expert
  int I_sh;              // n_shared * I_shared (0: no shared expert)
  int I_seg;             // I_shared: K-segment length of the shared down projection
  int64_t own_begin;
  int T_own;
  int mb;                // minibatch rows
  int n_slots;           // ring slots (ring rows = n_slots * mb); >= 8: split by XCD
  int Hld;               // ring row length in elements: max(I, I_sh)
  int max_mb;            // capacity of the minibatch tables
  int cap_u, cap_d;      // capacity of the up / down tile tables
  int cap_r;             // capacity of the ring-order table (ring work loop), else 0
  bool ring;             // persistent ring work loop (else stage-ordered launches)
  bool loop;             // the stage order run by the persistent loop (k_ring) instead
  bool xcd_split;        // ring: one item queue per XCD (whole-chip launch of 256 CUs)
  int64_t route_cap;     // rows of route_ids: a plan with more local routes is rejected
  int bm, bn;            // GEMM tile (rows, B-tile rows)
  int grid;              // workgroups of the tile loops
  // inputs
  const void* x;         // [T_pool, d] float32 or bf16
  const int32_t* route_ids;
  const float* topk_w;   // [T_pool*k]
  const int32_t* counts;
  const int32_t* offsets;
  const void *wg, *wu, *wd;     // routed weights (float32 / bf16) -- or MX codes
  const void *sg, *su, *sd;     // shared weights
  // MX scales (FP8 only), K-step major per matrix: routed gate/up one matrix of I rows per
  // expert, down d rows per expert; shared gate/up one matrix of I_sh rows, down d rows per
  // shared expert
  const uint8_t *wg_sc, *wu_sc, *wd_sc, *sg_sc, *su_sc, *sd_sc;
  // ring
  void* H;               // [n_slots*mb, Hld] (float32/bf16) -- MX: codes
  uint8_t* H_sc;         // MX: K-step-major scales of the n_slots*mb ring rows of H
  uint8_t* A_codes;      // MX: gathered x rows [n_slots*mb, d]
  uint8_t* A_sc;         // MX: K-step-major scales of the n_slots*mb ring rows of A
  // work list
  int32_t* wl;           // work list (layout in worklist.h)
  // outputs
  void* y_slots;
  void* y_shared;
};

size_t worklist_ints(int max_mb, int cap_u, int cap_d, int cap_r);
// Tile-table capacities for max_mb minibatches of mb rows; cap_g: gather items of the ring loop
// (MXFP8 only, else 0).
void gemm_tile_caps(int max_mb, int mb, int I, int I_sh, int d, bool gather_items, int* cap_u,
                    int* cap_d, int* cap_g);
// ev: optional hipEvent_t[2 * 7] (mok stage events; NULL entries skipped): GATHER on the work
// list (and the MXFP8 gather), UP on the gate/up launch, DOWN on the down launch (ring loop: UP
// on the one persistent launch, DOWN recorded empty).
// The plan of a forward, with the work list of its expert stages (p) built in the same launch.
hipError_t launch_plan_worklist(const int32_t* idx, int64_t n_tok, int64_t tokens_per_rank,
                                int32_t* rank_counts, int32_t* blk_counts, const ExpertPass& p,
                                hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
// The expert stages (MX gather, gate/up, down) over the work list launch_plan_worklist built.
hipError_t launch_expert_stages(const ExpertPass& p, hipStream_t s, void* const* ev);
hipError_t launch_combine(const void* y_shared, const void* y_slots, void* y, int64_t n_tok,
                          int k, int d, bool f32, hipStream_t s, hipEvent_t e0 = nullptr,
                          hipEvent_t e1 = nullptr);

// Standalone dispatch (dispatch.hip): pull gather of the plan's rows, push baseline.
hipError_t launch_pull_gather(const void* x, int d, int es, int k, const int32_t* route_ids,
                              const int32_t* offsets, int E_l, int64_t cap_rows, void* buf,
                              hipStream_t s);
hipError_t launch_push_dispatch(const void* x, int d, int es, const int32_t* topk_idx,
                                int64_t T_pool, int k, int e0, int E_l, int64_t cap,
                                int32_t* fill, void* buf, int32_t* src, hipStream_t s);

}  // namespace mok
