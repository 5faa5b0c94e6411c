// mok_dispatch_plan_noalloc: the dispatch plan with its scratch in a fixed device array, for
// callers that cannot allocate (code under graph capture, tight serving loops).
//
// The plan's scratch is one int32 table of plan_n_blocks(T_pool * k, E_l) x E_l entries (per
// chunk of routes, its histogram of local experts; at most 2^16 entries). Here it lives in
// `scratch`, a file-scope device array of kScratchInts int32 (256 KiB) that every GPU the
// library runs on holds until the process ends. The plan's first launch writes the whole table
// before its second reads it, so no call needs it cleared. Every call on one GPU shares that
// GPU's array: calls that overlap on one GPU (different streams, no order between them) race.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "mok.h"
#include "launch.h"

namespace {

constexpr int64_t kScratchInts = (int64_t)1 << 16;
constexpr int kMaxDevices = 64;

__device__ __align__(256) int32_t scratch[kScratchInts];

// The array's device address, per device. In host code `scratch` names a host-side stand-in:
// only the address hipGetSymbolAddress returns may reach a kernel or a copy.
int32_t* g_scratch[kMaxDevices] = {nullptr};
std::mutex g_mu;

int32_t* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = (int32_t*)p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int mok_dispatch_plan_noalloc(const int32_t* topk_idx, int64_t T_pool, int32_t k,
                                         int32_t E, int32_t e0, int32_t E_l,
                                         int32_t tokens_per_rank, int32_t* counts,
                                         int32_t* offsets, int32_t* rank_counts,
                                         int32_t* route_ids, void* stream) {
  if (T_pool < 0 || k < 1 || E < 1 || k > E || e0 < 0 || E_l < 1 || E_l > 1024 || e0 + E_l > E)
    return MOK_EINVAL;
  if (tokens_per_rank < 1 || T_pool % tokens_per_rank) return MOK_EINVAL;
  if (T_pool * (int64_t)k >= (int64_t)1 << 31) return MOK_EINVAL;
  if ((T_pool > 0 && !topk_idx) || !counts || !offsets || !rank_counts || !route_ids)
    return MOK_EINVAL;
  const int64_t nb = mok::plan_n_blocks(T_pool * k, E_l);
  const int64_t table = nb * E_l;                    // ints of the chunk histograms
  if (table > kScratchInts) return MOK_EWORKSPACE;   // larger than the fixed scratch
  int32_t* base = scratch_of_current_device();
  if (!base) return MOK_EHIP;
  const int64_t cap = std::max<int64_t>(1, T_pool * std::min(k, E_l));
  const hipError_t e = mok::launch_plan(topk_idx, T_pool, k, e0, E_l, tokens_per_rank, counts,
                                        offsets, rank_counts, route_ids, base, cap,
                                        (hipStream_t)stream);
  return e == hipSuccess ? MOK_OK : MOK_EHIP;
}
