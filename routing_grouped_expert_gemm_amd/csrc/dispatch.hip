// Standalone dispatch kernels: the pull gather and a push-dispatch baseline beside it.
//
// The Telegram post on MoK ("Method and experiments") contrasts two ways of bringing each
// expert its tokens. Push: every source writes its token into the expert's buffer, which needs
// a shared slot counter per expert (contended atomics) and scattered writes, and the slot a
// token lands in depends on timing. Pull: once the schedule lists each expert's tokens, the
// expert reads them itself in large contiguous pieces. The MoK write-up ("Choosing the right
// communication direction") picks pull for dispatch.
//
// Both kernels here move the same rows -- the token rows of every route to a local expert --
// into expert-contiguous buffers, so the two directions can be measured side by side on one
// GPU's HBM:
//   k_pull_gather:   destination row i of the plan reads pool row route_ids[i] / k. The plan
//                    fixes every position, so the result is deterministic.
//   k_push_dispatch: each wave reads 64 routes' expert ids, each lane with a local route
//                    claims the next slot of its expert with an atomic add, and the wave then
//                    copies those rows into their slots. Slot order varies from run to run.
// A row is copied 16 bytes a lane, 1 KB a wave instruction, several loads in flight per lane.
#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "mok.h"

namespace mok {

constexpr int DISPATCH_THREADS = 256;
constexpr int COPY_UNROLL = 4;

// Copy n16 16-byte chunks from src to dst with the whole wave, COPY_UNROLL loads in flight. The
// chunks are held as plain vector registers (a uint4 array filled under a condition was placed
// in scratch, and every load then waited for the one before).
MOK_DEV void wave_copy_row(const uint4* __restrict__ src_, uint4* __restrict__ dst_, int n16) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* src = (const u32x4*)src_;
  u32x4* dst = (u32x4*)dst_;
  const int lane = lane_id();
  for (int c0 = 0; c0 < n16; c0 += 64 * COPY_UNROLL) {
    u32x4 v[COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) {
      const int c = c0 + u * 64 + lane;
      v[u] = c < n16 ? src[c] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < n16) dst[c] = v[u];
    }
  }
}

// One wave per destination row (grid-stride); the row count offsets[E_l] is read on the device.
__global__ __launch_bounds__(DISPATCH_THREADS) void k_pull_gather(
    const uint4* __restrict__ x, const int32_t* __restrict__ route_ids,
    const int32_t* __restrict__ offsets, int E_l, int k, int n16, int64_t cap_rows,
    uint4* __restrict__ buf) {
  const int64_t n = min((int64_t)offsets[E_l], cap_rows);
  const int64_t waves = (int64_t)gridDim.x * (DISPATCH_THREADS / 64);
  for (int64_t i = (int64_t)blockIdx.x * (DISPATCH_THREADS / 64) + (threadIdx.x >> 6); i < n;
       i += waves) {
    const int64_t t = uniform(route_ids[i]) / k;
    wave_copy_row(x + t * n16, buf + i * n16, n16);
  }
}

__global__ void k_zero_i32(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Each wave takes 64 consecutive routes, one per lane. Lanes holding a local route claim a slot
// of their expert (atomic add on fill[e]); the wave then copies those rows one after another.
// Slots at or past cap are not written (the count in fill still grows: a caller sees drops).
__global__ __launch_bounds__(DISPATCH_THREADS) void k_push_dispatch(
    const uint4* __restrict__ x, const int32_t* __restrict__ topk_idx, int64_t n_routes, int k,
    int e0, int E_l, int n16, int64_t cap, int32_t* __restrict__ fill, uint4* __restrict__ buf,
    int32_t* __restrict__ src) {
  const int lane = lane_id();
  const int64_t waves = (int64_t)gridDim.x * (DISPATCH_THREADS / 64);
  for (int64_t w = (int64_t)blockIdx.x * (DISPATCH_THREADS / 64) + (threadIdx.x >> 6);
       w * 64 < n_routes; w += waves) {
    const int64_t r = w * 64 + lane;
    int le = -1;
    if (r < n_routes) {
      le = topk_idx[r] - e0;
      if (le < 0 || le >= E_l) le = -1;
    }
    int32_t slot = -1;
    if (le >= 0) {
      slot = atomicAdd(&fill[le], 1);     // the contended per-expert slot counter
      if (slot < cap) src[(int64_t)le * cap + slot] = (int32_t)r;
    }
    uint64_t pending = ballot(le >= 0 && slot < cap);
    while (pending) {
      const int l = __ffsll((unsigned long long)pending) - 1;
      pending &= pending - 1;
      const int e = __shfl(le, l, kWave), s = __shfl(slot, l, kWave);
      const int64_t t = (w * 64 + l) / k;
      wave_copy_row(x + t * n16, buf + ((int64_t)e * cap + s) * n16, n16);
    }
  }
}

static unsigned grid_for(int64_t waves_wanted) {
  const int64_t blocks = (waves_wanted + 3) / 4;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(blocks, 8192));
}

hipError_t launch_pull_gather(const void* x, int d, int es, int k, const int32_t* route_ids,
                              const int32_t* offsets, int E_l, int64_t cap_rows, void* buf,
                              hipStream_t s) {
  const int n16 = d * es / 16;
  launch_k(k_pull_gather, dim3(grid_for(cap_rows)), dim3(DISPATCH_THREADS), 0, s, nullptr,
           nullptr, (const uint4*)x, route_ids, offsets, E_l, k, n16, cap_rows, (uint4*)buf);
  return hipGetLastError();
}

hipError_t launch_push_dispatch(const void* x, int d, int es, const int32_t* topk_idx,
                                int64_t T_pool, int k, int e0, int E_l, int64_t cap,
                                int32_t* fill, void* buf, int32_t* src, hipStream_t s) {
  const int n16 = d * es / 16;
  launch_k(k_zero_i32, dim3(1), dim3(256), 0, s, nullptr, nullptr, fill, E_l);
  const int64_t n_routes = T_pool * k;
  if (n_routes > 0)
    launch_k(k_push_dispatch, dim3(grid_for((n_routes + 63) / 64)), dim3(DISPATCH_THREADS), 0, s,
             nullptr, nullptr, (const uint4*)x, topk_idx, n_routes, k, e0, E_l, n16, cap, fill,
             (uint4*)buf, src);
  return hipGetLastError();
}

}  // namespace mok

extern "C" {

int mok_pull_gather(const void* x, int64_t T_pool, int32_t d, int32_t k, int32_t io_dtype,
                    const int32_t* route_ids, const int32_t* offsets, int32_t E_l, void* buf,
                    void* stream) {
  if (T_pool < 0 || d < 1 || k < 1 || E_l < 1 || E_l > 1024) return MOK_EINVAL;
  if (io_dtype != MOK_FP32 && io_dtype != MOK_BF16) return MOK_EINVAL;
  const int es = io_dtype == MOK_FP32 ? 4 : 2;
  if ((d * es) % 16) return MOK_EINVAL;
  if (T_pool * (int64_t)k >= (int64_t)1 << 31) return MOK_EINVAL;
  if (T_pool == 0) return MOK_OK;
  if (!x || !route_ids || !offsets || !buf) return MOK_EINVAL;
  const int64_t cap_rows = T_pool * std::min(k, E_l);
  return mok::launch_pull_gather(x, d, es, k, route_ids, offsets, E_l, cap_rows, buf,
                                 (hipStream_t)stream) == hipSuccess ? MOK_OK : MOK_EHIP;
}

int mok_push_dispatch(const void* x, int64_t T_pool, int32_t d, int32_t k, int32_t io_dtype,
                      const int32_t* topk_idx, int32_t e0, int32_t E_l, int64_t capacity,
                      int32_t* fill, void* buf, int32_t* src_route, void* stream) {
  if (T_pool < 0 || d < 1 || k < 1 || e0 < 0 || E_l < 1 || E_l > 1024 || capacity < 1)
    return MOK_EINVAL;
  if (io_dtype != MOK_FP32 && io_dtype != MOK_BF16) return MOK_EINVAL;
  const int es = io_dtype == MOK_FP32 ? 4 : 2;
  if ((d * es) % 16) return MOK_EINVAL;
  if (T_pool * (int64_t)k >= (int64_t)1 << 31 || capacity >= (int64_t)1 << 31) return MOK_EINVAL;
  if (!fill || (T_pool > 0 && (!x || !topk_idx || !buf || !src_route))) return MOK_EINVAL;
  return mok::launch_push_dispatch(x, d, es, topk_idx, T_pool, k, e0, E_l, capacity, fill, buf,
                                   src_route, (hipStream_t)stream) == hipSuccess ? MOK_OK
                                                                                  : MOK_EHIP;
}

}  // extern "C"
