// Stage 2: the pull dispatch plan.
//
// Source: the MoK write-up, "Scheduling" section (the pull schedule is found by scanning the
// routing results, with no sort), and the Telegram post, "Method and experiments" (each
// expert fetches its own tokens; no contended slot counters).
//
// What is built for the local experts [e0, e0 + E_l): the number of routes each one receives,
// the number per (expert, source rank), the exclusive prefix sum of the per-expert numbers
// (region offsets), and route_ids: every local route id r = t*k + j, grouped by expert, in
// ascending r inside each group. Two launches keep it deterministic:
//   k_plan_count   -- per contiguous chunk of routes, a histogram of local experts;
//   k_plan_scatter -- every workgroup sums the chunk histograms itself (all of them: the
//                     per-expert counts and region offsets; those of the chunks before its
//                     own: its first free row in each region), then walks its routes in
//                     order and writes each local route at that row plus its rank among the
//                     chunk's earlier routes of that expert (wave ballots), i.e. a stable
//                     counting sort; the per-(expert, source rank) counts are integer sums
//                     added to totals that the first launch cleared. One more workgroup, when
//                     asked, builds the expert stages' work list from the same sums.
// Positions never come from an atomic, so the result does not depend on scheduling.
#include <algorithm>
#include <mutex>

#include "device_common.h"
#include "launch.h"
#include "worklist.h"

namespace mok {

constexpr int PLAN_THREADS = 1024;

// Also clears the per-(expert, source rank) counts, which the scatter accumulates.
__global__ __launch_bounds__(PLAN_THREADS) void k_plan_count(const int32_t* __restrict__ idx,
                                                             int64_t n_routes, int64_t chunk,
                                                             int e0, int E_l,
                                                             int32_t* __restrict__ blk_counts,
                                                             int32_t* __restrict__ rank_counts,
                                                             int64_t n_rank_counts) {
  extern __shared__ int32_t hist[];  // [E_l]
  if (rank_counts)
    for (int64_t q = (int64_t)blockIdx.x * PLAN_THREADS + threadIdx.x; q < n_rank_counts;
         q += (int64_t)gridDim.x * PLAN_THREADS)
      rank_counts[q] = 0;
  for (int e = threadIdx.x; e < E_l; e += PLAN_THREADS) hist[e] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * chunk;
  const int64_t r1 = min(n_routes, r0 + chunk);
  for (int64_t r = r0 + threadIdx.x; r < r1; r += PLAN_THREADS) {
    const int le = idx[r] - e0;
    if (le >= 0 && le < E_l) atomicAdd(&hist[le], 1);  // integer count: order-independent
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E_l; e += PLAN_THREADS)
    blk_counts[(int64_t)blockIdx.x * E_l + e] = hist[e];
}

// LDS of the scatter: the per-expert sums (tot, pre, off), then either the scatter's tables
// (base, per-wave counts, per-(source rank, expert) counts) or the work-list builder's.
constexpr int PLAN_NR = 4;            // source ranks a chunk counts in LDS
MOK_HOSTDEV inline int plan_sums_ints(int E_l) { return (3 * E_l + 1 + 3) & ~3; }
MOK_HOSTDEV inline int plan_scatter_ints(int E_l) { return (PLAN_THREADS / 64 + 1 + PLAN_NR) * E_l; }

// Workgroups 0 .. nb - 1 scatter chunk b; workgroup nb (launched only with a work list to
// build) builds it. rank_counts (optional): each workgroup counts its routes per (local expert,
// source rank) in LDS -- the chunk's first PLAN_NR source ranks; routes of later ones, which
// only very small ranks produce, go straight to global memory -- and adds the counts to the
// cleared totals (integer additions: the totals do not depend on their order).
__global__ __launch_bounds__(PLAN_THREADS) void k_plan_scatter(
    const int32_t* __restrict__ idx, int64_t n_routes, int64_t chunk, int nb, int e0, int E_l,
    const int32_t* __restrict__ blk_counts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ route_ids,
    int32_t* __restrict__ rank_counts, int k, int64_t tokens_per_rank, int64_t R, int64_t cap,
    WlBuild wb, int rank_sums) {
  extern __shared__ int32_t sm[];
  int32_t* tot = sm;                  // [E_l] routes of each expert
  int32_t* pre = sm + E_l;            // [E_l] ... in the chunks before this one
  int32_t* off = sm + 2 * E_l;        // [E_l + 1] region offsets
  int32_t* un = sm + plan_sums_ints(E_l);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x;
  for (int e = tid; e < E_l; e += PLAN_THREADS) tot[e] = pre[e] = 0;
  __syncthreads();
  // G threads per expert sum every G-th chunk histogram, 8 loads in flight; integer sums, so
  // the totals do not depend on the order of the LDS additions
  {
    const int G = PLAN_THREADS / E_l;
    if (tid < G * E_l) {
      const int e = tid % E_l, g = tid / E_l;
      int32_t st = 0, sp = 0;
      for (int c0 = g; c0 < nb; c0 += 8 * G) {
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = c0 + u * G;
          v[u] = c < nb ? blk_counts[(int64_t)c * E_l + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          st += v[u];
          if (c0 + u * G < b) sp += v[u];
        }
      }
      atomicAdd(&tot[e], st);
      atomicAdd(&pre[e], sp);
    }
  }
  __syncthreads();
  {
    int32_t total;
    const int32_t ex = block_excl_scan_1024(tid < E_l ? tot[tid] : 0, un, &total);
    if (tid < E_l) off[tid] = ex;
    if (tid == 0) off[E_l] = total;
    if (b == 0) {
      if (tid < E_l) {
        counts[tid] = tot[tid];
        offsets[tid] = ex;
      }
      if (tid == 0) offsets[E_l] = total;
    }
  }
  __syncthreads();
  if (b == nb) {                      // the work-list workgroup
    build_worklist(wb, tot, off, un);
    return;
  }
  if (rank_counts && rank_sums) {
    // chunks never straddle a source rank: rank rho's counts are the sums of its nb / R
    // chunks' histograms, which workgroup rho writes (no atomics on the totals)
    if (b < R) {
      const int64_t cpr = nb / R, c0 = (int64_t)b * cpr;
      int32_t* rsum = un;
      for (int e = tid; e < E_l; e += PLAN_THREADS) rsum[e] = 0;
      __syncthreads();
      const int G = PLAN_THREADS / E_l;
      if (tid < G * E_l) {
        const int e = tid % E_l, g = tid / E_l;
        int32_t st = 0;
        for (int64_t c1 = g; c1 < cpr; c1 += 8 * G) {
          int32_t v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int64_t c = c1 + u * G;
            v[u] = c < cpr ? blk_counts[(c0 + c) * E_l + e] : 0;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) st += v[u];
        }
        atomicAdd(&rsum[e], st);      // integer: order-independent
      }
      __syncthreads();
      for (int e = tid; e < E_l; e += PLAN_THREADS) rank_counts[(int64_t)e * R + b] = rsum[e];
      __syncthreads();
    }
    rank_counts = nullptr;            // nothing left to count per route
  }
  int32_t* base = un;                 // [E_l] next free row of each region (this chunk)
  int32_t* wcnt = un + E_l;           // [16][E_l] per-wave counts of the current sub-chunk
  int32_t* rc = un + (1 + PLAN_THREADS / 64) * E_l;   // [PLAN_NR][E_l] per-(rank, expert)
  const int64_t r0 = (int64_t)b * chunk;
  const int64_t rho0 = (r0 / k) / tokens_per_rank;   // first source rank of the chunk
  for (int e = tid; e < E_l; e += PLAN_THREADS) {
    base[e] = off[e] + pre[e];
    for (int q = 0; q < PLAN_THREADS / 64; ++q) wcnt[q * E_l + e] = 0;
    for (int q = 0; q < PLAN_NR; ++q) rc[q * E_l + e] = 0;
  }
  __syncthreads();
  const int64_t r1 = min(n_routes, r0 + chunk);
  for (int64_t rs = r0; rs < r1; rs += PLAN_THREADS) {
    const int64_t r = rs + tid;
    int le = -1;
    if (r < r1) {
      le = idx[r] - e0;
      if (le < 0 || le >= E_l) le = -1;
    }
    if (rank_counts && le >= 0) {
      const int64_t rho = (r / k) / tokens_per_rank;
      if (rho - rho0 < PLAN_NR) atomicAdd(&rc[(rho - rho0) * E_l + le], 1);
      else atomicAdd(&rank_counts[(int64_t)le * R + rho], 1);
    }
    // stable rank among the lanes of this wave with the same expert
    int rank = 0;
    bool leader = false;
    int cnt = 0;
    uint64_t remaining = ballot(le >= 0);
    while (remaining) {
      const int lead = __ffsll((unsigned long long)remaining) - 1;
      const int key = __shfl(le, lead, kWave);
      const uint64_t m = ballot(le == key);
      if (le == key) rank = __popcll(m & lanemask_lt());
      if (lane == lead) { leader = true; cnt = __popcll(m); }
      remaining &= ~m;
    }
    if (leader) wcnt[w * E_l + le] = cnt;
    __syncthreads();
    if (le >= 0) {
      int32_t pos = base[le] + rank;
      for (int q = 0; q < w; ++q) pos += wcnt[q * E_l + le];
      // a token that names one expert twice can push a region past the capacity: such rows
      // are dropped (offsets[E_l] > cap tells the caller)
      if (pos < cap) route_ids[pos] = (int32_t)r;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&base[le], cnt);      // integer: order-independent
      wcnt[w * E_l + le] = 0;
    }
    __syncthreads();
  }
  if (rank_counts) {
    for (int i = tid; i < PLAN_NR * E_l; i += PLAN_THREADS) {
      const int64_t rho = rho0 + i / E_l;
      const int32_t c = rc[i];
      if (c != 0 && rho < R) atomicAdd(&rank_counts[(int64_t)(i % E_l) * R + rho], c);
    }
  }
}

// Chunks of whole multiples of PLAN_THREADS routes, at most nb_max of them: every scatter
// workgroup reads all nb * E_l chunk counts, so nb^2 E_l stays below 2^23.
int64_t plan_chunk(int64_t n_routes, int E_l) {
  int64_t nb_max = 256;
  while (nb_max > 1 && nb_max * nb_max * E_l > ((int64_t)1 << 23)) nb_max /= 2;
  const int64_t per = PLAN_THREADS * nb_max;
  return PLAN_THREADS * std::max<int64_t>(1, (n_routes + per - 1) / per);
}

int64_t plan_n_blocks(int64_t n_routes, int E_l) {
  const int64_t c = plan_chunk(n_routes, E_l);
  return n_routes == 0 ? 1 : (n_routes + c - 1) / c;
}

hipError_t launch_plan(const int32_t* idx, int64_t n_tok, int k, int e0, int E_l,
                       int64_t tokens_per_rank, int32_t* counts, int32_t* offsets,
                       int32_t* rank_counts, int32_t* route_ids, int32_t* blk_counts,
                       int64_t route_cap, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                       const WlBuild* wb) {
  const int64_t n_routes = n_tok * k;
  const int64_t chunk = plan_chunk(n_routes, E_l);
  const int64_t nb = plan_n_blocks(n_routes, E_l);
  const int64_t R = n_tok / tokens_per_rank;
  WlBuild none = {};
  const WlBuild& w = wb ? *wb : none;
  const bool build = w.wl != nullptr;
  const int un = std::max(plan_scatter_ints(E_l), build ? WL_LDS_INTS : 0);
  const size_t sh_scatter = sizeof(int32_t) * (size_t)(plan_sums_ints(E_l) + std::max(un, 160));
  // the scatter's LDS passes 64 KiB for large E_l or with the work-list workgroup
  static std::once_flag lds_once;
  std::call_once(lds_once, [] {
    (void)hipFuncSetAttribute((const void*)k_plan_scatter,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
  });
  launch_k(k_plan_count, dim3((unsigned)nb), dim3(PLAN_THREADS),
           (uint32_t)(sizeof(int32_t) * E_l), s, ev0, nullptr, idx, n_routes, chunk, e0, E_l,
           blk_counts, rank_counts, (int64_t)E_l * R);
  // whole chunks per source rank: the rank counts are sums of chunk histograms
  const bool rank_sums = chunk % k == 0 && tokens_per_rank % (chunk / k) == 0;
  launch_k(k_plan_scatter, dim3((unsigned)(nb + (build ? 1 : 0))), dim3(PLAN_THREADS),
           (uint32_t)sh_scatter, s, nullptr, ev1, idx, n_routes, chunk, (int)nb, e0, E_l,
           blk_counts, counts, offsets, route_ids, rank_counts, k, tokens_per_rank, R, route_cap,
           w, rank_sums ? 1 : 0);
  return hipGetLastError();
}

}  // namespace mok
