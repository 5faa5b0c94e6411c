// Stage 2: the pull dispatch plan.
//
// Source: the MoK write-up, "Scheduling" section (the pull schedule is found by scanning the
// routing results, with no sort), and the Telegram post, "Method and experiments" (each
// expert fetches its own tokens; no contended slot counters).
//
// What is built for the local experts [e0, e0 + E_l): the number of routes each one receives,
// the number per (expert, source rank), the exclusive prefix sum of the per-expert numbers
// (region offsets), and route_ids: every local route id r = t*k + j, grouped by expert, in
// ascending r inside each group. Three launches keep it deterministic:
//   k_plan_count   -- per contiguous chunk of routes, a histogram of local experts;
//   k_plan_scan    -- one workgroup turns the chunk histograms into region offsets and the
//                     first free row of every (chunk, expert) pair;
//   k_plan_scatter -- each chunk walks its routes again in order and writes each local route
//                     at its (chunk, expert) base plus its rank among the chunk's earlier
//                     routes of that expert (wave ballots), i.e. a stable counting sort; the
//                     per-(expert, source rank) counts are integer sums added to totals that
//                     the first launch cleared.
// Positions never come from an atomic, so the result does not depend on scheduling.
#include "device_common.h"
#include "launch.h"

namespace mok {

constexpr int PLAN_THREADS = 256;

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

// One workgroup of 1024 threads.
//   blk_base[b][e] = sum_{b' < b} blk_counts[b'][e]   (the expert's offset is added later)
//   counts[e] = sum_b blk_counts[b][e],  offsets = exclusive prefix sum of counts.
// Each expert's block range is split over a group of P consecutive threads (P = 1024 / E_l
// rounded down to a power of two): per-thread segment sums, one block scan (a group's prefix
// is the scan minus its first thread's), then the segment walk. Scans: wave shuffles plus one
// pass over the wave totals.
__global__ __launch_bounds__(1024) void k_plan_scan(const int32_t* __restrict__ blk_counts,
                                                    int n_blk, int E_l,
                                                    int32_t* __restrict__ blk_base,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int32_t sh[64];
  __shared__ int32_t gbase[1024];
  const int t = threadIdx.x;
  int P = 1;
  while (P * 2 * E_l <= 1024) P *= 2;
  const int experts_per_round = 1024 / P;
  const int g = t % P, seg = (n_blk + P - 1) / P;
  const int b0 = min(n_blk, g * seg), b1 = min(n_blk, b0 + seg);
  for (int e_base = 0; e_base < E_l; e_base += experts_per_round) {
    const int e = e_base + t / P;
    const bool active = e < E_l;
    int32_t local = 0;
    if (active) {
#pragma unroll 4
      for (int b = b0; b < b1; ++b) local += blk_counts[(int64_t)b * E_l + e];
    }
    int32_t tot;
    const int32_t excl = block_excl_scan_1024(local, sh, &tot);
    if (g == 0) gbase[t / P] = excl;
    __syncthreads();
    if (active) {
      int32_t run = excl - gbase[t / P];
#pragma unroll 4
      for (int b = b0; b < b1; ++b) {
        blk_base[(int64_t)b * E_l + e] = run;
        run += blk_counts[(int64_t)b * E_l + e];
      }
      if (g == P - 1) counts[e] = run;
    }
    __syncthreads();
  }
  __threadfence_block();
  // exclusive scan of the counts over experts (E_l <= 1024)
  const int32_t c = t < E_l ? counts[t] : 0;
  int32_t total;
  const int32_t ex = block_excl_scan_1024(c, sh, &total);
  if (t < E_l) {
    offsets[t] = ex;
    if (t == E_l - 1) offsets[E_l] = total;
  }
}

// rank_counts (optional): each workgroup counts its routes per (local expert, source rank) in
// LDS -- the chunk's first PLAN_NR source ranks; routes of later ones, which only very small
// ranks produce, go straight to global memory -- and adds the counts to the cleared totals
// (integer additions: the totals do not depend on their order).
constexpr int PLAN_NR = 4;
__global__ __launch_bounds__(PLAN_THREADS) void k_plan_scatter(const int32_t* __restrict__ idx,
                                                               int64_t n_routes, int64_t chunk,
                                                               int e0, int E_l,
                                                               const int32_t* __restrict__ blk_base,
                                                               const int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ route_ids,
                                                               int32_t* __restrict__ rank_counts,
                                                               int k, int64_t tokens_per_rank,
                                                               int64_t R, int64_t cap) {
  extern __shared__ int32_t sm[];
  int32_t* base = sm;                 // [E_l] next free row of each region (this chunk)
  int32_t* wcnt = sm + E_l;           // [4][E_l] per-wave counts of the current sub-chunk
  int32_t* rc = sm + 5 * E_l;         // [PLAN_NR][E_l] per-(source rank, expert) counts
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * chunk;
  const int64_t rho0 = (r0 / k) / tokens_per_rank;   // first source rank of the chunk
  for (int e = tid; e < E_l; e += PLAN_THREADS) {
    base[e] = offsets[e] + blk_base[(int64_t)blockIdx.x * E_l + e];
    for (int q = 0; q < 4; ++q) wcnt[q * E_l + e] = 0;
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

int64_t plan_chunk(int64_t n_routes) {
  // 512 routes (2 sub-chunks of 256) per workgroup, at most 4096 workgroups
  int64_t chunk = 512;
  while ((n_routes + chunk - 1) / chunk > 4096) chunk *= 2;
  return chunk;
}

int64_t plan_n_blocks(int64_t n_routes) {
  const int64_t c = plan_chunk(n_routes);
  return n_routes == 0 ? 1 : (n_routes + c - 1) / c;
}

hipError_t launch_plan(const int32_t* idx, int64_t n_tok, int k, int e0, int E_l,
                       int64_t tokens_per_rank, int32_t* counts, int32_t* offsets,
                       int32_t* rank_counts, int32_t* route_ids, int32_t* blk_counts,
                       int32_t* blk_base, int64_t route_cap, hipStream_t s, hipEvent_t ev0,
                       hipEvent_t ev1) {
  const int64_t n_routes = n_tok * k;
  const int64_t chunk = plan_chunk(n_routes);
  const int64_t nb = plan_n_blocks(n_routes);
  const size_t sh_count = sizeof(int32_t) * (size_t)E_l;
  const int64_t R = n_tok / tokens_per_rank;
  launch_k(k_plan_count, dim3((unsigned)nb), dim3(PLAN_THREADS), (uint32_t)sh_count, s, ev0,
           nullptr, idx, n_routes, chunk, e0, E_l, blk_counts, rank_counts, (int64_t)E_l * R);
  launch_k(k_plan_scan, dim3(1), dim3(1024), 0, s, nullptr, nullptr, blk_counts, (int)nb, E_l,
           blk_base, counts, offsets);
  launch_k(k_plan_scatter, dim3((unsigned)nb), dim3(PLAN_THREADS),
           (uint32_t)(sh_count * (5 + PLAN_NR)), s, nullptr, ev1, idx, n_routes, chunk, e0, E_l,
           blk_base, offsets, route_ids, rank_counts, k, tokens_per_rank, R, route_cap);
  return hipGetLastError();
}

}  // namespace mok
