// Stage 1: router projection and top-k with renormalised weights.
//
// The MoK write-up ("Overlapping compute and communication in MoE") has a router projection
// pick the top-k routed experts of each token and give each a router weight. The projection
// is a dense [T, d] x [d, E] product, but its result decides integers (the expert ids), so
// it is computed on the VALU as one float32 fused multiply-add chain per logit, over the
// model dim in ascending order: the result is reproducible bit for bit. At the layer's sizes
// it is ~0.2% of the layer's FLOPs.
#include "device_common.h"
#include "launch.h"

namespace mok {

// ----------------------------------------------------------------------------- logits
// Workgroup tile: 32 tokens x 64 experts, 256 threads as 16 x 16; each thread owns tokens
// {ty, ty+16} x experts {tx, tx+16, tx+32, tx+48}. The d loop is staged through LDS in
// chunks of 32 (converted to float32 once); every thread walks i strictly ascending.
constexpr int RT_T = 32, RT_E = 64, RT_K = 32;

template <class T>
__global__ __launch_bounds__(256) void k_router_logits(const T* __restrict__ x,
                                                       const T* __restrict__ wr, int64_t n_tok,
                                                       int d, int E, float* __restrict__ logits) {
  __shared__ float xs[RT_T][RT_K + 1];
  __shared__ float ws[RT_E][RT_K + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * RT_T;
  const int e0 = blockIdx.y * RT_E;
  float acc[2][4] = {};
  for (int k0 = 0; k0 < d; k0 += RT_K) {
    // x chunk: 32 x 32 elements, 4 per thread
    for (int q = tid; q < RT_T * RT_K; q += 256) {
      int r = q / RT_K, c = q % RT_K;
      int64_t t = t0 + r;
      xs[r][c] = (t < n_tok && k0 + c < d) ? load_as_f32<T>(x + t * d + k0 + c) : 0.0f;
    }
    for (int q = tid; q < RT_E * RT_K; q += 256) {
      int r = q / RT_K, c = q % RT_K;
      int e = e0 + r;
      ws[r][c] = (e < E && k0 + c < d) ? load_as_f32<T>(wr + (int64_t)e * d + k0 + c) : 0.0f;
    }
    __syncthreads();
    const int kn = min(RT_K, d - k0);
    for (int i = 0; i < kn; ++i) {
      const float xa = xs[ty][i], xb = xs[ty + 16][i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float w = ws[tx + 16 * q][i];
        acc[0][q] = __builtin_fmaf(xa, w, acc[0][q]);
        acc[1][q] = __builtin_fmaf(xb, w, acc[1][q]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    int64_t t = t0 + ty + 16 * a;
    if (t >= n_tok) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = e0 + tx + 16 * q;
      if (e < E) logits[t * E + e] = acc[a][q];
    }
  }
}

// ----------------------------------------------------------------------------- top-k
// One wave per token; lane l holds experts l, l+64, ... Each of the k rounds takes the wave
// maximum of a 64-bit key (order-preserving bits of the logit, then the complemented expert
// id, so equal logits go to the lower id; -0 is folded onto +0 first).
constexpr int TK_MAXQ = 16;  // E <= 1024

MOK_DEV uint32_t float_order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 == +0
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

MOK_DEV float float_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int64_t n_tok,
                                              int E, int k, int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n_tok) return;
  const int nq = (E + 63) >> 6;
  uint32_t key[TK_MAXQ];
#pragma unroll
  for (int q = 0; q < TK_MAXQ; ++q) {
    const int e = lane + 64 * q;
    key[q] = (q < nq && e < E) ? float_order_key(logits[t * E + e]) : 0u;
  }
  uint32_t taken = 0;  // bit q: expert lane+64q already picked (or absent)
#pragma unroll
  for (int q = 0; q < TK_MAXQ; ++q)
    if (!(q < nq && lane + 64 * q < E)) taken |= 1u << q;
  float val0 = 0.0f;
  double wsum = 0.0;
  float my_val = 0.0f;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int q = 0; q < TK_MAXQ; ++q) {
      if (taken & (1u << q)) continue;
      const uint64_t c = ((uint64_t)key[q] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * q));
      best = c > best ? c : best;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const uint64_t o = shfl_xor_u64(best, m);
      best = o > best ? o : best;
    }
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float v = float_from_order_key((uint32_t)(best >> 32));
    if ((e & 63) == lane) taken |= 1u << (e >> 6);
    if (j == 0) val0 = v;
    wsum += exp((double)v - (double)val0);
    if (lane == j) { my_val = v; my_idx = e; }
  }
  if (lane < k) {
    topk_idx[t * k + lane] = my_idx;
    topk_w[t * k + lane] = (float)(exp((double)my_val - (double)val0) / wsum);
  }
}

hipError_t launch_router_logits(const void* x, const void* wr, int64_t n_tok, int d, int E,
                                bool bf16, float* logits, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  dim3 grid((unsigned)((n_tok + RT_T - 1) / RT_T), (unsigned)((E + RT_E - 1) / RT_E));
  if (bf16)
    hipLaunchKernelGGL(k_router_logits<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)wr, n_tok, d, E, logits);
  else
    hipLaunchKernelGGL(k_router_logits<float>, grid, dim3(256), 0, s, (const float*)x,
                       (const float*)wr, n_tok, d, E, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t n_tok, int E, int k, int32_t* idx,
                       float* w, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk, dim3((unsigned)((n_tok + 3) / 4)), dim3(256), 0, s, logits, n_tok,
                     E, k, idx, w);
  return hipGetLastError();
}

}  // namespace mok
