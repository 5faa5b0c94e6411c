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
// Workgroup tile: 32 tokens x 64 experts, 256 threads as 16 x 16; thread (tt, te) owns tokens
// tt + 16a (a < 2) and experts te + 16b (b < 4): 8 independent chains. The d loop runs in
// chunks of 64 staged through two LDS buffers (float32); the next chunk's global loads are
// in flight while the current one is consumed 4 values of i at a time (float4 LDS reads).
// Every chain takes i strictly in ascending order, one FMA per step.
constexpr int RT_T = 32, RT_E = 64, RT_K = 64, RT_LD = RT_K + 4;

template <class T> struct Stage;
template <> struct Stage<bf16_t> {   // 8 bf16 per 16-byte load
  static constexpr int V = 8;
  typedef uint4 Raw;
  static MOK_DEV void cvt(const Raw& r, float* dst) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dst[2 * q] = __uint_as_float(w[q] << 16);
      dst[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  }
};
template <> struct Stage<float> {    // 4 floats per 16-byte load
  static constexpr int V = 4;
  typedef float4 Raw;
  static MOK_DEV void cvt(const Raw& r, float* dst) {
    dst[0] = r.x; dst[1] = r.y; dst[2] = r.z; dst[3] = r.w;
  }
};

// Global -> registers for rows [r0, r0 + ROWS) x cols [k0, k0 + 64) of a [n_rows, d] matrix;
// vector loads when the row chunk is whole and aligned, element loads otherwise (zero fill).
template <class T, int ROWS>
struct ChunkLoader {
  static constexpr int V = Stage<T>::V, PER_ROW = RT_K / V, N = ROWS * PER_ROW / 256;
  typename Stage<T>::Raw raw[N];
  float tail[N][Stage<T>::V];
  bool vec[N];
  MOK_DEV void load(const T* __restrict__ src, int64_t n_rows, int d, int64_t r0, int k0) {
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const int idx = threadIdx.x + 256 * q;
      const int r = idx / PER_ROW, c = (idx % PER_ROW) * V;
      const int64_t row = r0 + r;
      vec[q] = row < n_rows && k0 + c + V <= d && (d % V) == 0;
      if (vec[q]) {
        raw[q] = *(const typename Stage<T>::Raw*)(src + row * d + k0 + c);
      } else {
#pragma unroll
        for (int v = 0; v < V; ++v)
          tail[q][v] = (row < n_rows && k0 + c + v < d) ? load_as_f32<T>(src + row * d + k0 + c + v) : 0.0f;
      }
    }
  }
  MOK_DEV void store(float (*dst)[RT_LD]) const {
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const int idx = threadIdx.x + 256 * q;
      const int r = idx / PER_ROW, c = (idx % PER_ROW) * V;
      float v[V];
      if (vec[q]) Stage<T>::cvt(raw[q], v);
      else
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = tail[q][e];
#pragma unroll
      for (int e = 0; e < V; e += 4) *(float4*)&dst[r][c + e] = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
    }
  }
};

template <class T>
__global__ __launch_bounds__(256) void k_router_logits(const T* __restrict__ x,
                                                       const T* __restrict__ wr, int64_t n_tok,
                                                       int d, int E, float* __restrict__ logits) {
  __shared__ __align__(16) float xs[2][RT_T][RT_LD];
  __shared__ __align__(16) float ws[2][RT_E][RT_LD];
  const int tid = threadIdx.x;
  const int te = tid & 15, tt = tid >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * RT_T;
  const int e0 = blockIdx.y * RT_E;
  float acc[2][4] = {};
  ChunkLoader<T, RT_T> lx;
  ChunkLoader<T, RT_E> lw;
  lx.load(x, n_tok, d, t0, 0);
  lw.load(wr, E, d, e0, 0);
  lx.store(xs[0]);
  lw.store(ws[0]);
  __syncthreads();
  const int n_chunks = (d + RT_K - 1) / RT_K;
  for (int ck = 0; ck < n_chunks; ++ck) {
    const int cur = ck & 1;
    const int k0 = ck * RT_K;
    if (ck + 1 < n_chunks) {
      lx.load(x, n_tok, d, t0, k0 + RT_K);
      lw.load(wr, E, d, e0, k0 + RT_K);
    }
    const int kn = min(RT_K, d - k0);
    for (int i = 0; i < kn; i += 4) {
      float4 xa[2], wb[4];
#pragma unroll
      for (int a = 0; a < 2; ++a) xa[a] = *(const float4*)&xs[cur][tt + 16 * a][i];
#pragma unroll
      for (int b = 0; b < 4; ++b) wb[b] = *(const float4*)&ws[cur][te + 16 * b][i];
      if (i + 4 <= kn) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            float c = acc[a][b];
            c = __builtin_fmaf(xa[a].x, wb[b].x, c);
            c = __builtin_fmaf(xa[a].y, wb[b].y, c);
            c = __builtin_fmaf(xa[a].z, wb[b].z, c);
            c = __builtin_fmaf(xa[a].w, wb[b].w, c);
            acc[a][b] = c;
          }
      } else {  // d % 4 != 0: the last kn - i < 4 steps one at a time (no padding term enters)
        const float xv[2][4] = {{xa[0].x, xa[0].y, xa[0].z, xa[0].w}, {xa[1].x, xa[1].y, xa[1].z, xa[1].w}};
        const float wv[4][4] = {{wb[0].x, wb[0].y, wb[0].z, wb[0].w}, {wb[1].x, wb[1].y, wb[1].z, wb[1].w},
                                {wb[2].x, wb[2].y, wb[2].z, wb[2].w}, {wb[3].x, wb[3].y, wb[3].z, wb[3].w}};
        for (int q = 0; q < kn - i; ++q)
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(xv[a][q], wv[b][q], acc[a][b]);
      }
    }
    if (ck + 1 < n_chunks) {
      lx.store(xs[cur ^ 1]);
      lw.store(ws[cur ^ 1]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int64_t t = t0 + tt + 16 * a;
    if (t >= n_tok) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int e = e0 + te + 16 * b;
      if (e < E) logits[t * E + e] = acc[a][b];
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
