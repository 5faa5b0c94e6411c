// Stage 1: router projection and top-k with renormalised weights.
//
// The MoK write-up ("Overlapping compute and communication in MoE") has a router projection
// pick the top-k routed experts of each token and give each a router weight. The projection
// is a dense [T, d] x [d, E] product, but its result decides integers (the expert ids), so
// it is computed on the VALU as one float32 fused multiply-add chain per logit, over the
// model dim in ascending order: the result is reproducible bit for bit. At the layer's sizes
// it is ~0.2% of the layer's FLOPs.
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace mok {

// ----------------------------------------------------------------------------- logits
// One wave: 64 tokens (one per lane) x 8 experts. A chunk is 16 values of i. Within each row
// of 16 lanes, lane L holds W_r[e0 + L/2][i0 + 8 (L%2) + q], q = 0..7, as float32 (one 16-byte
// load and 8 shifts), so the row holds the chunk's 8 x 16 weights once; the FMA of expert e at
// i0 + j takes its weight straight from register j%8 of lane 2e + j/8 of the row (DPP
// row_newbcast), so one VALU instruction is one step of one chain for 64 tokens. Each lane
// also loads its own token's 16 values of x. Chunks are loaded RT_NPRE ahead into a ring of
// registers (one wave per SIMD: nothing else hides the load latency). The 4 waves of a
// workgroup share their 64 tokens, so x rows are fetched once per workgroup. Every chain
// takes i strictly in ascending order from +0.
constexpr int RT_TOK = 64, RT_EXP = 8, RT_K = 16, RT_NPRE = 4;

// acc = fma(w of lane J of this 16-lane row, x, acc): the product is exact either way round.
template <int J>
MOK_DEV void fma_bcast(float& acc, float w, float x) {
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
               : "+v"(acc) : "v"(w), "v"(x), "i"(J));
}

// Raw (unconverted) loads of one chunk: 16 values of the lane's token row, and the lane's 8
// weights.
template <class T> struct RtRaw;
template <> struct RtRaw<bf16_t> {
  uint4 x[2];
  uint4 w;
  MOK_DEV void load(const bf16_t* xp, const bf16_t* wp) {
    x[0] = *(const uint4*)xp;
    x[1] = *(const uint4*)(xp + 8);
    w = *(const uint4*)wp;
  }
  MOK_DEV static float bf(uint32_t u, int hi) {
    return hi ? __uint_as_float(u & 0xFFFF0000u) : __uint_as_float(u << 16);
  }
  MOK_DEV float xv(int q) const {     // q compile-time after unrolling
    const uint4 v = x[q >> 3];
    const int d = (q >> 1) & 3;
    return bf(d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w, q & 1);
  }
  MOK_DEV float wv(int q) const {
    const int d = q >> 1;
    return bf(d == 0 ? w.x : d == 1 ? w.y : d == 2 ? w.z : w.w, q & 1);
  }
};
template <> struct RtRaw<float> {
  float4 x[4];
  float4 w[2];
  MOK_DEV void load(const float* xp, const float* wp) {
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = *(const float4*)(xp + 4 * q);
    w[0] = *(const float4*)wp;
    w[1] = *(const float4*)(wp + 4);
  }
  MOK_DEV static float pick(const float4 v, int q) {
    return (q & 3) == 0 ? v.x : (q & 3) == 1 ? v.y : (q & 3) == 2 ? v.z : v.w;
  }
  MOK_DEV float xv(int q) const { return pick(x[q >> 2], q); }
  MOK_DEV float wv(int q) const { return pick(w[q >> 2], q); }
};

template <int J, int... Es>
MOK_DEV void step_experts(float (&acc)[RT_EXP], const float (&wf)[8], float xj,
                          std::integer_sequence<int, Es...>) {
  (fma_bcast<2 * Es + J / 8>(acc[Es], wf[J % 8], xj), ...);
}

template <class T, int... J>
MOK_DEV void chunk_all(float (&acc)[RT_EXP], const RtRaw<T>& c, std::integer_sequence<int, J...>) {
  float wf[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) wf[q] = c.wv(q);
  (step_experts<J>(acc, wf, c.xv(J), std::make_integer_sequence<int, RT_EXP>{}), ...);
}

template <class T>
__global__ __launch_bounds__(256) void k_router_logits(const T* __restrict__ x,
                                                       const T* __restrict__ wr, int64_t n_tok,
                                                       int d, int E, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, j = lane & 15;
  const int n_eg = (E + RT_EXP - 1) / RT_EXP;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t tb = wave / n_eg;
  const int e0 = uniform((int)(wave % n_eg) * RT_EXP);
  if (tb * RT_TOK >= n_tok) return;
  const int64_t t = tb * RT_TOK + lane;
  const T* xr = x + min(t, n_tok - 1) * (int64_t)d;
  // this lane's weight row and offset within a chunk
  const T* wl = wr + (int64_t)min(e0 + j / 2, E - 1) * d + 8 * (j & 1);
  float acc[RT_EXP];
#pragma unroll
  for (int e = 0; e < RT_EXP; ++e) acc[e] = 0.0f;
  const int nc = (d % RT_K) == 0 ? d / RT_K : 0;   // whole 16-value chunks (aligned rows)
  if (nc > 0) {
    RtRaw<T> ring[RT_NPRE];
#pragma unroll
    for (int q = 0; q < RT_NPRE; ++q) {
      const int c = min(q, nc - 1);
      ring[q].load(xr + c * RT_K, wl + c * RT_K);
    }
    // ring slot c % NPRE holds chunk c; after computing it, chunk c + NPRE is loaded into it
    // (clamped to the last chunk past the end: a harmless reload). Unrolled by NPRE so every
    // slot index is static, and without branches inside, so the wait for a slot's loads
    // counts only the younger loads in flight; the scheduling barriers keep each load after
    // the FMAs that read its slot and ahead of the next chunk's FMAs. The last nc % NPRE
    // chunks sit in the first slots and are computed after the loop.
    const int nc_main = nc - nc % RT_NPRE;
    for (int c0 = 0; c0 < nc_main; c0 += RT_NPRE) {
#pragma unroll
      for (int q = 0; q < RT_NPRE; ++q) {
        chunk_all<T>(acc, ring[q], std::make_integer_sequence<int, RT_K>{});
        __builtin_amdgcn_sched_barrier(0);
        const int cn = min(c0 + q + RT_NPRE, nc - 1);
        ring[q].load(xr + cn * RT_K, wl + cn * RT_K);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int q = 0; q + 1 < RT_NPRE; ++q)
      if (nc_main + q < nc) chunk_all<T>(acc, ring[q], std::make_integer_sequence<int, RT_K>{});
  }
  const T* wrow[RT_EXP];
#pragma unroll
  for (int e = 0; e < RT_EXP; ++e) wrow[e] = wr + (int64_t)min(e0 + e, E - 1) * d;
  for (int i = nc * RT_K; i < d; ++i) {            // rows that are not whole 16-value chunks
    const float xi = load_as_f32<T>(xr + i);
#pragma unroll
    for (int e = 0; e < RT_EXP; ++e) acc[e] = __builtin_fmaf(xi, load_as_f32<T>(wrow[e] + i), acc[e]);
  }
  if (t < n_tok) {
#pragma unroll
    for (int e = 0; e < RT_EXP; ++e)
      if (e0 + e < E) logits[t * E + e0 + e] = acc[e];
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

// The k picks of one token from its keys (lane l holds experts l, l + 64, ...: NQ of them):
// each of the k rounds takes the wave maximum of a 64-bit key (order-preserving bits of the
// logit, then the complemented expert id, so equal logits go to the lower id). Lane j < k
// returns pick j (expert and logit) in *e_out / *v_out; every lane returns l_0 in *v0_out.
template <int NQ>
MOK_DEV void topk_picks(const uint32_t (&key)[NQ], int E, int k, int lane, int* e_out,
                        float* v_out, float* v0_out) {
  uint32_t taken = 0;  // bit q: expert lane+64q already picked (or absent)
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    if (!(lane + 64 * q < E)) taken |= 1u << q;
  float val0 = 0.0f;
  float my_val = 0.0f;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
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
    if (lane == j) { my_val = v; my_idx = e; }
  }
  *e_out = my_idx;
  *v_out = my_val;
  *v0_out = val0;
}

// The renormalised weights of the k picks: lane j < k computes exp(l_j - l_0) once; the sum
// runs over j ascending, in double. Returns lane j's weight (lanes >= k: unused).
MOK_DEV float topk_weight(float my_val, float val0, int k, int lane) {
  const double ej = lane < k ? exp((double)my_val - (double)val0) : 0.0;
  double wsum = 0.0;
  for (int j = 0; j < k; ++j) wsum += __shfl(ej, j, kWave);
  return (float)(ej / wsum);
}

// NQ = keys per lane: the smallest power of two with 64 NQ >= E (compile time, so that a
// 64-expert top-k does one compare per lane per round, not TK_MAXQ). One wave per token.
template <int NQ>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int64_t n_tok,
                                              int E, int k, int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n_tok) return;
  uint32_t key[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    key[q] = e < E ? float_order_key(logits[t * E + e]) : 0u;
  }
  int my_idx;
  float my_val, val0;
  topk_picks<NQ>(key, E, k, lane, &my_idx, &my_val, &val0);
  const float w = topk_weight(my_val, val0, k, lane);
  if (lane < k) {
    topk_idx[t * k + lane] = my_idx;
    topk_w[t * k + lane] = w;
  }
}

// ----------------------------------------------------------------- router + top-k fused
// For E = 2 NW EPL experts (16, 32 or 64; NW = 4 waves, one per SIMD) and d a multiple of 16:
// one workgroup takes 32 tokens and all E experts, so the top-k reads its logits from LDS in
// the same launch (no second launch, no logits round trip through memory). Lanes l and l + 32
// hold the same token (l & 31); the two halves of wave w take expert groups 2w and 2w + 1
// (EPL experts each). Each 16-lane DPP row holds its group's weights for a 16-value chunk of i
// (16 / EPL lanes per expert, EPL consecutive values each), so the FMA of expert q at i0 + j
// takes its weight from register j % EPL of lane q (16 / EPL) + j / EPL of the row. Every
// chain runs over i in ascending order from +0, as in k_router_logits. (Eight waves of four
// experts a lane, two per SIMD, took ~20 us longer on 8,192 tokens x 64 experts.)
constexpr int RF_TOK = 32, RF_K = 16, RF_NPRE = 4;

template <class T, int EPL> struct RfRaw;   // EPL = 2, 4 or 8
template <int EPL> struct RfRaw<bf16_t, EPL> {
  uint4 x[2];
  uint32_t w[(EPL + 1) / 2];
  MOK_DEV void load(const bf16_t* xp, const bf16_t* wp) {
    x[0] = *(const uint4*)xp;
    x[1] = *(const uint4*)(xp + 8);
    if constexpr (EPL == 8) {
      const uint4 v = *(const uint4*)wp;
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (EPL == 4) {
      const uint2 v = *(const uint2*)wp;
      w[0] = v.x;
      w[1] = v.y;
    } else {
      w[0] = *(const uint32_t*)wp;
    }
  }
  MOK_DEV float xv(int q) const { return RtRaw<bf16_t>::bf(pick4(x[q >> 3], (q >> 1) & 3), q & 1); }
  MOK_DEV float wv(int q) const { return RtRaw<bf16_t>::bf(w[q >> 1], q & 1); }
  MOK_DEV static uint32_t pick4(const uint4 v, int d) {
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
  }
};
template <int EPL> struct RfRaw<float, EPL> {
  float4 x[4];
  float w[EPL];
  MOK_DEV void load(const float* xp, const float* wp) {
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = *(const float4*)(xp + 4 * q);
    if constexpr (EPL == 8) {
      const float4 v = *(const float4*)wp, u = *(const float4*)(wp + 4);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      w[4] = u.x; w[5] = u.y; w[6] = u.z; w[7] = u.w;
    } else if constexpr (EPL == 4) {
      const float4 v = *(const float4*)wp;
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
      const float2 v = *(const float2*)wp;
      w[0] = v.x; w[1] = v.y;
    }
  }
  MOK_DEV float xv(int q) const { return RtRaw<float>::pick(x[q >> 2], q); }
  MOK_DEV float wv(int q) const { return w[q]; }
};

template <int EPL, int J, int... Qs>
MOK_DEV void rf_step(float (&acc)[EPL], const float (&wf)[EPL], float xj,
                     std::integer_sequence<int, Qs...>) {
  (fma_bcast<Qs * (16 / EPL) + J / EPL>(acc[Qs], wf[J % EPL], xj), ...);
}

template <class T, int EPL, int... J>
MOK_DEV void rf_chunk(float (&acc)[EPL], const RfRaw<T, EPL>& c, std::integer_sequence<int, J...>) {
  float wf[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) wf[q] = c.wv(q);
  (rf_step<EPL, J>(acc, wf, c.xv(J), std::make_integer_sequence<int, EPL>{}), ...);
}

template <class T, int EPL, int NW>
__global__ __launch_bounds__(64 * NW) void k_route(
    const T* __restrict__ x, const T* __restrict__ wr, int64_t n_tok, int d, int k,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int E = 2 * NW * EPL, LPE = 16 / EPL, LDW = E + 1;
  __shared__ float lg[RF_TOK * LDW];
  __shared__ double pe[RF_TOK][E];                    // exp(l_j - l_0) of each row's picks
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, j = lane & 15;
  const int grp = 2 * wv + (lane >> 5);               // expert group of the lane's half
  const int64_t tb = (int64_t)blockIdx.x * RF_TOK;
  const int tr = lane & 31;                           // token row within the workgroup
  const int64_t t = tb + tr;
  const T* xr = x + min(t, n_tok - 1) * (int64_t)d;
  const T* wl = wr + (int64_t)(grp * EPL + j / LPE) * d + (j % LPE) * EPL;
  float acc[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) acc[q] = 0.0f;
  const int nc = d / RF_K;
  {
    RfRaw<T, EPL> ring[RF_NPRE];
#pragma unroll
    for (int q = 0; q < RF_NPRE; ++q) {
      const int c = min(q, nc - 1);
      ring[q].load(xr + c * RF_K, wl + c * RF_K);
    }
    // the ring of k_router_logits: slot c % NPRE holds chunk c, reloaded with chunk c + NPRE
    // (clamped to the last chunk) once its FMAs are issued; the last nc % NPRE chunks are
    // computed after the loop
    const int nc_main = nc - nc % RF_NPRE;
    for (int c0 = 0; c0 < nc_main; c0 += RF_NPRE) {
#pragma unroll
      for (int q = 0; q < RF_NPRE; ++q) {
        rf_chunk<T, EPL>(acc, ring[q], std::make_integer_sequence<int, RF_K>{});
        __builtin_amdgcn_sched_barrier(0);
        const int cn = min(c0 + q + RF_NPRE, nc - 1);
        ring[q].load(xr + cn * RF_K, wl + cn * RF_K);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int q = 0; q + 1 < RF_NPRE; ++q)
      if (nc_main + q < nc) rf_chunk<T, EPL>(acc, ring[q], std::make_integer_sequence<int, RF_K>{});
  }
  // the logits of the lane's token and its EPL experts (rows 0 and 1 of a half hold tokens
  // 0-15 and 16-31, so each (token, expert) is held by exactly one lane)
#pragma unroll
  for (int q = 0; q < EPL; ++q) lg[tr * LDW + grp * EPL + q] = acc[q];
  __syncthreads();
  // the logits go out as the workgroup's contiguous [32, E] block
  for (int i = tid; i < RF_TOK * E; i += 64 * NW) {
    const int r = i / E;
    if (tb + r < n_tok) logits[tb * E + i] = lg[r * LDW + i % E];
  }
  // top-k: 8 lanes per token row (row = tid / 8; lane s of the row holds experts s, s + 8, ...),
  // all 32 rows at once: each round takes the maximum of the lane's untaken keys, then of the
  // row's 8 lanes (three xor shuffles), with the keys and tie rule of topk_picks. Lane j % 8 of
  // the row writes pick j and its exp(l_j - l_0) (double), which the row then sums over j
  // ascending, as topk_weight does.
  static_assert(64 * NW == 8 * RF_TOK, "8 lanes per token row");
  constexpr int EPT = E / 8;
  const int row = tid >> 3, sub = tid & 7;
  const int64_t tt = tb + row;
  const bool live = tt < n_tok;
  uint32_t key[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) key[q] = float_order_key(lg[row * LDW + sub + 8 * q]);
  uint32_t taken = 0;
  float v0 = 0.0f;
  for (int jj = 0; jj < k; ++jj) {
    uint64_t best = 0;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const uint64_t c = ((uint64_t)key[q] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(sub + 8 * q));
      if (!((taken >> q) & 1u)) best = c > best ? c : best;
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      const uint64_t o = shfl_xor_u64(best, m);
      best = o > best ? o : best;
    }
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float v = float_from_order_key((uint32_t)(best >> 32));
    if ((e & 7) == sub) taken |= 1u << (e >> 3);
    if (jj == 0) v0 = v;
    if ((jj & 7) == sub && live) {
      topk_idx[tt * k + jj] = e;
      pe[row][jj] = exp((double)v - (double)v0);
    }
  }
  __syncthreads();
  if (live) {
    double wsum = 0.0;
    for (int jj = 0; jj < k; ++jj) wsum += pe[row][jj];
    for (int jj = sub; jj < k; jj += 8) topk_w[tt * k + jj] = (float)(pe[row][jj] / wsum);
  }
}

hipError_t launch_router_logits(const void* x, const void* wr, int64_t n_tok, int d, int E,
                                bool bf16, float* logits, hipStream_t s, hipEvent_t e0,
                                hipEvent_t e1) {
  if (n_tok == 0) return mark_empty(s, e0, e1), hipSuccess;
  const int64_t waves = ((n_tok + RT_TOK - 1) / RT_TOK) * ((E + RT_EXP - 1) / RT_EXP);
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (bf16)
    launch_k(k_router_logits<bf16_t>, grid, dim3(256), 0, s, e0, e1, (const bf16_t*)x,
             (const bf16_t*)wr, n_tok, d, E, logits);
  else
    launch_k(k_router_logits<float>, grid, dim3(256), 0, s, e0, e1, (const float*)x,
             (const float*)wr, n_tok, d, E, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t n_tok, int E, int k, int32_t* idx,
                       float* w, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (n_tok == 0) return mark_empty(s, e0, e1), hipSuccess;
  if (E > 64 * TK_MAXQ) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n_tok + 3) / 4)), block(256);
  if (E <= 64)
    launch_k(k_topk<1>, grid, block, 0, s, e0, e1, logits, n_tok, E, k, idx, w);
  else if (E <= 128)
    launch_k(k_topk<2>, grid, block, 0, s, e0, e1, logits, n_tok, E, k, idx, w);
  else if (E <= 256)
    launch_k(k_topk<4>, grid, block, 0, s, e0, e1, logits, n_tok, E, k, idx, w);
  else if (E <= 512)
    launch_k(k_topk<8>, grid, block, 0, s, e0, e1, logits, n_tok, E, k, idx, w);
  else
    launch_k(k_topk<TK_MAXQ>, grid, block, 0, s, e0, e1, logits, n_tok, E, k, idx, w);
  return hipGetLastError();
}

int64_t route_fused_blocks(int64_t n_tok, int d, int E, int k) {
  if (n_tok <= 0 || d <= 0 || d % RF_K != 0 || k < 1 || k > E) return 0;
  if (E != 16 && E != 32 && E != 64) return 0;
  return (n_tok + RF_TOK - 1) / RF_TOK;
}


hipError_t launch_route(const void* x, const void* wr, int64_t n_tok, int d, int E, int k,
                        bool bf16, float* logits, int32_t* idx, float* w, hipStream_t s,
                        hipEvent_t e0, hipEvent_t e1) {
  if (n_tok == 0) return mark_empty(s, e0, e1), hipSuccess;
  const int64_t nb = route_fused_blocks(n_tok, d, E, k);
  if (nb == 0) {
    hipError_t e = launch_router_logits(x, wr, n_tok, d, E, bf16, logits, s, e0, nullptr);
    if (e != hipSuccess) return e;
    return launch_topk(logits, n_tok, E, k, idx, w, s, nullptr, e1);
  }
  // four waves (one per SIMD: 256 workgroups of 32 tokens fill the chip at 8,192 tokens)
  const dim3 grid((unsigned)nb);
#define MOK_ROUTE_LAUNCH(T, EPL, NW)                                                           \
  launch_k(k_route<T, EPL, NW>, grid, dim3(64 * NW), 0, s, e0, e1, (const T*)x, (const T*)wr, \
           n_tok, d, k, logits, idx, w)
  if (bf16) {
    if (E == 16) MOK_ROUTE_LAUNCH(bf16_t, 2, 4);
    else if (E == 32) MOK_ROUTE_LAUNCH(bf16_t, 4, 4);
    else MOK_ROUTE_LAUNCH(bf16_t, 8, 4);
  } else {
    if (E == 16) MOK_ROUTE_LAUNCH(float, 2, 4);
    else if (E == 32) MOK_ROUTE_LAUNCH(float, 4, 4);
    else MOK_ROUTE_LAUNCH(float, 8, 4);
  }
#undef MOK_ROUTE_LAUNCH
  return hipGetLastError();
}

}  // namespace mok
