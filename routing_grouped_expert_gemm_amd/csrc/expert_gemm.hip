// Stages 3-5: pull gather, grouped SwiGLU expert GEMMs, shared expert, fixed-order combine.
//
// The MoK write-up ("Overlapping compute and communication in MoE"): each picked expert runs
// a standard FFN -- up and gate projections, SwiGLU, down projection -- and the layer
// combines shared and routed outputs with the router weights. The Telegram summary's pull
// dispatch: once an expert knows its tokens it fetches them itself, reading whole rows, with
// no scattered writes. The news summary: work is cut into minibatches of tunable size that
// flow through a "macrobatch" ring buffer, with no token dropped and no CPU-GPU sync.
//
// MI355X mapping:
//  * Work unit = a minibatch: <= mb consecutive rows of one expert's plan region (or of the
//    own tokens, for the shared experts). The work list (minibatches, tile counts and their
//    prefix sums) is built on the device from the plan's counts; the host never sees them.
//  * Ring: a minibatch's hidden activations live in ring slot m % n_slots.
//  * Up tile (gate/up GEMM + SwiGLU): the A tile is PULLED straight from the token pool by
//    route id (row = route_id / k), 128 B per row per K step, staged through LDS; the B tile
//    holds matching gate and up rows so each lane holds gate and up of the same (row, col)
//    in its accumulators and applies SwiGLU in registers before one store to the ring.
//  * Down tile: A = the ring rows, B = W_down; the epilogue scales each row by its routing
//    weight and stores it to the route's source-indexed slot (t*k + j) of y_slots.
//  * MFMA: v_mfma_f32_32x32x16_bf16 (bf16), v_mfma_f32_32x32x2_f32 (fp32),
//    v_mfma_scale_f32_32x32x64_f8f6f4 with E8M0 block scales (MXFP8). fp32 accumulation.
//  * LDS rows are 128 B (8 chunks of 16 B) per K step, chunk c of row r stored at c ^ (r & 7)
//    so the per-lane fragment reads and the row-wise tile writes are bank-conflict free.
#include "device_common.h"
#include "launch.h"

namespace mok {

// ------------------------------------------------------------------------- work list
// int32 block layout (offsets in ints)
constexpr int WL_N_MB = 0, WL_N_U = 1, WL_N_D = 2, WL_TICKET = 3, WL_ERR = 4, WL_HDR = 16;
MOK_DEV int32_t* wl_group(int32_t* wl, int cap) { return wl + WL_HDR; }
MOK_DEV int32_t* wl_row0(int32_t* wl, int cap) { return wl + WL_HDR + cap; }
MOK_DEV int32_t* wl_rows(int32_t* wl, int cap) { return wl + WL_HDR + 2 * cap; }
MOK_DEV int32_t* wl_ustart(int32_t* wl, int cap) { return wl + WL_HDR + 3 * cap; }
MOK_DEV int32_t* wl_dstart(int32_t* wl, int cap) { return wl + WL_HDR + 4 * cap + 1; }

size_t worklist_ints(int max_mb) { return WL_HDR + 5 * (size_t)max_mb + 2; }

// Block-wide exclusive scan of one int per thread (1024 threads). Returns the exclusive
// prefix; *total receives the sum.
MOK_DEV int32_t block_excl_scan_1024(int32_t v, int32_t* sh, int32_t* total) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t a = t >= off ? sh[t - off] : 0;
    __syncthreads();
    sh[t] += a;
    __syncthreads();
  }
  const int32_t incl = sh[t];
  *total = sh[1023];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(1024) void k_build_worklist(const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ offsets,
                                                         int E_l, int T_own, int mb, int bm,
                                                         int nU_r, int nU_s, int nD, int cap,
                                                         int32_t* __restrict__ wl) {
  __shared__ int32_t sh[1024];
  const int t = threadIdx.x;
  int32_t* grp = wl_group(wl, cap);
  int32_t* r0 = wl_row0(wl, cap);
  int32_t* nr = wl_rows(wl, cap);
  int32_t* us = wl_ustart(wl, cap);
  int32_t* ds = wl_dstart(wl, cap);
  // routed minibatches: experts ascending, rows ascending within each region
  int32_t n_routed = 0;
  for (int c0 = 0; c0 < E_l; c0 += 1024) {
    const int e = c0 + t;
    const int32_t cnt = e < E_l ? counts[e] : 0;
    const int32_t nm = (cnt + mb - 1) / mb;
    int32_t tot;
    const int32_t base = n_routed + block_excl_scan_1024(nm, sh, &tot);
    for (int i = 0; i < nm; ++i) {
      const int m = base + i;
      if (m < cap) {
        grp[m] = e;
        r0[m] = offsets[e] + i * mb;
        nr[m] = min(mb, cnt - i * mb);
      }
    }
    n_routed += tot;
  }
  const int32_t n_sh = (nU_s > 0 && T_own > 0) ? (T_own + mb - 1) / mb : 0;
  for (int i = t; i < n_sh; i += 1024) {
    const int m = n_routed + i;
    if (m < cap) {
      grp[m] = E_l;
      r0[m] = i * mb;
      nr[m] = min(mb, T_own - i * mb);
    }
  }
  const int32_t n_mb = min(cap, n_routed + n_sh);
  __syncthreads();
  // tile prefix sums: tiles of a minibatch = ceil(rows / bm) * n-tiles of its stage
  int32_t carry_u = 0, carry_d = 0;
  for (int c0 = 0; c0 < n_mb; c0 += 1024) {
    const int m = c0 + t;
    int32_t nu = 0, nd = 0;
    if (m < n_mb) {
      const int32_t mt = (nr[m] + bm - 1) / bm;
      nu = mt * (grp[m] < E_l ? nU_r : nU_s);
      nd = mt * nD;
    }
    int32_t tu, td;
    const int32_t eu = block_excl_scan_1024(nu, sh, &tu);
    const int32_t ed = block_excl_scan_1024(nd, sh, &td);
    if (m < n_mb) {
      us[m] = carry_u + eu;
      ds[m] = carry_d + ed;
    }
    carry_u += tu;
    carry_d += td;
  }
  if (t == 0) {
    us[n_mb] = carry_u;
    ds[n_mb] = carry_d;
    wl[WL_N_MB] = n_mb;
    wl[WL_N_U] = carry_u;
    wl[WL_N_D] = carry_d;
    wl[WL_TICKET] = 0;
    wl[WL_ERR] = (n_routed + n_sh > cap) ? 1 : 0;
  }
}

// largest m with start[m] <= t (start ascending, start[0] == 0)
MOK_DEV int find_mb(const int32_t* start, int n_mb, int32_t t) {
  int lo = 0, hi = n_mb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------------------- GEMM tiles
constexpr int BM = 128, BN = 128, NT = 256;
constexpr int WAVES_M = 2, WAVES_N = 2, WM = BM / WAVES_M, WN = BN / WAVES_N;
constexpr int FM = WM / 32, FN = WN / 32;
constexpr int ROWS_PER_PASS = NT / 8;               // 32 rows per pass of 8 x 16 B chunks
constexpr int A_PASSES = BM / ROWS_PER_PASS, B_PASSES = BN / ROWS_PER_PASS;

template <Elem EL> struct Tr;
template <> struct Tr<Elem::BF16> { static constexpr int ES = 2, KT = 64, SUB = 4, CPL = 1; };
template <> struct Tr<Elem::F32> { static constexpr int ES = 4, KT = 32, SUB = 2, CPL = 2; };
template <> struct Tr<Elem::FP8> { static constexpr int ES = 1, KT = 128, SUB = 2, CPL = 2; };

struct Smem {
  uint4 A[2][BM][8];
  uint4 B[2][BN][8];
  uint32_t Asc[2][BM];
  uint32_t Bsc[2][BN];
  int32_t row_dst[BM];
  float row_w[BM];
};

MOK_DEV int swz(int r, int c) { return c ^ (r & 7); }

// 16-byte chunk (of a 128 B LDS row) that lane half h feeds to the MFMA of K sub-step s.
//  bf16 32x32x16: one chunk, k = 16s + 8h + [0, 8).
//  fp32 32x32x2 (x8): two chunks, k = 16s + 8h + [0, 8).
//  fp8 32x32x64 (scaled): bytes 0-15 of a lane belong to the MFMA's first 32-wide K block and
//  bytes 16-31 to the second, each lane half taking 16 of a block's 32 k; the E8M0 scale of
//  lane l covers (row l % 32, block l / 32). So: chunks 4s + h and 4s + 2 + h.
template <Elem EL>
MOK_DEV int frag_chunk(int s, int h, int q) {
  if (EL == Elem::BF16) return 2 * s + h;
  if (EL == Elem::F32) return 4 * s + 2 * h + q;
  return 4 * s + 2 * q + h;
}

template <Elem EL>
MOK_DEV void mfma_step(const uint4 (&a)[FM][2], const uint4 (&b)[FN][2], const uint32_t* asc,
                       const uint32_t* bsc, f32x16_t (&acc)[FM][FN]);

template <>
MOK_DEV void mfma_step<Elem::BF16>(const uint4 (&a)[FM][2], const uint4 (&b)[FN][2],
                                   const uint32_t*, const uint32_t*, f32x16_t (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, a[i][0]), __builtin_bit_cast(bf16x8_t, b[j][0]), acc[i][j],
          0, 0, 0);
}

template <>
MOK_DEV void mfma_step<Elem::F32>(const uint4 (&a)[FM][2], const uint4 (&b)[FN][2],
                                  const uint32_t*, const uint32_t*, f32x16_t (&acc)[FM][FN]) {
  // Lane half h supplies k = 8h + q of a 16-wide K step to the q-th 32x32x2 product; A and B
  // use the same assignment, so the 8 products cover the step exactly once.
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const float* av = reinterpret_cast<const float*>(&a[i][0]);
      const float* bv = reinterpret_cast<const float*>(&b[j][0]);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[q], bv[q], acc[i][j], 0, 0, 0);
    }
}

template <>
MOK_DEV void mfma_step<Elem::FP8>(const uint4 (&a)[FM][2], const uint4 (&b)[FN][2],
                                  const uint32_t* asc, const uint32_t* bsc,
                                  f32x16_t (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      i32x8_t av, bv;
      av[0] = a[i][0].x; av[1] = a[i][0].y; av[2] = a[i][0].z; av[3] = a[i][0].w;
      av[4] = a[i][1].x; av[5] = a[i][1].y; av[6] = a[i][1].z; av[7] = a[i][1].w;
      bv[0] = b[j][0].x; bv[1] = b[j][0].y; bv[2] = b[j][0].z; bv[3] = b[j][0].w;
      bv[4] = b[j][1].x; bv[5] = b[j][1].y; bv[6] = b[j][1].z; bv[7] = b[j][1].w;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 0, 0, 0,
                                                                   (int)asc[i], 0, (int)bsc[j]);
    }
}

// Output element of the epilogues.
template <bool F32OUT> struct Out;
template <> struct Out<true> { typedef float T; };
template <> struct Out<false> { typedef bf16_t T; };

// One tile of the up (UP = true) or down (UP = false) stage of minibatch m.
template <Elem EL, bool UP, bool F32OUT>
MOK_DEV void run_tile(const ExpertPass& p, Smem& sm, int m, int local) {
  typedef Tr<EL> TR;
  typedef typename Out<F32OUT>::T OT;
  const int cap = p.max_mb;
  int32_t* wl = p.wl;
  const int g = wl_group(wl, cap)[m];
  const int row0 = wl_row0(wl, cap)[m];
  const int rows = wl_rows(wl, cap)[m];
  const bool shared = g >= p.E_l;
  const int slot = m % p.n_slots;
  const int64_t ring_row0 = (int64_t)slot * p.mb;
  const int n_mt = (rows + BM - 1) / BM;
  const int mt = local % n_mt, nt = local / n_mt;
  const int m0 = mt * BM;
  const int rows_valid = min(BM, rows - m0);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int K = UP ? p.d : (shared ? p.I_sh : p.I);
  const int nk = K / TR::KT;

  // ---- operand row pointers (each thread loads chunk c of rows (tid>>3) + 32*i)
  const int ldc = tid & 7;
  const char* a_ptr[A_PASSES];
  const char* b_ptr[B_PASSES];
  const uint8_t* a_sc = nullptr;   // MX scales row pointer (thread < BM: row tid)
  const uint8_t* b_sc = nullptr;   // MX scales row pointer (thread >= BM: row tid - BM)
  int64_t b_seg_len = K, b_seg_stride = 0;
#pragma unroll
  for (int i = 0; i < A_PASSES; ++i) {
    const int r = min((tid >> 3) + ROWS_PER_PASS * i, rows_valid - 1);
    int64_t base;
    if (UP && EL != Elem::FP8) {
      const int64_t tok = shared ? p.own_begin + row0 + m0 + r
                                 : (int64_t)(p.route_ids[row0 + m0 + r] / p.k);
      base = tok * p.d * TR::ES;
      a_ptr[i] = (const char*)p.x + base;
    } else if (UP) {
      a_ptr[i] = (const char*)p.A_codes + (ring_row0 + m0 + r) * p.d;
    } else {
      a_ptr[i] = (const char*)p.H + (ring_row0 + m0 + r) * (int64_t)p.Hld * TR::ES;
    }
  }
#pragma unroll
  for (int i = 0; i < B_PASSES; ++i) {
    const int j = (tid >> 3) + ROWS_PER_PASS * i;
    if (UP) {
      const int jw = j / WN, jj = j % WN;
      const int n = nt * (BN / 2) + jw * (WN / 2) + (jj % (WN / 2));
      const bool up = jj >= WN / 2;
      const void* W = shared ? (up ? p.su : p.sg) : (up ? p.wu : p.wg);
      const int64_t wrow = shared ? (int64_t)n : (int64_t)g * p.I + n;
      b_ptr[i] = (const char*)W + wrow * p.d * TR::ES;
    } else {
      const int n = nt * BN + j;
      if (shared) {
        b_ptr[i] = (const char*)p.sd + (int64_t)n * p.I_seg * TR::ES;
      } else {
        b_ptr[i] = (const char*)p.wd + ((int64_t)g * p.d + n) * p.I * TR::ES;
      }
    }
  }
  if (!UP && shared) {
    b_seg_len = p.I_seg;
    b_seg_stride = (int64_t)p.d * p.I_seg * TR::ES;
  }
  if (EL == Elem::FP8) {
    if (tid < BM) {
      const int r = min(tid, rows_valid - 1);
      a_sc = UP ? p.A_sc + (ring_row0 + m0 + r) * (int64_t)(p.d / 32)
                : p.H_sc + (ring_row0 + m0 + r) * (int64_t)(p.Hld / 32);
    } else {
      const int j = tid - BM;
      if (UP) {
        const int jw = j / WN, jj = j % WN;
        const int n = nt * (BN / 2) + jw * (WN / 2) + (jj % (WN / 2));
        const bool up = jj >= WN / 2;
        const uint8_t* S = shared ? (up ? p.su_sc : p.sg_sc) : (up ? p.wu_sc : p.wg_sc);
        const int64_t wrow = shared ? (int64_t)n : (int64_t)g * p.I + n;
        b_sc = S + wrow * (p.d / 32);
      } else {
        const int n = nt * BN + j;
        b_sc = shared ? p.sd_sc + (int64_t)n * (p.I_seg / 32)
                      : p.wd_sc + ((int64_t)g * p.d + n) * (p.I / 32);
      }
    }
  }
  // epilogue row table (down stage)
  if (!UP && tid < BM) {
    if (tid < rows_valid) {
      if (shared) {
        sm.row_dst[tid] = row0 + m0 + tid;
        sm.row_w[tid] = 1.0f;
      } else {
        const int32_t route = p.route_ids[row0 + m0 + tid];
        sm.row_dst[tid] = route;
        sm.row_w[tid] = p.topk_w[route];
      }
    }
  }

  // ---- main loop
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  uint4 ra[A_PASSES], rb[B_PASSES];
  uint32_t rsc = 0;
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * TR::KT;
    const int64_t aoff = k0 * TR::ES + ldc * 16;
    const int64_t seg = k0 / b_seg_len;
    const int64_t boff = seg * b_seg_stride + (k0 - seg * b_seg_len) * TR::ES + ldc * 16;
#pragma unroll
    for (int i = 0; i < A_PASSES; ++i) ra[i] = *(const uint4*)(a_ptr[i] + aoff);
#pragma unroll
    for (int i = 0; i < B_PASSES; ++i) rb[i] = *(const uint4*)(b_ptr[i] + boff);
    if (EL == Elem::FP8) {
      const int64_t kb = k0 / 32;
      if (tid < BM) rsc = *(const uint32_t*)(a_sc + kb);
      else {
        const int64_t kbs = (k0 - seg * b_seg_len) / 32;
        rsc = *(const uint32_t*)(b_sc + kbs + (seg * b_seg_stride) / 32);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PASSES; ++i) {
      const int r = (tid >> 3) + ROWS_PER_PASS * i;
      sm.A[buf][r][swz(r, ldc)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PASSES; ++i) {
      const int r = (tid >> 3) + ROWS_PER_PASS * i;
      sm.B[buf][r][swz(r, ldc)] = rb[i];
    }
    if (EL == Elem::FP8) {
      if (tid < BM) sm.Asc[buf][tid] = rsc;
      else sm.Bsc[buf][tid - BM] = rsc;
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  const int h = lane >> 5, l32 = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < TR::SUB; ++s) {
      uint4 fa[FM][2], fb[FN][2];
      uint32_t asc[FM], bsc[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WM + i * 32 + l32;
        fa[i][0] = sm.A[cur][r][swz(r, frag_chunk<EL>(s, h, 0))];
        if (TR::CPL == 2) fa[i][1] = sm.A[cur][r][swz(r, frag_chunk<EL>(s, h, 1))];
        if (EL == Elem::FP8) asc[i] = (sm.Asc[cur][r] >> (8 * (2 * s + h))) & 0xFFu;
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WN + j * 32 + l32;
        fb[j][0] = sm.B[cur][r][swz(r, frag_chunk<EL>(s, h, 0))];
        if (TR::CPL == 2) fb[j][1] = sm.B[cur][r][swz(r, frag_chunk<EL>(s, h, 1))];
        if (EL == Elem::FP8) bsc[j] = (sm.Bsc[cur][r] >> (8 * (2 * s + h))) & 0xFFu;
      }
      mfma_step<EL>(fa, fb, asc, bsc, acc);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue. Accumulator v of block (i, j) is (row 8*(v/4) + 4*h + v%4, col l32).
  if (UP) {
    const int64_t col0 = (int64_t)nt * (BN / 2) + wn * (WN / 2);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        const int64_t col = col0 + j * 32 + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          const float hv = silu(acc[i][j][v]) * acc[i][j + FN / 2][v];
          if (EL == Elem::FP8) {
            // MXFP8 along I: the 32 columns of this block row sit in the 32 lanes of half h
            float amax = fabsf(hv);
#pragma unroll
            for (int msk = 1; msk < 32; msk <<= 1) amax = fmaxf(amax, __shfl_xor(amax, msk, kWave));
            const int se = mx_shared_exp(amax);
            if (r < rows_valid) {
              const int64_t hr = ring_row0 + m0 + r;
              ((uint8_t*)p.H)[hr * p.Hld + col] = (uint8_t)e4m3_encode(hv, se);
              if (l32 == 0) p.H_sc[hr * (p.Hld / 32) + col / 32] = (uint8_t)(se + 127);
            }
          } else if (r < rows_valid) {
            const int64_t hr = ring_row0 + m0 + r;
            ((OT*)p.H)[hr * p.Hld + col] = f32_to<OT>(hv);
          }
        }
      }
  } else {
    const int64_t col0 = (int64_t)nt * BN + wn * WN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t col = col0 + j * 32 + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          if (r < rows_valid) {
            const int64_t dst = sm.row_dst[r];
            OT* out = shared ? (OT*)p.y_shared : (OT*)p.y_slots;
            out[dst * p.d + col] = f32_to<OT>(acc[i][j][v] * sm.row_w[r]);
          }
        }
      }
  }
  __syncthreads();  // LDS (row table, operand buffers) is reused by the next tile
}

// Stage kernel: the workgroups walk the stage's tiles; consecutive tile ids land on the same
// XCD (workgroups are dispatched round-robin over the 8 XCDs), so tiles that share operand
// rows share that XCD's L2.
template <Elem EL, bool UP, bool F32OUT>
__global__ __launch_bounds__(NT, 2) void k_expert_stage(ExpertPass p) {
  __shared__ Smem sm;
  const int cap = p.max_mb;
  const int n_mb = p.wl[WL_N_MB];
  const int32_t total = p.wl[UP ? WL_N_U : WL_N_D];
  const int32_t* start = UP ? wl_ustart(p.wl, cap) : wl_dstart(p.wl, cap);
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int xcd_slot = (b & 7) * (G >> 3) + (b >> 3);
  for (int32_t t0 = 0; t0 < total; t0 += G) {
    const int32_t t = t0 + xcd_slot;
    if (t >= total) break;
    const int m = find_mb(start, n_mb, t);
    run_tile<EL, UP, F32OUT>(p, sm, m, t - start[m]);
  }
}

// ------------------------------------------------------------------------- MXFP8 gather
// Pull-gather + quantise: the A rows of every minibatch (token rows of the pool picked by
// route id, or the own rows for the shared experts) become MXFP8 rows of its ring slot.
// One wave per row; lane i quantises blocks i, i+64, ... of the row.
__global__ __launch_bounds__(256) void k_gather_quantize(ExpertPass p) {
  const int cap = p.max_mb;
  const int n_mb = p.wl[WL_N_MB];
  const int32_t* grp = wl_group(p.wl, cap);
  const int32_t* r0 = wl_row0(p.wl, cap);
  const int32_t* nr = wl_rows(p.wl, cap);
  const int nbr = p.d / 32;
  const int lane = threadIdx.x & 63;
  const int64_t total_rows = (int64_t)n_mb * p.mb;
  for (int64_t q = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); q < total_rows;
       q += (int64_t)gridDim.x * 4) {
    const int m = (int)(q / p.mb), r = (int)(q % p.mb);
    if (r >= nr[m]) continue;
    const int64_t tok = grp[m] >= p.E_l ? p.own_begin + r0[m] + r
                                        : (int64_t)(p.route_ids[r0[m] + r] / p.k);
    const int64_t ring_row = (int64_t)(m % p.n_slots) * p.mb + r;
    const bf16_t* src = (const bf16_t*)p.x + tok * p.d;
    for (int b = lane; b < nbr; b += 64)
      quantize_block32(src + 32 * b, p.A_codes + ring_row * p.d + 32 * b,
                       p.A_sc + ring_row * nbr + b);
  }
}

// ------------------------------------------------------------------------- combine
// y[t] = S[t] + sum_{j ascending} P[t*k + j], float32 accumulator, one rounding. One thread
// per 16 B of a row: the k + 1 rows of a token are read once, y is written once.
template <class OT>
__global__ __launch_bounds__(256) void k_combine(const OT* __restrict__ S, const OT* __restrict__ P,
                                                 OT* __restrict__ y, int64_t n_tok, int k, int d) {
  constexpr int V = 16 / sizeof(OT);
  const int64_t per_row = d / V;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n_tok * per_row) return;
  const int64_t t = q / per_row, c = (q % per_row) * V;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0f;
  if (S) {  // no shared expert: S = 0
    const uint4 s = *(const uint4*)(S + t * d + c);
    const OT* sv = (const OT*)&s;
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = load_as_f32<OT>(sv + v);
  }
  for (int j = 0; j < k; ++j) {
    const uint4 pv = *(const uint4*)(P + (t * k + j) * d + c);
    const OT* pp = (const OT*)&pv;
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] += load_as_f32<OT>(pp + v);
  }
  uint4 o;
  OT* ov = (OT*)&o;
#pragma unroll
  for (int v = 0; v < V; ++v) ov[v] = f32_to<OT>(acc[v]);
  *(uint4*)(y + t * d + c) = o;
}

hipError_t launch_combine(const void* y_shared, const void* y_slots, void* y, int64_t n_tok,
                          int k, int d, bool f32, hipStream_t s) {
  const int V = f32 ? 4 : 8;
  const int64_t n = n_tok * (d / V);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (f32)
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(256), 0, s, (const float*)y_shared,
                       (const float*)y_slots, (float*)y, n_tok, k, d);
  else
    hipLaunchKernelGGL(k_combine<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)y_shared,
                       (const bf16_t*)y_slots, (bf16_t*)y, n_tok, k, d);
  return hipGetLastError();
}

// ------------------------------------------------------------------------- launch
static void record(void* const* ev, int i, hipStream_t s) {
  if (ev) (void)hipEventRecord((hipEvent_t)ev[i], s);
}

template <Elem EL, bool F32OUT>
static hipError_t launch_stages_t(const ExpertPass& p, hipStream_t s, void* const* ev) {
  hipLaunchKernelGGL((k_expert_stage<EL, true, F32OUT>), dim3(p.grid), dim3(NT), 0, s, p);
  record(ev, 2 * 3 + 1, s);
  record(ev, 2 * 4, s);
  hipLaunchKernelGGL((k_expert_stage<EL, false, F32OUT>), dim3(p.grid), dim3(NT), 0, s, p);
  record(ev, 2 * 4 + 1, s);
  return hipGetLastError();
}

hipError_t launch_expert_stages(const ExpertPass& p, hipStream_t s, void* const* ev) {
  const int nU_r = p.I / (BN / 2);
  const int nU_s = p.I_sh / (BN / 2);
  const int nD = p.d / BN;
  record(ev, 2 * 3, s);
  hipLaunchKernelGGL(k_build_worklist, dim3(1), dim3(1024), 0, s, p.counts, p.offsets, p.E_l,
                     p.T_own, p.mb, BM, nU_r, nU_s, nD, p.max_mb, p.wl);
  if (p.elem == Elem::BF16) return launch_stages_t<Elem::BF16, false>(p, s, ev);
  if (p.elem == Elem::F32) return launch_stages_t<Elem::F32, true>(p, s, ev);
  hipLaunchKernelGGL(k_gather_quantize, dim3(p.grid * 4), dim3(256), 0, s, p);
  return launch_stages_t<Elem::FP8, false>(p, s, ev);
}

}  // namespace mok
