// Backward of the MoE layer (or one rank's share of it) with the routing held fixed.
//
// The layer of the MoK write-up ("Overlapping compute and communication in MoE"): each local
// route r = t*k + j runs P_r = w_r * W_down (silu(W_gate a) * (W_up a)) on a = x[t]; the shared
// experts run the same FFN, unweighted, on the own tokens. The write-up presents MoK as a
// training kernel (its introduction) and the Telegram post reports forward and backward gains
// ("Method and experiments"); this file computes, through the same pull plan as the forward:
//   recompute   G = A Wg^T, U = A Wu^T                       (per expert, rows of its region)
//   dgrad down  D = dP Wd           (dP: the slot gradients gathered in plan order)
//   SwiGLU bwd  H = silu(G) U;  dw_r = <D_r, H_r>  (= <dP_r, W_down h_r>, the routing-weight
//               gradient);  dH = w D;  dG = dH U silu'(G);  dU = dH silu(G);  dO = w dP
//   dgrad up    dA = dG Wg + dU Wu  -> dx through each route (source-indexed slots)
//   wgrad       dWg = dG^T A, dWu = dU^T A, dWd = dO^T H     (ragged K: the expert's rows)
// and for a whole layer dx = dx_shared + sum_j dx_slot[t*k + j] with the forward's fixed-order
// combine. Every product is one launch of a grouped GEMM whose groups (one per expert and
// matrix) are described on the device from the plan's counts: the host never reads a count.
//
// Grouped GEMM: C_g (+)= A_g B_g^T over tiles of 256 x 256, K steps of 64, bf16 operands and
// float32 accumulation on v_mfma_f32_32x32x16_bf16, 4 waves of 128 x 128, operands moved to
// LDS by LDS-DMA. An operand is read either K-contiguous (row-major [rows, K]) or "transposed"
// (row-major [K, rows]: the wgrad operands, whose K is the token dimension, and the weights
// read along their output dimension); a transposed tile is kept in LDS as it lies in memory and
// gfx950's transposing LDS read turns it into the MFMA's K-contiguous fragments.
#include <algorithm>
#include <utility>

#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"
#include "mok.h"

namespace mok {

// One product of a grouped-GEMM launch. K may come in two segments: A and B for k < kseg,
// A2 and B2 beyond (kseg = K: one segment). The SwiGLU recompute reads B's rows as gate rows
// (B) and up rows (B2) instead, and its epilogue takes D, the routing weights (w[rid[row]], or
// 1 without rid) and writes dG, dU, w H and the per-row routing-weight-gradient partials.
struct GGroup {
  const bf16_t *A, *A2, *B, *B2;
  float* C;
  int64_t lda, ldb, ldc;
  int32_t M, N, K, tile0;   // tile0: the group's first flat tile
  int32_t kseg;
  int32_t ldp;              // SwiGLU: partials per row
  const bf16_t* D;          // SwiGLU: [M, ldc] bf16 (the dgrad-down product)
  bf16_t *dG, *dU, *Hw;     // SwiGLU: [M, ldc] bf16
  float* dwp;               // SwiGLU: [M, ldp] float32, or null
  const int32_t* rid;       // SwiGLU: route id of each row, or null (weight 1)
  const float* w;           // SwiGLU: routing weights by route id
  bf16_t* Cb;               // bf16 output instead of C: row rmap[m] (or m) of Cb, ld ldc
  const int32_t* rmap;      // output row of each row, or null
};
// A group table: header {groups, tiles, error, pad} then the groups.
constexpr int GT_HDR = 4;
MOK_HOSTDEV inline size_t gtable_bytes(int n_groups) {
  return sizeof(int32_t) * GT_HDR * 4 + sizeof(GGroup) * (size_t)n_groups;
}
MOK_DEV GGroup* gtable_groups(int32_t* t) { return (GGroup*)(t + GT_HDR * 4); }

constexpr int GB_M = 256, GB_N = 256, GB_K = 64;   // tile rows, tile columns, K step
constexpr int GB_MAX_GROUPS = 3 * 1024 + 4 + 64 + 256;   // groups of a table (E_l <= 1024,
                                                         // n_s <= 64, 256 K pieces)
constexpr int GB_NT = 256;                           // threads: 4 waves of 128 x 128
constexpr int GB_TILE = GB_M * GB_K * 2;             // bytes of one operand tile per K step
constexpr int GB_DMA = GB_TILE / 1024 / 4;           // LDS-DMA instructions per wave and operand

// One operand tile of a K step in LDS (32 KB), filled by LDS-DMA (every lane 16 bytes, an
// instruction 1 KB). Two layouts:
//  K-contiguous operand (row-major [rows, K]): 256 rows x 128 bytes; 16-byte chunk c of row r
//    at slot c ^ ((r >> 1) & 7) (as in the forward's tiles), read by ds_read_b128: lane (h, l32)
//    takes chunk 2 s + h of its row, the 8 K values of sub-step s.
//  Transposed operand (row-major [K, rows], e.g. a weight read along its output dimension, or
//    activations whose K is the token dimension): 64 k rows x 512 bytes; chunk c of k row kr at
//    slot c ^ (4 (kr & 3)). gfx950's transposing LDS read (ds_read_b64_tr_b16) turns it into
//    the same fragments: in each group of 16 lanes, lane p addresses 4 consecutive rows-of-the-
//    operand (4 (p % 4) further on) at k row kbase + p / 4, and lane i receives operand row
//    mbase + i at k rows kbase .. kbase + 3; two such reads give a lane its 8 K values. The
//    swizzle puts the 16 (k row, chunk) pairs a 32-lane half reads on 16 distinct slots, so
//    the 64 banks serve it in one pass.
template <bool T>
struct GOperand {
  // this lane's byte offset, from the tile's uniform base, of DMA instruction q of wave w
  // (K-contiguous: relative to row m0 at K offset k0; transposed: to k row k0, column 0)
  MOK_DEV static uint32_t dma_off(int w, int q, int lane, int64_t ld, int m0, int rows,
                                  int kk_max) {
    if constexpr (!T) {
      const int r = 64 * w + 8 * q + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int rr = min(m0 + r, rows - 1) - m0;       // rows past the operand: clamped
      return (uint32_t)(((int64_t)rr * ld + 8 * c) * 2);
    } else {
      const int kr = 16 * w + 2 * q + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (kr & 3));
      const int m = min(m0 + 8 * c, rows - 8);         // columns past the operand: clamped
      const int kk = min(kr, kk_max);                  // k rows past K: clamped (masked later)
      return (uint32_t)(((int64_t)kk * ld + m) * 2);
    }
  }
  // the 8 bf16 of K sub-step s for operand row blk + l32 (blk: the 32-row block, tile-relative)
  MOK_DEV static bf16x8_t frag(const char* tile, int blk, int s, int lane) {
    const int h = lane >> 5, l32 = lane & 31;
    if constexpr (!T) {
      const int r = blk + l32;
      const int c = (2 * s + h) ^ ((r >> 1) & 7);
      return *(const bf16x8_t*)(tile + r * 128 + c * 16);
    } else {
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4i16 lds_v4;
      const int g = lane >> 4, p = lane & 15;
      const int m = blk + 16 * (g & 1) + 4 * (p & 3);
      v4i16 v[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kr = 16 * s + 8 * (g >> 1) + 4 * kb + (p >> 2);
        const int off = kr * 512 + (((m >> 3) ^ (4 * (kr & 3))) << 4) + (m & 7) * 2;
        v[kb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4*)(uintptr_t)(lds_addr(tile) + off));
      }
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
};

// C_g (+)= A_g B_g^T for every group of the table; TA / TB: operand stored transposed.
// 256 x 256 tiles, 4 waves of 128 x 128 (4 x 4 accumulator blocks of 32 x 32: every LDS
// fragment feeds four MFMAs). K steps of 64 in two LDS buffers filled by LDS-DMA: the DMA of
// step kt + 1 is issued once every wave is past step kt - 1 and lands under the MFMAs of kt.
// A ragged K (the wgrad products: K is an expert's rows) clamps the DMA rows and zeroes the
// fragments' K values past the end in the last step.
template <bool TA, bool TB, bool SWIGLU>
__global__ __launch_bounds__(GB_NT) void k_ggemm(const int32_t* __restrict__ table) {
  static_assert(!SWIGLU || (!TA && !TB), "the SwiGLU recompute reads K-contiguous operands");
  __shared__ uint4 lds_a[2][GB_TILE / 16], lds_b[2][GB_TILE / 16];
  __shared__ int g_sh[2];
  __shared__ int32_t t0[GB_MAX_GROUPS];
  const int n_groups = table[0], total = table[1];
  // Persistent: workgroup w (on XCD w % 8; the grid is a multiple of 256) runs tiles
  // tile_of(0), tile_of(1), ... In each window of 256 consecutive tile slots XCD x takes 32
  // consecutive tiles, so tiles that share an operand tile share an L2, while the 8 XCDs still
  // work on neighbouring tiles (one expert's operands, which the last-level cache then serves
  // to all of them).
  auto tile_of = [&](int it) {
    const int w = blockIdx.x + it * gridDim.x, win = w & ~255, in = w & 255;
    return win + (in & 7) * 32 + (in >> 3);
  };
  int b = tile_of(0);
  if (b >= total) return;
  const GGroup* G = gtable_groups(const_cast<int32_t*>(table));
  // the group of a tile: the groups' first tiles come to LDS once, with one load per thread
  // (all in flight together); one thread then searches them there for each tile
  for (int q = threadIdx.x; q < n_groups; q += GB_NT) t0[q] = G[q].tile0;
  __syncthreads();
  auto find = [&](int bt) {
    int lo = 0, hi = n_groups;                  // t0[lo] <= bt < t0[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (t0[mid] <= bt) lo = mid; else hi = mid;
    }
    return lo;
  };
  if (threadIdx.x == 0) g_sh[0] = find(b);
  __syncthreads();
  // a tile's descriptor is read with scalar loads (constant address space, uniform index): a
  // vector load would count in vmcnt, and waiting for it would wait for every DMA and store
  // issued before it
  auto load_group = [&](int q) {
    static_assert(sizeof(GGroup) % 8 == 0, "whole 8-byte words");
    typedef const __attribute__((address_space(4))) uint64_t* WordsC;
    const WordsC w = (WordsC)(G + q);
    GGroup r;
    uint64_t* d = (uint64_t*)&r;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(GGroup) / 8); ++i) d[i] = w[i];
    return r;
  };
  GGroup g = load_group(uniform(g_sh[0]));
  const int tid = threadIdx.x, lane = tid & 63, wid = uniform(tid >> 6);
  const int wm = wid >> 1, wn = wid & 1, h = lane >> 5;
  constexpr int FM = 4, FN = 4;
  // a tile's origin and K steps
  auto origin = [&](const GGroup& gg, int bt, int& m0, int& n0) {
    const int tiles_n = (gg.N + GB_N - 1) / GB_N, local = bt - gg.tile0;
    m0 = (local / tiles_n) * GB_M;
    n0 = (local % tiles_n) * GB_N;
  };
  // uniform base of an operand's tile at K offset kin of its segment
  auto base = [&](const bf16_t* P, int64_t ld, int r0, bool T, int kin) {
    return uniform_ptr(T ? P + (int64_t)kin * ld : P + (int64_t)r0 * ld + kin);
  };
  // DMA instruction q (A: q < GB_DMA, B: the rest) of K step kt of tile (gg, tm0, tn0) into
  // buffer buf. SwiGLU recompute: tile column R is a gate row (slab R / 64 even) or an up row
  // (odd) of output column tn0 / 2 + (R / 128) * 64 + R % 64, so each wave's 128 columns pair
  // 64 gate columns with the same 64 up columns; wave w loads slab w.
  auto issue_q = [&](const GGroup& gg, int tm0, int tn0, int kt, int buf, int q) {
    __builtin_amdgcn_sched_barrier(0);
    const int k0 = kt * GB_K;
    const bool seg2 = k0 >= gg.kseg;
    const int kin = seg2 ? k0 - gg.kseg : k0;
    const int kk_max = (seg2 ? gg.K : gg.kseg) - 1 - k0;   // last valid k row of the step
    if (q < GB_DMA) {
      const uint32_t la = uniform(lds_addr(&lds_a[buf][0])) + (wid * GB_DMA + q) * 1024;
      dma_b128(base(seg2 ? gg.A2 : gg.A, gg.lda, tm0, TA, kin),
               GOperand<TA>::dma_off(wid, q, lane, gg.lda, tm0, gg.M, kk_max), la);
    } else {
      const int r = q - GB_DMA;
      const int b_r0 = SWIGLU ? tn0 / 2 + (wid >> 1) * 64 - 64 * wid : tn0;
      const int b_rows = SWIGLU ? gg.N / 2 : gg.N;
      const uint32_t lb = uniform(lds_addr(&lds_b[buf][0])) + (wid * GB_DMA + r) * 1024;
      const bf16_t* pb = SWIGLU ? ((wid & 1) ? gg.B2 : gg.B) : (seg2 ? gg.B2 : gg.B);
      dma_b128(base(pb, gg.ldb, b_r0, TB, kin),
               GOperand<TB>::dma_off(wid, r, lane, gg.ldb, b_r0, b_rows, kk_max), lb);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // the first two K steps of a tile, into buffers 0 and 1
  auto issue_head = [&](const GGroup& gg, int tm0, int tn0) {
    const int tnk = (gg.K + GB_K - 1) / GB_K;
    for (int kt = 0; kt < 2 && kt < tnk; ++kt)
      for (int q = 0; q < 2 * GB_DMA; ++q) issue_q(gg, tm0, tn0, kt, kt, q);
  };
  // every wave's DMA issued so far has landed and every wave's LDS reads are back
  auto barrier_x = [&]() {
    __builtin_amdgcn_s_waitcnt(0x70);   // vmcnt(0) lgkmcnt(0) (gfx9 encoding, expcnt left at 7)
    lds_barrier();
  };
  // the same, but the last N vector-memory operations this wave issued may still be in flight
  // (vmcnt counts in issue order): a barrier for a DMA that N younger operations follow
  auto barrier_n = [&](auto N_) {
    constexpr int N = decltype(N_)::value;
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));   // lgkmcnt(0)
    lds_barrier();
  };
  // Plain products: of a tile's 64 stores (16 bytes of float32 or 8 of bf16 a lane each), the
  // first ST_A go out before the next tile's first two K steps and the other ST_B after them, so
  // that the next tile's first barrier waits for its step-0 DMA and ST_A stores only (ST_B + 16
  // younger operations: at most vmcnt's 63).
  constexpr int ST_A = 17, ST_B = FM * FN * 4 - ST_A;
  static_assert(ST_B + 2 * GB_DMA == 63, "vmcnt range");
  bool tail_st = false;                 // the previous tile left ST_B stores behind its head
  int m0, n0;
  origin(g, b, m0, n0);
  issue_head(g, m0, n0);
  for (int it = 0;; ++it) {
    const int bn = tile_of(it + 1);
    const bool more = bn < total;
    if (more && tid == 0) g_sh[(it + 1) & 1] = find(bn);   // read after X(0) below
    const int nk = (g.K + GB_K - 1) / GB_K;
    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    float wrow[FM];
    int32_t orow[FM];
    bf16x8_t fa[2][FM], fb[2][FN];
    // fragments of K sub-step s of step kt into slot f; K values past a ragged end zeroed
    auto frags = [&](int kt, int s, int f) {
      const char* ta = (const char*)&lds_a[kt & 1][0];
      const char* tb = (const char*)&lds_b[kt & 1][0];
      // in the order the MFMAs (row-block major) first use them: A block 0, the B blocks, the
      // other A blocks
      fa[f][0] = GOperand<TA>::frag(ta, wm * 128, s, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[f][j] = GOperand<TB>::frag(tb, wn * 128 + 32 * j, s, lane);
#pragma unroll
      for (int i = 1; i < FM; ++i) fa[f][i] = GOperand<TA>::frag(ta, wm * 128 + 32 * i, s, lane);
      const int k_left = g.K - kt * GB_K;
      if (k_left < GB_K) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (16 * s + 8 * h + q >= k_left) {
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[f][i][q] = (__bf16)0.0f;
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[f][j][q] = (__bf16)0.0f;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // the 16 MFMAs of the fragments in slot f; after(n) follows MFMA n
    auto mfmas = [&](int f, auto&& after) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f][j], fa[f][i], acc[i][j], 0, 0, 0);
          after(i * FN + j);
        }
      __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(2 * GB_DMA == FM * FN && GB_K / 16 == 4, "one DMA per MFMA of the last sub-step");
    // K loop. The tile's first two steps were issued before (the first tile's here, later ones'
    // under the previous tile's epilogue). Step kt: sub-steps 0-2 (each reading the next
    // sub-step's fragments part-way through), then barrier X(kt + 1) (step kt + 1 has landed;
    // every wave has its reads of step kt back), and sub-step 3 of kt, whose MFMAs are
    // interleaved with the DMA of step kt + 2 into the buffer kt just released and, part-way,
    // with the reads of step kt + 1's first sub-step.
    // The reads of sub-step s + 1 go out after the first NEXT_AT MFMAs of s: issued before
    // them, they would sit ahead of s's own reads in the LDS counter (which tracks 15), and the
    // first MFMA would wait for most of both sub-steps' reads.
    constexpr int NEXT_AT = 8;
    // X(0): step 0 has landed; younger in flight: step 1's DMA and the previous tile's ST_B
    // stores (a count below the true one only waits longer)
    const bool two = nk > 1;
    if (tail_st) {
      if (two) barrier_n(std::integral_constant<int, 2 * GB_DMA + ST_B>{});
      else barrier_n(std::integral_constant<int, ST_B>{});
    } else {
      if (two) barrier_n(std::integral_constant<int, 2 * GB_DMA>{});
      else barrier_x();
    }
    // SwiGLU: the routing weight of the lane's row in each block row; bf16 output: its output
    // row (both loaded under the K loop, after X(0), so that no wait above counts them)
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = m0 + wm * 128 + 32 * i + (lane & 31);
      wrow[i] = 1.0f;
      orow[i] = m;
      if constexpr (SWIGLU) {
        if (g.rid && m < g.M) {                  // global loads: a flat one would also count in
          const int32_t r = *(const __attribute__((address_space(1))) int32_t*)(g.rid + m);
          wrow[i] = *(const __attribute__((address_space(1))) float*)(g.w + r);   // the LDS counter
        }
      } else {
        if (g.rmap && m < g.M) orow[i] = *(const __attribute__((address_space(1))) int32_t*)(g.rmap + m);
      }
    }
    GGroup gn = g;
    if (more) gn = load_group(uniform(g_sh[(it + 1) & 1]));
    if (nk > 0) frags(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int s = 0; s < 3; ++s)
        mfmas(s & 1, [&](int n) {
          if (n == NEXT_AT - 1) frags(kt, s + 1, (s + 1) & 1);
        });
      const bool next = kt + 1 < nk, more2 = kt + 2 < nk;
      if (next) {                               // X(kt + 1)
        if (kt == 0 && tail_st) barrier_n(std::integral_constant<int, ST_B>{});
        else barrier_x();
      }
      mfmas(1, [&](int n) {
        if (more2) issue_q(g, m0, n0, kt + 2, kt & 1, n);
        if (next && n == NEXT_AT - 1) frags(kt + 1, 0, 0);
      });
    }
    // the next tile's first two steps go out before this tile's stores, so that their loads
    // and the store drain overlap
    int m0n = 0, n0n = 0;
    if (more) {
      origin(gn, bn, m0n, n0n);
      barrier_x();                              // every wave is done with both buffers
    }
    // lane (h, l32) of block (i, j): row m0 + wm*128 + 32 i + l32, columns n0 + wn*128 + 32 j +
    // 8 q + 4 h + [0, 4) in values 4q .. 4q + 3 (the B fragment is the MFMA's first operand)
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const int l32 = lane & 31;
    if constexpr (!SWIGLU) {
      // store t = 16 i + 4 j + q; every one is issued (one past the matrix goes to the table
      // header's spare words), so the counts above are exact
      char* trash = (char*)(const_cast<int32_t*>(table) + 8);
      auto store = [&](int t) {
        const int i = t / 16, j = (t / 4) % 4, q = t % 4;
        const int m = m0 + wm * 128 + 32 * i + l32;
        const int n = n0 + wn * 128 + 32 * j + 8 * q + 4 * h;
        const bool ok = m < g.M && n < g.N;
        f32x4v o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = acc[i][j][4 * q + r];
        // global (not flat) stores: a flat store would also count in the LDS counter, which
        // every fragment read waits on
        if (g.Cb) {
          bf16_t* dst = g.Cb + (int64_t)orow[i] * g.ldc + n;
          typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
          const u32x2v v2 = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          *(__attribute__((address_space(1))) u32x2v*)(ok ? (char*)dst : trash) = v2;
        } else {
          float* dst = g.C + (int64_t)m * g.ldc + n;
          *(__attribute__((address_space(1))) f32x4v*)(ok ? (char*)dst : trash) = o;
        }
      };
#pragma unroll
      for (int t = 0; t < ST_A; ++t) store(t);
      if (more) issue_head(gn, m0n, n0n);
#pragma unroll
      for (int t = ST_A; t < ST_A + ST_B; ++t) store(t);
      tail_st = more;
    } else {
      if (more) issue_head(gn, m0n, n0n);
      // SwiGLU backward of the wave's 64 output columns (blocks j = 0, 1: G; j + 2: U, the same
      // columns): H = silu(G) U, dH = w D, dG = dH U silu'(G), dU = dH silu(G), and the row's
      // partial <D, H> over these columns (fixed order: the lane's 32 values, then its h pair).
      const int I = g.N / 2, ic0 = n0 / 2 + 64 * wn;   // I is a multiple of 64
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * 128 + 32 * i + l32;
        const bool ok = m < g.M && ic0 < I;
        const float wv = wrow[i];
        float dws = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = ic0 + 32 * j + 8 * q + 4 * h;
            const int64_t at = (int64_t)m * g.ldc + col;
            f32x4v d4 = {0.0f, 0.0f, 0.0f, 0.0f};
            if (ok) {
              typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
              const u32x2v w = *(const __attribute__((address_space(1))) u32x2v*)(g.D + at);
              d4[0] = __uint_as_float(w[0] << 16); d4[1] = __uint_as_float(w[0] & 0xFFFF0000u);
              d4[2] = __uint_as_float(w[1] << 16); d4[3] = __uint_as_float(w[1] & 0xFFFF0000u);
            }
            float og[4], ou[4], oh[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float gv = acc[i][j][4 * q + r], uv = acc[i][j + 2][4 * q + r], dd = d4[r];
              const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv));
              const float sl = gv * sg, hv = sl * uv, dh = wv * dd;
              dws += dd * hv;
              og[r] = dh * uv * sg * (1.0f + gv * (1.0f - sg));
              ou[r] = dh * sl;
              oh[r] = wv * hv;
            }
            if (ok) {
              *(uint2*)(g.dG + at) = make_uint2(pack_bf16x2(og[0], og[1]), pack_bf16x2(og[2], og[3]));
              *(uint2*)(g.dU + at) = make_uint2(pack_bf16x2(ou[0], ou[1]), pack_bf16x2(ou[2], ou[3]));
              *(uint2*)(g.Hw + at) = make_uint2(pack_bf16x2(oh[0], oh[1]), pack_bf16x2(oh[2], oh[3]));
            }
          }
        dws += __shfl_xor(dws, 32, 64);
        if (g.dwp && h == 0 && m < g.M)                // a wave past I contributes 0
          g.dwp[(int64_t)m * g.ldp + (n0 / GB_N) * 2 + wn] = ic0 < I ? dws : 0.0f;
      }
    }
    if (!more) break;
    g = gn;
    b = bn;
    m0 = m0n;
    n0 = n0n;
  }
}

// ------------------------------------------------------------------------- descriptions
// Everything the backward's kernels need (device pointers).
struct BwdPass {
  int d, k, I, E_l, I_s, n_s, T_own;
  int64_t cap;                   // routed rows the buffers hold
  int ldp;                       // routing-weight-gradient partials per routed row
  const int32_t *counts, *offsets, *route_ids;
  const float* topk_w;
  const bf16_t *wg, *wu, *wd, *sg, *su, *sd;
  const bf16_t* A_own;           // x own rows [T_own, d]
  const bf16_t* dP_own;          // their output gradient [T_own, d]
  bf16_t *Ar, *dPr, *dGr, *dUr, *Hr, *dGo, *dUo, *Ho;   // Hr: w H
  bf16_t *Dr, *Do;               // D = dP Wd in bf16 (read by the recompute epilogue)
  float* dwp;
  bf16_t *dx_slots, *dx_shared;  // outputs: dx through each route, the shared experts' dx
  float *dwg, *dwu, *dwd, *dsg, *dsu, *dsd;
  int32_t *t_rec, *t_dd, *t_du, *t_wg;   // group tables
  int32_t* err;                  // error word (routes past the capacity)
  // the wgrad table's last window, when it holds only part of one: its shared-expert tiles
  // split along K (ws_kept shared tiles stay whole; each later one becomes ws_P pieces of
  // ws_plen rows, summed by k_bwd_split_sum); ws_kept < 0: no split
  int ws_kept, ws_P, ws_plen;
  float* ws_part;                // [split tiles][ws_P][256][256] partial gradients
  struct SplitTile* ws_split;    // [split tiles] where each sum goes
};

// A weight-gradient tile computed in K pieces: its block of the gradient matrix.
struct SplitTile {
  float* C;
  int ldc, M, N;
};

MOK_DEV GGroup plain(const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb, float* C,
                     int64_t ldc, int M, int N, int K) {
  GGroup g = {};
  g.A = A; g.A2 = A; g.B = B; g.B2 = B; g.C = C;
  g.lda = lda; g.ldb = ldb; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K; g.kseg = K;
  return g;
}
MOK_DEV void put(GGroup* G, int& n, int32_t& tiles, GGroup g) {
  g.tile0 = tiles;
  G[n++] = g;
  tiles += ((g.M + GB_M - 1) / GB_M) * ((g.N + GB_N - 1) / GB_N);
}
MOK_DEV void close_table(int32_t* t, int n, int32_t tiles) { t[0] = n; t[1] = tiles; }

// Thread e writes expert e's groups of every table; the shared experts' groups follow the
// routed ones and are written by thread 0. A routed group's place and first tile come from two
// block scans over the experts: of "has rows" (the recompute and dgrad tables list only experts
// with rows) and of their M tile counts (a group's tiles are its M tiles times a column count
// that is the same for every expert of a table). The wgrad table lists three groups per expert,
// rows or not, each of the same tile count, then the shared experts' groups (K = all own
// tokens), the tiles of its last partial window split along K when the host asks for it.
constexpr int BD_THREADS = 1024;
__global__ __launch_bounds__(BD_THREADS) void k_bwd_describe(BwdPass p) {
  __shared__ int32_t sh[64];
  const int E = p.E_l, d = p.d, I = p.I, Ish = p.n_s * p.I_s, e = threadIdx.x;
  const bool over = (int64_t)p.offsets[E] > p.cap;
  const int c = (e < E && !over) ? p.counts[e] : 0;
  const int64_t o = e < E ? (int64_t)p.offsets[e] : 0;
  const int mt = (c + GB_M - 1) / GB_M;
  int32_t n_has, mt_all;
  const int32_t pos = block_excl_scan_1024(c > 0 ? 1 : 0, sh, &n_has);
  const int32_t mt0 = block_excl_scan_1024(mt, sh, &mt_all);
  auto cols = [](int N) { return (N + GB_N - 1) / GB_N; };
  auto rows = [](int M) { return (M + GB_M - 1) / GB_M; };
  auto tiles = [&](const GGroup& g) { return rows(g.M) * cols(g.N); };
  GGroup* Grec = gtable_groups(p.t_rec);
  GGroup* Gdd = gtable_groups(p.t_dd);
  GGroup* Gdu = gtable_groups(p.t_du);
  GGroup* Gwg = gtable_groups(p.t_wg);
  // recompute + SwiGLU backward: G, U = A [Wg; Wu]^T, paired column by column, with D (from the
  // dgrad-down launch before) in the epilogue
  auto rec = [&](const bf16_t* A, const bf16_t* Wg, const bf16_t* Wu, int M, int In,
                 const bf16_t* D, bf16_t* dG, bf16_t* dU, bf16_t* Hw, float* dwp,
                 const int32_t* rid) {
    GGroup g = plain(A, d, Wg, d, nullptr, In, M, 2 * In, d);
    g.B2 = Wu;
    g.D = D; g.dG = dG; g.dU = dU; g.Hw = Hw; g.dwp = dwp; g.ldp = p.ldp;
    g.rid = rid; g.w = p.topk_w;
    return g;
  };
  // dgrad up: dA = [dG dU] [Wg; Wu] as one product over K = 2 I in two segments (the weights
  // read along d: transposed B); dx rows in bf16: a routed row to its source-indexed slot, an
  // own row to dx_shared
  auto du = [&](const bf16_t* dG, const bf16_t* dU, const bf16_t* Wg, const bf16_t* Wu,
                bf16_t* dx, const int32_t* rmap, int M, int In) {
    GGroup g = plain(dG, In, Wg, d, nullptr, d, M, d, 2 * In);
    g.A2 = dU; g.B2 = Wu; g.kseg = In;
    g.Cb = dx; g.rmap = rmap;
    return g;
  };
  if (e < E) {
    if (c > 0) {
      GGroup g = rec(p.Ar + o * d, p.wg + (int64_t)e * I * d, p.wu + (int64_t)e * I * d, c, I,
                     p.Dr + o * I, p.dGr + o * I, p.dUr + o * I, p.Hr + o * I, p.dwp + o * p.ldp,
                     p.route_ids + o);
      g.tile0 = mt0 * cols(2 * I);
      Grec[pos] = g;
      // dgrad down: D = dP Wd (Wd read along its output dimension: transposed B)
      g = plain(p.dPr + o * d, d, p.wd + (int64_t)e * d * I, I, nullptr, I, c, I, d);
      g.Cb = p.Dr + o * I;
      g.tile0 = mt0 * cols(I);
      Gdd[pos] = g;
      g = du(p.dGr + o * I, p.dUr + o * I, p.wg + (int64_t)e * I * d, p.wu + (int64_t)e * I * d,
             p.dx_slots, p.route_ids + o, c, I);
      g.tile0 = mt0 * cols(d);
      Gdu[pos] = g;
    }
    // wgrad (both operands transposed: K is the expert's rows); with no rows the gradient is
    // written as zero. dWd = dP^T (w H).
    const GGroup w3[3] = {
        plain(p.dGr + o * I, I, p.Ar + o * d, d, p.dwg + (int64_t)e * I * d, d, I, d, c),
        plain(p.dUr + o * I, I, p.Ar + o * d, d, p.dwu + (int64_t)e * I * d, d, I, d, c),
        plain(p.dPr + o * d, d, p.Hr + o * I, I, p.dwd + (int64_t)e * d * I, I, d, I, c)};
    for (int j = 0; j < 3; ++j) {
      GGroup g = w3[j];
      g.tile0 = (3 * e + j) * tiles(w3[0]);
      Gwg[3 * e + j] = g;
    }
  }
  // the split tiles' operands, for the pieces every thread writes at the end
  struct PieceSrc {
    const bf16_t *A, *B;
    int64_t lda, ldb;
    int K, M, N;
  };
  __shared__ PieceSrc src[128];                  // ws_P >= 2 pieces of <= 256 slots
  __shared__ int32_t piece0[3];                  // first piece group, its first tile, tiles split
  if (e == 0) {
  *p.err = over ? (int32_t)MOK_DEVERR_OVERFLOW : 0;
  int n_rec = n_has, n_dd = n_has, n_du = n_has, n_wg = 3 * E;
  int32_t tl_rec = mt_all * cols(2 * I), tl_dd = mt_all * cols(I), tl_du = mt_all * cols(d);
  int32_t tl_wg = 3 * E * ((I + GB_M - 1) / GB_M) * cols(d);
  if (Ish > 0 && p.T_own > 0) {
    put(Grec, n_rec, tl_rec,
        rec(p.A_own, p.sg, p.su, p.T_own, Ish, p.Do, p.dGo, p.dUo, p.Ho, nullptr, nullptr));
    for (int s = 0; s < p.n_s; ++s)
    {
      GGroup gd = plain(p.dP_own, d, p.sd + (int64_t)s * d * p.I_s, p.I_s, nullptr, Ish, p.T_own,
                        p.I_s, d);
      gd.Cb = p.Do + s * p.I_s;
      put(Gdd, n_dd, tl_dd, gd);
    }
    if (p.dx_shared)
      put(Gdu, n_du, tl_du, du(p.dGo, p.dUo, p.sg, p.su, p.dx_shared, nullptr, p.T_own, Ish));
  }
  int n_split = 0;
  if (Ish > 0) {
    // the shared experts' wgrad groups in order; past the first ws_kept of their tiles, each
    // tile becomes ws_P one-tile groups over consecutive K ranges (written below by every
    // thread), whose partial sums k_bwd_split_sum adds
    int32_t left = p.ws_kept < 0 ? INT32_MAX : p.ws_kept;
    auto put_sh = [&](GGroup g) {
      const int tn = cols(g.N), tiles = rows(g.M) * tn;
      const int keep = min(tiles, left);
      if (keep > 0) {
        g.tile0 = tl_wg;
        Gwg[n_wg++] = g;
        tl_wg += keep;                           // its tiles end where the next group begins
      }
      left -= keep;
      for (int l = keep; l < tiles; ++l, ++n_split) {
        const int m0 = (l / tn) * GB_M, n0 = (l % tn) * GB_N;
        const SplitTile st = {g.C + (int64_t)m0 * g.ldc + n0, (int)g.ldc, min(GB_M, g.M - m0),
                              min(GB_N, g.N - n0)};
        p.ws_split[n_split] = st;
        src[n_split] = {g.A + m0, g.B + n0, g.lda, g.ldb, g.K, st.M, st.N};
      }
    };
    put_sh(plain(p.dGo, Ish, p.A_own, d, p.dsg, d, Ish, d, p.T_own));
    put_sh(plain(p.dUo, Ish, p.A_own, d, p.dsu, d, Ish, d, p.T_own));
    for (int s = 0; s < p.n_s; ++s)
      put_sh(plain(p.dP_own, d, p.Ho + s * p.I_s, Ish, p.dsd + (int64_t)s * d * p.I_s, p.I_s, d,
                   p.I_s, p.T_own));
  }
  close_table(p.t_rec, n_rec, tl_rec);
  close_table(p.t_dd, n_dd, tl_dd);
  close_table(p.t_du, n_du, tl_du);
  const int n_pieces = n_split * p.ws_P;       // one tile each, after every other group
  close_table(p.t_wg, n_wg + n_pieces, tl_wg + n_pieces);
  piece0[0] = n_wg;
  piece0[1] = tl_wg;
  piece0[2] = n_split;
  }
  __syncthreads();
  const int P = p.ws_P;
  for (int t = e; t < piece0[2] * P; t += BD_THREADS) {
    const PieceSrc& g = src[t / P];
    const int k0 = (t % P) * p.ws_plen;
    GGroup pg = plain(g.A + (int64_t)k0 * g.lda, g.lda, g.B + (int64_t)k0 * g.ldb, g.ldb,
                      p.ws_part + (int64_t)t * GB_M * GB_N, GB_N, g.M, g.N,
                      min(p.ws_plen, g.K - k0));
    pg.tile0 = piece0[1] + t;
    Gwg[piece0[0] + t] = pg;
  }
}

// The split tiles' gradients: the ws_P partial sums of each element added in ascending piece
// order (deterministic). Workgroup (t, m): row m of split tile t, a thread per column; the
// partials are loaded 16 at a time, all in flight together, then added in order.
__global__ __launch_bounds__(256) void k_bwd_split_sum(BwdPass p) {
  const SplitTile st = p.ws_split[blockIdx.x];
  const int m = blockIdx.y, n = threadIdx.x;
  if (m >= st.M || n >= st.N) return;
  const float* part = p.ws_part + (int64_t)blockIdx.x * p.ws_P * GB_M * GB_N + m * GB_N + n;
  float acc = 0.0f;
  for (int q0 = 0; q0 < p.ws_P; q0 += 16) {
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = q0 + q < p.ws_P ? part[(int64_t)(q0 + q) * GB_M * GB_N] : 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (q0 + q < p.ws_P) acc += v[q];
  }
  st.C[(int64_t)m * st.ldc + n] = acc;
}

// The routing-weight gradient of each routed row: its partials summed in ascending order, to
// [t, j] (the dgrad-up product writes dx itself). One thread per row.
__global__ __launch_bounds__(256) void k_bwd_dtopk(BwdPass p, float* __restrict__ dtopk_w) {
  const int64_t N = min((int64_t)p.offsets[p.E_l], p.cap);
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (*p.err || row >= N) return;
  float s = 0.0f;
  for (int q = 0; q < p.ldp; ++q) s += p.dwp[row * p.ldp + q];
  dtopk_w[p.route_ids[row]] = s;
}

}  // namespace mok

// ------------------------------------------------------------------------- C ABI
using namespace mok;

namespace {

constexpr size_t kAl = 256;
size_t al(size_t v) { return (v + kAl - 1) / kAl * kAl; }

struct BwdLayout {
  size_t counts, offsets, route_ids, blk_counts, err, ws_part, ws_split;
  size_t Ar, dPr, dGr, dUr, Hr, dGo, dUo, Ho, Dr, Do, dwp;
  size_t t_rec, t_dd, t_du, t_wg, total;
  int64_t cap;
  int ldp;                       // routing-weight-gradient partials per routed row
  int64_t tiles_rec, tiles_dd, tiles_du, tiles_wg;
  int ws_kept, ws_r, ws_P, ws_plen;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The wgrad launch's tile count is fixed by the shapes: 3 E_l routed groups of
// ceil(I/256) x ceil(d/256) tiles (every expert, rows or not), then the shared experts'. The
// persistent grid runs 256 tiles a window, so when the last window holds only r < 256 tiles and
// they are shared-expert tiles of K = T_own, r workgroups would run them alone (with EP1's
// 8,192 own tokens ~0.2 ms). Those r tiles are split instead into P K pieces each (P r <= 256,
// pieces of >= 256 rows), which fill one window, and summed afterwards.
void wgrad_split(const mok_moe_bwd_args* a, BwdLayout& L) {
  L.ws_kept = -1;
  L.ws_r = L.ws_P = L.ws_plen = 0;
  if (a->n_shared <= 0 || a->T_own < 512) return;
  const int64_t d = a->d, I = a->I, Ish = (int64_t)a->n_shared * a->I_shared;
  const int64_t sh = 2 * cdiv(Ish, GB_M) * cdiv(d, GB_N) +
                     (int64_t)a->n_shared * cdiv(d, GB_M) * cdiv(a->I_shared, GB_N);
  const int64_t total = 3 * (int64_t)a->E_l * cdiv(I, GB_M) * cdiv(d, GB_N) + sh;
  const int64_t r = total % 256;
  if (r == 0 || r > sh) return;
  int64_t P = std::min<int64_t>(256 / r, a->T_own / 256);
  if (P < 2) return;
  const int64_t plen = cdiv(cdiv(a->T_own, P), GB_K) * GB_K;
  P = cdiv(a->T_own, plen);
  if (P < 2) return;
  L.ws_kept = (int)(sh - r);
  L.ws_r = (int)r;
  L.ws_P = (int)P;
  L.ws_plen = (int)plen;
}

int validate_bwd(const mok_moe_bwd_args* a) {
  if (!a) return MOK_EINVAL;
  if (a->dtype != MOK_BF16) return MOK_EUNSUPPORTED;   // the backward runs on bf16 operands
  if (a->d <= 0 || a->E <= 0 || a->E > 1024 || a->k < 1 || a->k > a->E) return MOK_EINVAL;
  if (a->I <= 0 || a->e0 < 0 || a->E_l < 1 || a->e0 + a->E_l > a->E) return MOK_EINVAL;
  if (a->T_pool < 0 || a->tokens_per_rank < 1 || a->T_pool % a->tokens_per_rank) return MOK_EINVAL;
  if (a->T_pool * (int64_t)a->k >= (int64_t)1 << 31) return MOK_EINVAL;
  if (a->own_begin < 0 || a->T_own < 0 || a->own_begin + a->T_own > a->T_pool) return MOK_EINVAL;
  if (a->n_shared < 0 || a->n_shared > 64 || a->route_rows_cap < 0) return MOK_EINVAL;
  if (a->d % 128 || a->I % 64) return MOK_EINVAL;
  if (a->n_shared > 0 && (a->I_shared <= 0 || a->I_shared % 64)) return MOK_EINVAL;
  if (!a->x || !a->topk_idx || !a->topk_w || !a->w_gate || !a->w_up || !a->w_down) return MOK_EINVAL;
  if (!a->dx_slots || !a->dw_gate || !a->dw_up || !a->dw_down) return MOK_EINVAL;
  if (a->n_shared > 0 && (!a->ws_gate || !a->ws_up || !a->ws_down || !a->dws_gate ||
                          !a->dws_up || !a->dws_down))
    return MOK_EINVAL;
  const bool full = a->E_l == a->E;
  if (full) {
    if (!a->dy || a->dy_slots || a->dy_shared || !a->dx || a->own_begin != 0 ||
        (a->n_shared > 0 && a->T_own != a->T_pool))
      return MOK_EINVAL;
  } else {
    if (a->dy || !a->dy_slots || a->dx || (a->n_shared > 0 && a->T_own > 0 && !a->dy_shared))
      return MOK_EINVAL;
  }
  if (a->n_shared > 0 && a->T_own > 0 && !a->dx_shared) return MOK_EINVAL;
  return MOK_OK;
}

BwdLayout layout_bwd(const mok_moe_bwd_args* a) {
  BwdLayout L{};
  const int64_t worst = a->T_pool * (int64_t)std::min(a->k, a->E_l);
  L.cap = a->route_rows_cap > 0 ? std::min<int64_t>(a->route_rows_cap, worst) : worst;
  const int64_t cap = std::max<int64_t>(1, L.cap), d = a->d, I = a->I;
  const int64_t Ish = (int64_t)a->n_shared * a->I_shared, To = std::max(1, a->T_own);
  size_t off = 0;
  auto take = [&](size_t n) { size_t o = off; off = al(off + n); return o; };
  L.counts = take(4 * a->E_l);
  L.offsets = take(4 * (a->E_l + 1));
  L.route_ids = take(4 * std::max<int64_t>(1, worst));
  const int64_t nb = plan_n_blocks(a->T_pool * a->k, a->E_l);
  L.blk_counts = take(4 * nb * a->E_l);
  L.err = take(16);
  L.Ar = take(2 * cap * d); L.dPr = take(2 * cap * d);
  L.dGr = take(2 * cap * I); L.dUr = take(2 * cap * I); L.Hr = take(2 * cap * I);
  L.Dr = take(2 * cap * I);
  L.ldp = (int)(2 * cdiv(2 * I, GB_N));            // one partial per wave's 64 output columns
  L.dwp = take(4 * cap * L.ldp);
  const int64_t Io = std::max<int64_t>(1, Ish);
  L.dGo = take(2 * To * Io); L.dUo = take(2 * To * Io); L.Ho = take(2 * To * Io);
  L.Do = take(2 * To * Io);
  wgrad_split(a, L);
  L.ws_part = take(4 * (size_t)L.ws_r * L.ws_P * GB_M * GB_N);
  L.ws_split = take(sizeof(SplitTile) * (size_t)L.ws_r);
  const int ng = 3 * a->E_l + 2 + a->n_shared + 2;
  L.t_rec = take(gtable_bytes(ng)); L.t_dd = take(gtable_bytes(ng)); L.t_du = take(gtable_bytes(ng));
  L.t_wg = take(gtable_bytes(ng + L.ws_r * L.ws_P));
  L.total = off;
  // upper bounds of each launch's tiles (the device fills in the exact counts)
  const int64_t mt_r = cdiv(cap, GB_M) + a->E_l, mt_o = cdiv(a->T_own, GB_M);
  L.tiles_rec = mt_r * cdiv(2 * I, GB_N) + mt_o * cdiv(2 * Ish, GB_N);
  L.tiles_dd = mt_r * cdiv(I, GB_N) + (int64_t)a->n_shared * mt_o * cdiv(a->I_shared, GB_N);
  L.tiles_du = (mt_r + mt_o) * cdiv(d, GB_N);
  L.tiles_wg = (int64_t)a->E_l * (2 * cdiv(I, GB_M) * cdiv(d, GB_N) + cdiv(d, GB_M) * cdiv(I, GB_N)) +
               2 * cdiv(Ish, GB_M) * cdiv(d, GB_N) +
               (int64_t)a->n_shared * cdiv(d, GB_M) * cdiv(a->I_shared, GB_N) +
               (int64_t)L.ws_r * (L.ws_P - 1);
  return L;
}

}  // namespace

extern "C" {

int mok_moe_backward_workspace_bytes(const mok_moe_bwd_args* a, size_t* bytes) {
  if (!bytes) return MOK_EINVAL;
  const int st = validate_bwd(a);
  if (st != MOK_OK) return st;
  *bytes = layout_bwd(a).total;
  return MOK_OK;
}

int mok_moe_backward(const mok_moe_bwd_args* a, void* stream) {
  const int st = validate_bwd(a);
  if (st != MOK_OK) return st;
  const BwdLayout L = layout_bwd(a);
  if (!a->workspace || a->workspace_bytes < L.total) return MOK_EWORKSPACE;
  if (L.tiles_rec >= INT32_MAX || L.tiles_wg >= INT32_MAX) return MOK_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)a->workspace;
  auto at = [&](size_t o) { return (void*)(ws + o); };
  BwdPass p{};
  p.d = a->d; p.k = a->k; p.I = a->I; p.E_l = a->E_l; p.I_s = a->I_shared;
  p.n_s = a->n_shared; p.T_own = a->n_shared > 0 ? a->T_own : 0; p.cap = L.cap;
  p.counts = (int32_t*)at(L.counts); p.offsets = (int32_t*)at(L.offsets);
  p.route_ids = (int32_t*)at(L.route_ids); p.topk_w = a->topk_w;
  p.wg = (const bf16_t*)a->w_gate; p.wu = (const bf16_t*)a->w_up; p.wd = (const bf16_t*)a->w_down;
  p.sg = (const bf16_t*)a->ws_gate; p.su = (const bf16_t*)a->ws_up; p.sd = (const bf16_t*)a->ws_down;
  const bf16_t* x = (const bf16_t*)a->x;
  p.A_own = x + a->own_begin * a->d;
  p.dP_own = a->dy ? (const bf16_t*)a->dy + a->own_begin * a->d : (const bf16_t*)a->dy_shared;
  p.Ar = (bf16_t*)at(L.Ar); p.dPr = (bf16_t*)at(L.dPr); p.dGr = (bf16_t*)at(L.dGr);
  p.dUr = (bf16_t*)at(L.dUr); p.Hr = (bf16_t*)at(L.Hr);
  p.dGo = (bf16_t*)at(L.dGo); p.dUo = (bf16_t*)at(L.dUo); p.Ho = (bf16_t*)at(L.Ho);
  p.Dr = (bf16_t*)at(L.Dr); p.Do = (bf16_t*)at(L.Do);
  p.dx_slots = (bf16_t*)a->dx_slots; p.dx_shared = (bf16_t*)a->dx_shared;
  p.dwp = (float*)at(L.dwp); p.ldp = L.ldp;
  p.dwg = a->dw_gate; p.dwu = a->dw_up; p.dwd = a->dw_down;
  p.dsg = a->dws_gate; p.dsu = a->dws_up; p.dsd = a->dws_down;
  p.t_rec = (int32_t*)at(L.t_rec); p.t_dd = (int32_t*)at(L.t_dd); p.t_du = (int32_t*)at(L.t_du);
  p.t_wg = (int32_t*)at(L.t_wg);
  p.err = (int32_t*)at(L.err);
  p.ws_kept = L.ws_kept; p.ws_P = L.ws_P; p.ws_plen = L.ws_plen;
  p.ws_part = (float*)at(L.ws_part); p.ws_split = (SplitTile*)at(L.ws_split);
  const int64_t worst = a->T_pool * (int64_t)std::min(a->k, a->E_l);
  // the plan (also yields route_ids for the gathers), then the rows in plan order
  if (launch_plan(a->topk_idx, a->T_pool, a->k, a->e0, a->E_l, a->tokens_per_rank,
                  (int32_t*)p.counts, (int32_t*)p.offsets, nullptr, (int32_t*)p.route_ids,
                  (int32_t*)at(L.blk_counts), std::max<int64_t>(1, worst), s) != hipSuccess)
    return MOK_EHIP;
  launch_k(k_bwd_describe, dim3(1), dim3(BD_THREADS), 0, s, nullptr, nullptr, p);
  // routed x rows and their slot gradients, gathered in plan order (rows past the capacity
  // are not gathered; the description then runs no tile)
  if (a->T_pool > 0) {
    if (launch_pull_gather(a->x, a->d, 2, a->k, p.route_ids, p.offsets, a->E_l, L.cap, p.Ar, s) !=
        hipSuccess)
      return MOK_EHIP;
    // slot r's gradient: dy[r / k] for a whole layer, dy_slots[r] for a share
    if (launch_pull_gather(a->dy ? a->dy : a->dy_slots, a->d, 2, a->dy ? a->k : 1, p.route_ids,
                           p.offsets, a->E_l, L.cap, p.dPr, s) != hipSuccess)
      return MOK_EHIP;
  }
  auto gg = [&](auto kernel, int32_t* table, int64_t tiles) {
    if (tiles <= 0) return;
    const dim3 grid(256), block(GB_NT);          // persistent: one workgroup per CU
    launch_k(kernel, grid, block, 0, s, nullptr, nullptr, table);
  };
  gg(k_ggemm<false, true, false>, p.t_dd, L.tiles_dd);     // D = dP Wd
  gg(k_ggemm<false, false, true>, p.t_rec, L.tiles_rec);   // G, U; SwiGLU backward
  gg(k_ggemm<false, true, false>, p.t_du, L.tiles_du);     // dx = dG Wg + dU Wu
  gg(k_ggemm<true, true, false>, p.t_wg, L.tiles_wg);      // dWg, dWu, dWd (+ shared)
  if (L.ws_r > 0)
    launch_k(k_bwd_split_sum, dim3((unsigned)L.ws_r, GB_M), dim3(256), 0, s, nullptr,
             nullptr, p);
  if (L.cap > 0 && a->dtopk_w)
    launch_k(k_bwd_dtopk, dim3((unsigned)((L.cap + 255) / 256)), dim3(256), 0, s, nullptr, nullptr,
             p, a->dtopk_w);
  if (a->E_l == a->E) {
    if (launch_combine(p.T_own > 0 ? a->dx_shared : nullptr, a->dx_slots, a->dx, a->T_pool, a->k,
                       a->d, false, s) != hipSuccess)
      return MOK_EHIP;
  }
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EHIP;
}

int mok_moe_backward_error(const void* workspace, const mok_moe_bwd_args* a, uint32_t* err,
                           void* stream) {
  if (!workspace || !err) return MOK_EINVAL;
  const int st = validate_bwd(a);
  if (st != MOK_OK) return st;
  const BwdLayout L = layout_bwd(a);
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOK_EHIP;
  int32_t v = 0;
  if (hipMemcpy(&v, (const char*)workspace + L.err, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
    return MOK_EHIP;
  *err = (uint32_t)v;
  return MOK_OK;
}

}  // extern "C"
