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
#include <algorithm>
#include <utility>

#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"
#include "worklist.h"

namespace mok {

size_t worklist_ints(int max_mb, int cap_u, int cap_d, int cap_r) {
  return wl_tab_off(max_mb) + 4 * ((size_t)cap_u + (size_t)cap_d + (size_t)cap_r);
}


// ------------------------------------------------------------------------- GEMM tiles
// Tile geometry. A workgroup of WAVES_M x WAVES_N waves computes a BM x BN block of the
// stage's product; each wave a WM x WN block of 32 x 32 MFMA accumulators (FM x FN). Each K
// step moves ROW_B bytes of every operand row into one of STAGES LDS buffers by LDS-DMA
// (global_load_lds_dwordx4); loader wave w fills A rows [RA w, RA w + RA) and B rows
// [RB w, RB w + RB), RPI rows per instruction.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int ROW_B_, int STAGES_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int ROW_B = ROW_B_, STAGES = STAGES_;
  static constexpr int CH = ROW_B / 16;            // 16-byte chunks per LDS row
  static constexpr int RPI = 64 / CH;              // rows one wave instruction covers
  static constexpr int SWZ_SHIFT = CH == 8 ? 1 : 2;
  static constexpr int RA = BM / NW, RB = BN / NW;
  static constexpr int A_SLABS = RA / RPI, B_SLABS = RB / RPI;
  static_assert(CH == 8 || CH == 4, "64 or 128 bytes per row per K step");
  static_assert(FN % 2 == 0, "gate/up pairing needs an even number of N blocks per wave");
  static_assert(RA % RPI == 0 && RB % RPI == 0, "whole slabs per wave");
  static_assert((WN / 2) % RPI == 0, "a slab holds gate rows or up rows, not both");
  static_assert(STAGES == 2, "two LDS stages: each K step waits for all requests (vmcnt 0)");
};
// Rows of the M tiles of a minibatch (the work list's tiling).
constexpr int TILE_M = 256;
// 256 x 256 tiles, 4 waves of 128 x 128 (16 accumulator blocks = 256 AGPRs per lane), one
// workgroup per CU: each 1 KB LDS operand fragment feeds 4 MFMAs. Two 64 KB K stages of
// 128 bytes per row (whole cache lines), filled by LDS-DMA.
typedef Cfg<256, 256, 2, 2, 128, 2> Big;
// Every element type uses the same tile and K steps of 128 bytes a row: 64 bf16, 128 E4M3 or
// 256 E2M1 elements, i.e. one MX scale word (4 blocks of 32) a row and step for MXFP8, two for
// MXFP4.
template <Elem EL> struct CfgOf { typedef Big type; };
template <Elem EL> constexpr int scale_words() { return EL == Elem::FP4 ? 2 : 1; }

// Per element type: bytes per two elements (KB2), the MFMA's K per instruction (MK) and the 16-
// byte chunks a lane feeds one MFMA (CPL).
template <Elem EL> struct Tr;
template <> struct Tr<Elem::BF16> { static constexpr int KB2 = 4, MK = 16, CPL = 1; };
template <> struct Tr<Elem::F32> { static constexpr int KB2 = 8, MK = 16, CPL = 2; };
template <> struct Tr<Elem::FP8> { static constexpr int KB2 = 2, MK = 64, CPL = 2; };
template <> struct Tr<Elem::FP4> { static constexpr int KB2 = 1, MK = 64, CPL = 1; };
// Bytes of n elements along K (n even).
template <Elem EL> MOK_HOSTDEV constexpr int64_t nbytes(int64_t n) { return n * Tr<EL>::KB2 / 2; }
// Operands in an MX format (E8M0 block scales; quantised on the device).
template <Elem EL> constexpr bool is_mx() { return EL == Elem::FP8 || EL == Elem::FP4; }

// LDS: STAGES buffers of the A and B tiles (ROW_B per row per K step), their MX scale words and
// the down stage's row table. Logical 16-byte chunk c of row r sits at slot
// c ^ ((r >> SWZ_SHIFT) & (CH - 1)): 16 consecutive rows read at one logical chunk then hit
// 16 distinct groups of the 64 banks. The buffers are separate LDS objects, so the compiler
// can see that accesses to one do not touch another.
template <class C>
struct Bufs {
  uint4 (*A)[C::CH];
  uint4 (*B)[C::CH];
  uint32_t* As;
  uint32_t* Bs;
};
template <class C>
struct Lds {
  Bufs<C> buf[C::STAGES];
  int32_t* row_dst;
  float* row_w;
};

// Buffer i (a run-time index), chosen with selects: indexing the pointer array itself at run
// time would place it in private (scratch) memory.
template <class C>
MOK_DEV Bufs<C> pick(const Lds<C>& sm, int i) {
  Bufs<C> r = sm.buf[0];
#pragma unroll
  for (int q = 1; q < C::STAGES; ++q)
    if (i == q) {
      r.A = sm.buf[q].A; r.B = sm.buf[q].B; r.As = sm.buf[q].As; r.Bs = sm.buf[q].Bs;
    }
  return r;
}

// 16-byte chunk that lane half h feeds to the MFMA of K sub-step s (16 or 64 elements).
//  bf16 32x32x16: one chunk, k = 16s + 8h + [0, 8).
//  fp32 32x32x2 (x8): two chunks, k = 16s + 8h + [0, 8).
//  fp8 32x32x64 (scaled): bytes 0-15 of a lane belong to the MFMA's first 32-wide K block and
//  bytes 16-31 to the second, each lane half taking 16 of a block's 32 k; the E8M0 scale of
//  lane l covers (row l % 32, block l / 32). So: chunks 4s + h and 4s + 2 + h.
//  fp4 32x32x64 (scaled): a lane's 16 bytes are the 32 consecutive k of block l / 32 (a probe
//  of the instruction with exact small inputs and per-block scales matched only this layout),
//  and its E8M0 scale covers that block: chunk 2s + h of the 64-byte K step.
template <Elem EL>
MOK_DEV constexpr int frag_chunk(int s, int h, int q) {
  return EL == Elem::BF16 ? 2 * s + h
       : EL == Elem::F32 ? 4 * s + 2 * h + q
       : EL == Elem::FP4 ? 2 * s + h : 4 * s + 2 * q + h;
}

// The weight fragment is the MFMA's first operand and the token-row fragment its second, so
// each accumulator block holds the transposed product: lane (h, l32) of block (i, j) carries
// output row 32i + l32 and output columns 32j + 8g + 4h + [0, 4) in values 4g .. 4g + 3 --
// four consecutive columns of one row per register quad, which the epilogues store whole.
// MXFP8: asc / bsc hold scale words; byte SCB of each is the MFMA's E8M0 scale (op_sel).
template <Elem EL, int FM, int FN, int SCB = 0, class After>
MOK_DEV void mfma_step(const uint4 (&a)[FM][2], const uint4 (&b)[FN][2], const uint32_t* asc,
                       const uint32_t* bsc, f32x16_t (&acc)[FM][FN], After&& after) {
  if constexpr (EL == Elem::BF16) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, b[j][0]), __builtin_bit_cast(bf16x8_t, a[i][0]),
            acc[i][j], 0, 0, 0);
        after(i * FN + j);
      }
  } else if constexpr (EL == Elem::F32) {
    // Lane half h supplies k = 8h + q of a 16-wide K step to the q-th 32x32x2 product; A and
    // B use the same assignment, so the 8 products cover the step exactly once.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const float* av = reinterpret_cast<const float*>(&a[i][0]);
        const float* bv = reinterpret_cast<const float*>(&b[j][0]);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[q], av[q], acc[i][j], 0, 0, 0);
        after(i * FN + j);
      }
  } else if constexpr (EL == Elem::FP4) {
    // operand format 4 (E2M1) for both; the instruction reads the first four registers
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        i32x8_t av = {0, 0, 0, 0, 0, 0, 0, 0}, bv = av;
        av[0] = a[i][0].x; av[1] = a[i][0].y; av[2] = a[i][0].z; av[3] = a[i][0].w;
        bv[0] = b[j][0].x; bv[1] = b[j][0].y; bv[2] = b[j][0].z; bv[3] = b[j][0].w;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bv, av, acc[i][j], 4, 4, SCB, (int)bsc[j], SCB, (int)asc[i]);
        after(i * FN + j);
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        i32x8_t av, bv;
        av[0] = a[i][0].x; av[1] = a[i][0].y; av[2] = a[i][0].z; av[3] = a[i][0].w;
        av[4] = a[i][1].x; av[5] = a[i][1].y; av[6] = a[i][1].z; av[7] = a[i][1].w;
        bv[0] = b[j][0].x; bv[1] = b[j][0].y; bv[2] = b[j][0].z; bv[3] = b[j][0].w;
        bv[4] = b[j][1].x; bv[5] = b[j][1].y; bv[6] = b[j][1].z; bv[7] = b[j][1].w;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bv, av, acc[i][j], 0, 0, SCB, (int)bsc[j], SCB, (int)asc[i]);
        after(i * FN + j);
      }
  }
}

// One tile of the up (UP = true) or down (UP = false) stage of minibatch m.
//  up:   the minibatch's rows x (gate, up rows of H columns n0 .. n0 + BN/2) -> H
//  down: the minibatch's H rows x (W_down rows n0 .. n0 + BN) -> output columns
// The tile is M tile mt (rows [TILE_M mt, ...) of the minibatch) and N tile nt of the entry;
// C::BM >= its valid rows. Loader wave w fills rows [RA w, RA w + RA) of the A tile and
// [RB w, RB w + RB) of the B tile, RPI rows per instruction; lane L carries row RPI*q + L / CH
// of slab q, LDS slot L % CH, so it fetches global chunk (L % CH) ^ swz(row) and the swizzle
// costs nothing. Row addresses are a uniform base plus a 32-bit offset. M and N tails:
// rows/columns past the end are clamped on load, skipped on store.
// Pool rows of the A-operand slabs of tile `entry` for the calling lane (gate/up stage, bf16 or
// float32, routed minibatch): the route ids it loads (divided by k at the use). Issued one tile
// ahead, so that a tile's first DMA does not wait on this dependent load.
template <Elem EL, bool UP, class C>
MOK_DEV void prefetch_a_rows(const ExpertPass& p, const int4 entry, int32_t (&route)[C::A_SLABS]) {
  if constexpr (UP && !is_mx<EL>()) {
    const int local = uniform(entry.y) & ((1 << KIND_SHIFT) - 1), row0 = uniform(entry.z);
    const int g = uniform(entry.w >> 16), rows = uniform(entry.w & 0xFFFF);
    const int n_mt = (rows + TILE_M - 1) / TILE_M;
    const int m0 = (local % n_mt) * TILE_M, rows_valid = min(C::BM, rows - m0);
    const int tid = opaque(threadIdx.x), lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int q = 0; q < C::A_SLABS; ++q) {
      const int r = min(C::RA * wid + C::RPI * q + lane / C::CH, rows_valid - 1);
      route[q] = g < p.E_l ? p.route_ids[row0 + m0 + r] : 0;
    }
  }
}

// Field of the kernel's argument block (an ExpertPass, the kernel's only parameter) at byte
// offset off, read again from the kernarg segment with a scalar load at each call: a value
// used by the K loop but loaded once per kernel would be held in registers across every
// epilogue, where the register file is full.
template <class T>
MOK_DEV T kernarg_field(size_t off) {
  typedef __attribute__((address_space(4))) const char kchar;
  kchar* base = (kchar*)__builtin_amdgcn_kernarg_segment_ptr();
  return *(__attribute__((address_space(4))) const volatile T*)(base + off);
}

// The pool rows of the route ids prefetch_a_rows loaded (route id / k). k is read from the
// kernarg segment here, so the division's reciprocal is not hoisted out of a tile loop and
// held (or spilled) across the tiles.
template <class C>
MOK_DEV void route_rows(const ExpertPass& p, int32_t (&r)[C::A_SLABS]) {
  const int k = kernarg_field<int>(offsetof(ExpertPass, k));
#pragma unroll
  for (int q = 0; q < C::A_SLABS; ++q) r[q] /= k;
}

// One tile. slot: the ring slot of the entry's minibatch. pre (routed gate/up tiles of the
// bf16 / float32 path): the pool rows of the tile's A slabs (prefetch_a_rows, route_rows).
// after_step(s) runs after the barrier of K steps s = 0 .. 3 (for shorter K loops, the missing
// ones run after the loop): there every vector load issued before the step's DMA has landed;
// after_step(-1) runs before the tile's first DMA. The stage kernel fetches the next tile's
// entry there (a scalar load, which the first barrier waits for with the DMA), and its slot and
// A rows over steps 1 .. 2, and parks the rows in LDS, so they hold no register across the K
// loop; the ring loop fetches its next item over steps 0 .. 3.
template <Elem EL, bool UP, bool F32OUT, class C, bool RING = false, class F>
MOK_DEV void run_tile(const ExpertPass& p, const Lds<C>& sm, const int4 entry, const int slot,
                      const int32_t (&pre)[C::A_SLABS], F&& after_step) {
  // A operands written during this launch (ring loop): H (down) and the MXFP8 A rows (up)
  constexpr bool MXE = is_mx<EL>();
  constexpr bool A_L2C = RING && (!UP || MXE);
  typedef Tr<EL> TR;
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, FM = C::FM, FN = C::FN;
  constexpr int A_SLABS = C::A_SLABS, B_SLABS = C::B_SLABS, ST = C::STAGES, CH = C::CH;
  constexpr int RPI = C::RPI, SWS = C::SWZ_SHIFT, RA = C::RA, RB = C::RB;
  static_assert(!MXE || (RA == 64 && RB == 64),
                "MX scales: lane L of loader wave w carries tile row 64 w + L");
  constexpr int KT = C::ROW_B * 2 / TR::KB2;       // elements per K step
  constexpr int SUB = KT / TR::MK;                 // MFMA sub-steps per K step
  constexpr int SC_B = KT / 32;                    // MX scale bytes per row per K step
  // LDS-DMA instructions one wave issues per K step
  constexpr int SCW = scale_words<EL>();           // MX scale words per row and K step
  constexpr int DMA_PER_STEP = A_SLABS + B_SLABS + (MXE ? 2 * SCW : 0);
  // K-loop barrier placement: before the last sub-step of the previous step (bf16, float32),
  // or at the start of the step (MXFP8)
  constexpr bool EARLY_X = !MXE;
  const int m = uniform(entry.x), local = uniform(entry.y);
  const int row0 = uniform(entry.z);
  const int g = uniform(entry.w >> 16), rows = uniform(entry.w & 0xFFFF);
  const bool shared = g >= p.E_l;
  const int64_t ring_row0 = (int64_t)slot * p.mb;
  const int n_mt = (rows + TILE_M - 1) / TILE_M;
  const int mt = local % n_mt, nt = local / n_mt;
  const int m0 = mt * TILE_M;
  const int rows_valid = min(BM, rows - m0);
  // The thread index is made opaque here and again before the epilogue: values derived from it
  // are then computed per tile and per phase instead of being hoisted out of the tile loop,
  // where they would live across the K loop, be spilled to scratch and be reloaded with a
  // vmcnt(0) wait that also drains the epilogue's stores.
  const int tid = opaque(threadIdx.x), lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / C::WAVES_N, wn = wid % C::WAVES_N;
  auto blk_row = [&](int i) { return wm * WM + 32 * i; };   // first tile row of block row i
  // K from the kernarg segment per tile: hoisted out of the tile loop, its "nk > 0" and
  // "nk > 1" flags were spilled to scratch, and their reload's wait held the first DMA back
  // until the previous epilogue's stores had drained
  const int K = UP ? kernarg_field<int>(offsetof(ExpertPass, d))
                 : (shared ? kernarg_field<int>(offsetof(ExpertPass, I_sh)) : kernarg_field<int>(offsetof(ExpertPass, I)));
  const int N = UP ? (shared ? p.I_sh : p.I) : p.d;   // output columns of the stage
  const int nk = K / KT;
  // global byte of lane L's chunk in slab q: slot L % CH of row RPI*q + L / CH (+ RA or RB * w)
  auto chunk_b = [&](int q) {
    const int row = RPI * q + lane / CH;
    return ((lane % CH) ^ ((row >> SWS) & (CH - 1))) * 16;
  };

  // ---- A operand: uniform base + per-slab 32-bit row offsets
  const char* a_base;
  int64_t a_row_bytes;
  if (UP && !MXE) {
    a_base = (const char*)kernarg_field<const void*>(offsetof(ExpertPass, x));
    a_row_bytes = nbytes<EL>(p.d);
  } else if (UP) {
    a_base = (const char*)p.A_codes + (ring_row0 + m0) * nbytes<EL>(p.d);
    a_row_bytes = nbytes<EL>(p.d);
  } else {
    a_base = (const char*)p.H + (ring_row0 + m0) * nbytes<EL>(p.Hld);
    a_row_bytes = nbytes<EL>(p.Hld);
  }
  a_base = uniform_ptr(a_base);
  uint32_t a_off[A_SLABS];
#pragma unroll
  for (int q = 0; q < A_SLABS; ++q) {
    const int r = min(RA * wid + RPI * q + lane / CH, rows_valid - 1);
    int64_t row;
    if (UP && !MXE)
      row = shared ? p.own_begin + row0 + m0 + r : (int64_t)pre[q];
    else
      row = r;
    a_off[q] = (uint32_t)(row * a_row_bytes) + chunk_b(q);
  }
  // ---- B operand. Up: B tile row R belongs to compute wave R / WN, whose WN rows are WN/2
  // gate rows then the WN/2 up rows of the same H columns nt*BN/2 + (R / WN)*WN/2 + [0, WN/2):
  // each accumulator block of gate then pairs with the block FN/2 further holding up. A slab
  // lies wholly in the gate or the up half (b_up_slab). Down: W_down rows nt*BN + R.
  const char* b_base;              // down: W_down (segment 0); up: gate rows
  const char* b_up = nullptr;      // up: up rows
  int64_t b_row_bytes, b_seg_len = K, b_seg_stride = 0;
  auto b_up_slab = [&](int q) { return ((RB * wid + RPI * q) % WN) >= WN / 2; };
  if (UP) {
    const int64_t e_off = shared ? 0 : (int64_t)g * p.I * nbytes<EL>(p.d);
    b_base = (const char*)(shared ? p.sg : p.wg) + e_off;
    b_up = uniform_ptr((const char*)(shared ? p.su : p.wu) + e_off);
    b_row_bytes = nbytes<EL>(p.d);
  } else {
    if (shared) {
      b_base = (const char*)p.sd;
      b_row_bytes = nbytes<EL>(p.I_seg);
      b_seg_len = p.I_seg;
      b_seg_stride = (int64_t)p.d * nbytes<EL>(p.I_seg);
    } else {
      b_base = (const char*)p.wd + (int64_t)g * p.d * nbytes<EL>(p.I);
      b_row_bytes = nbytes<EL>(p.I);
    }
  }
  b_base = uniform_ptr(b_base);
  // first B row (weight row) of slab q's lanes, lane offset excluded
  auto b_row0 = [&](int q) {
    const int R = RB * wid + RPI * q;
    return UP ? nt * (BN / 2) + (R / WN) * (WN / 2) + (R % (WN / 2)) : nt * BN + R;
  };
  uint32_t b_off[B_SLABS];
#pragma unroll
  for (int q = 0; q < B_SLABS; ++q) {
    const int n = min(b_row0(q) + lane / CH, N - 1);
    b_off[q] = (uint32_t)(n * b_row_bytes) + chunk_b(q);
  }
  // ---- MX scales: lane L of wave w carries tile row 64w + L. A K step needs the 4 scale bytes
  // of a row, one word of the K-step-major layout (mx_kmajor_scale): the step's words of
  // consecutive rows are contiguous, so a wave's scale load reads 256 consecutive bytes.
  const uint8_t* a_sc_base = nullptr;
  const uint8_t* b_sc_base = nullptr;
  uint32_t a_sc_off = 0, b_sc_off = 0;
  int64_t a_sc_R = 0, b_sc_R = 0;                    // rows of the scale matrices
  if (MXE) {
    const int r = min(RA * wid + lane, rows_valid - 1);
    a_sc_R = (int64_t)p.n_slots * p.mb;              // A rows and H: the ring rows
    a_sc_base = (UP ? p.A_sc : p.H_sc) + (ring_row0 + m0) * 4;
    a_sc_off = (uint32_t)(r * 4);
    if (UP) {
      const bool uph = b_up_slab(0);               // the wave's 64 rows are all gate or all up
      const uint8_t* S = shared ? (uph ? p.su_sc : p.sg_sc) : (uph ? p.wu_sc : p.wg_sc);
      b_sc_R = shared ? p.I_sh : p.I;
      b_sc_base = S + (shared ? 0 : (int64_t)g * p.I * (p.d / 32));
    } else {
      b_sc_R = p.d;
      b_sc_base = shared ? p.sd_sc : p.wd_sc + (int64_t)g * p.d * (p.I / 32);
    }
    const int n = min(b_row0(0) + lane, N - 1);
    b_sc_off = (uint32_t)(n * 4);
    a_sc_base = uniform_ptr(a_sc_base);
    b_sc_base = uniform_ptr(b_sc_base);
  }
  // epilogue row table (down stage): destination row and routing weight of tile row tid. The
  // route id is loaded here and written to LDS after the first K step's barrier (by then every
  // wave is done with the previous tile's epilogue, and the load, older than that step's DMA,
  // has landed); its weight is loaded then and written after the K loop. Neither load holds up
  // the K loop.
  const bool rt_lane = !UP && tid < BM && tid < rows_valid;
  int32_t rt_dst = 0;
  float rt_w = 1.0f;
  if (rt_lane) rt_dst = shared ? row0 + m0 + tid : p.route_ids[row0 + m0 + tid];
  auto at_step0 = [&]() {
    if (rt_lane) {
      sm.row_dst[tid] = rt_dst;
      if (!shared) rt_w = p.topk_w[rt_dst];
    }
    after_step(0);
  };

  // address pieces of K step kt
  // Uniform base addresses of K step kt's operand rows (A, B, and for the gate/up stage the up
  // rows of B) and MX scale words. The step's K offset rides on these scalar bases, so the
  // per-lane offsets of the DMA instructions stay fixed over the K loop and no vector register
  // or instruction is spent on addresses per step.
  struct StepAddr { const char *a, *b, *bu; const uint8_t *sa, *sb; };
  auto step_addr = [&](int kt) {
    StepAddr s;
    const uint32_t k0 = (uint32_t)kt * KT;
    const uint32_t seg = k0 / (uint32_t)b_seg_len;
    const uint32_t kin = k0 - seg * (uint32_t)b_seg_len;
    s.a = uniform_ptr(a_base + nbytes<EL>(k0));
    s.b = uniform_ptr(b_base + (int64_t)seg * b_seg_stride + nbytes<EL>(kin));
    s.bu = UP ? uniform_ptr(b_up + nbytes<EL>(kin)) : nullptr;
    if (MXE) {                                       // one scale word per 128 elements of K
      // a shared down segment's scales: d rows x I_seg / 32 bytes per shared expert
      s.sa = uniform_ptr(a_sc_base + (int64_t)(k0 / 128) * a_sc_R * 4);
      s.sb = uniform_ptr(b_sc_base + (int64_t)seg * p.d * (p.I_seg / 32) +
                         (int64_t)(kin / 128) * b_sc_R * 4);
    } else {
      s.sa = s.sb = nullptr;
    }
    return s;
  };
  // LDS-DMA instruction q of K step kt into buffer b (A slabs, B slabs, then the MX scale words).
  auto issue_one = [&](const StepAddr& s, const Bufs<C>& b, int q) {
    __builtin_amdgcn_sched_barrier(0);             // keeps the DMA between its two MFMAs
    if (q < A_SLABS) {
      dma_b128<A_L2C>(s.a, a_off[q], uniform(lds_addr(&b.A[RA * wid][0])) + 1024 * q);
    } else if (q < A_SLABS + B_SLABS) {
      const int r = q - A_SLABS;
      const char* bb = (UP && b_up_slab(r)) ? s.bu : s.b;
      dma_b128(bb, b_off[r], uniform(lds_addr(&b.B[RB * wid][0])) + 1024 * r);
    } else {
      // scale words: A word 0, B word 0 (, A word 1, B word 1); word w of the step is the
      // K-step-major word of 128-element step (k0 / 128 + w), R rows further on
      const int t = q - A_SLABS - B_SLABS, w = t >> 1;
      if ((t & 1) == 0)
        dma_b32<A_L2C>(s.sa + (int64_t)w * a_sc_R * 4, a_sc_off,
                       uniform(lds_addr(&b.As[w * BM + 64 * wid])));
      else
        dma_b32(s.sb + (int64_t)w * b_sc_R * 4, b_sc_off,
                uniform(lds_addr(&b.Bs[w * BN + 64 * wid])));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // A step's DMA is spread over 2 MPS MFMA slots, about one instruction per two MFMAs: slot
  // sigma(q) = q * 2 MPS / DMA_PER_STEP. Slots [0, MPS) are the last sub-step of the
  // step two before it, slots [MPS, 2 MPS) the first sub-step of the step before it.
  constexpr int MPS = FM * FN;                      // MFMAs per sub-step and wave
  static_assert(SUB >= 2 && SUB % 2 == 0, "the last sub-step uses fragment slot 1");
  auto issue_slot = [&](const StepAddr& s, const Bufs<C>& b, int slot) {
#pragma unroll
    for (int q = 0; q < DMA_PER_STEP; ++q)
      if (q * 2 * MPS / DMA_PER_STEP == slot) issue_one(s, b, q);
  };
  f32x16_t acc[FM][FN];                             // cleared once the first DMA is out

  const int h = lane >> 5, l32 = lane & 31;
  const int xsw = (l32 >> SWS) & (CH - 1);         // swizzle of the lane's fragment rows
  // Fragments, double-buffered across the K sub-steps (slot s & 1 for sub-step s): the reads of
  // sub-step s + 1 are issued before the MFMAs of s, and the reads of the next step's sub-step
  // 0 before the MFMAs of this step's last sub-step. Scheduling barriers pin that order (left
  // alone the scheduler sinks each read to just before its first use, and every sub-step waits
  // on LDS latency).
  uint4 fa[2][FM][2], fb[2][FN][2];
  uint32_t asc[2][FM], bsc[2][FN];
  auto load = [&](const Bufs<C>& b, int kt, int s, int f) {
    const char* a_buf = (const char*)&b.A[blk_row(0) + l32][0];
    const char* b_buf = (const char*)&b.B[wn * WN + l32][0];
    const int sc_shift = 8 * (((uint32_t)kt * SC_B) & 3);
    const int c0 = ((frag_chunk<EL>(s, h, 0)) ^ xsw) * 16;
    const int c1 = ((frag_chunk<EL>(s, h, 1)) ^ xsw) * 16;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      fa[f][i][0] = *(const uint4*)(a_buf + i * 32 * C::ROW_B + c0);
      if (TR::CPL == 2) fa[f][i][1] = *(const uint4*)(a_buf + i * 32 * C::ROW_B + c1);
      if (MXE)
        asc[f][i] = (b.As[blk_row(i) + l32] >> (sc_shift + 8 * (2 * s + h))) & 0xFFu;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      fb[f][j][0] = *(const uint4*)(b_buf + j * 32 * C::ROW_B + c0);
      if (TR::CPL == 2) fb[f][j][1] = *(const uint4*)(b_buf + j * 32 * C::ROW_B + c1);
      if (MXE)
        bsc[f][j] = (b.Bs[wn * WN + j * 32 + l32] >> (sc_shift + 8 * (2 * s + h))) & 0xFFu;
    }
  };
  // MFMAs of sub-steps 0 .. SUB - 2 of step kt from buffer b (sub-step 0's fragments already
  // read); after(n) runs after MFMA n of sub-step 0 (the DMA slots there).
  auto phase_b = [&](const Bufs<C>& b, int kt, auto&& after) {
#pragma unroll
    for (int s = 0; s + 1 < SUB; ++s) {
      load(b, kt, s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);   // the reads of s + 1 go out before the MFMAs of s
      mfma_step<EL, FM, FN>(fa[s & 1], fb[s & 1], asc[s & 1], bsc[s & 1], acc,
                            [&](int n) { if (s == 0) after(n); });
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // MFMAs of the last sub-step (fragments in slot 1); after(n) after MFMA n.
  auto phase_e = [&](auto&& after) {
    mfma_step<EL, FM, FN>(fa[1], fb[1], asc[1], bsc[1], acc, [&](int n) { after(n); });
    __builtin_amdgcn_sched_barrier(0);
  };
  // Barrier X(kt) of K step kt: every wave's DMA of step kt has landed, and every wave has its
  // reads of step kt - 1 back (so that buffer may be refilled). It sits before the last
  // sub-step of step kt - 1, whose fragments are already in registers.
  auto barrier_x = [&]() {
    __builtin_amdgcn_s_waitcnt(0x70);   // vmcnt(0) lgkmcnt(0) (gfx9 encoding, expcnt left at 7)
    lds_barrier();
  };

  // Late-barrier K loop (MXFP8: its fragments and scales leave no registers for the early
  // barrier's overlap). issue_at(kt, b, n) issues the DMA instructions of step kt that belong
  // after MFMA n of the current step (q * SPAN / DMA_PER_STEP == n), spread over the step's
  // first half (spread over all of it, the last ones land too late: MXFP8 EP64 share gate/up
  // 1.16 ms against 1.13).
  constexpr int N_MFMA = SUB * FM * FN;             // MFMAs per K step and wave
  constexpr int SPAN = N_MFMA / 2;                  // the first half of the step
  auto issue_at = [&](const StepAddr& s, const Bufs<C>& b, int n) {
#pragma unroll
    for (int q = 0; q < DMA_PER_STEP; ++q)
      if ((SPAN == 0 ? -1 : q * SPAN / DMA_PER_STEP) == n) issue_one(s, b, q);
  };
  auto issue_all = [&](int kt, const Bufs<C>& b) {
    const StepAddr s = step_addr(kt);
#pragma unroll
    for (int q = 0; q < DMA_PER_STEP; ++q) issue_one(s, b, q);
  };
  // MFMAs of one K step from buffer b (kt: the step, for the MX scale byte position).
  // Fragments are double-buffered across the K sub-steps: the reads of sub-step s + 1 are
  // issued before the MFMAs of s (scheduling barriers pin that order; left alone the scheduler
  // sinks each read to just before its first use and every sub-step waits on LDS latency).
  // after(n) runs after MFMA n of the step (n = -1: after the first reads, before any MFMA):
  // the K loop issues the next step's LDS-DMA there, a few instructions at a time, so that no
  // MFMA waits behind a burst of memory instructions.
  auto compute = [&](const Bufs<C>& b, int kt, auto&& after) {
    const char* a_buf = (const char*)&b.A[blk_row(0) + l32][0];
    const char* b_buf = (const char*)&b.B[wn * WN + l32][0];
    uint4 fa[2][FM][2], fb[2][FN][2];
    // MX scale bytes of the lane's blocks, one register per row block, read once per step.
    // MXFP8 (one word of 4 blocks a row and step): the word shifted right by 8 h, so byte 2 s
    // holds block 2 s + h of sub-step s. MXFP4 (two words a step): a byte permute packs the
    // bytes h and 2 + h of both words, so byte sc_byte(s) holds block 2 s + h.
    uint32_t asc[FM], bsc[FN];
    const uint32_t perm_sel = 0x06020400u + 0x01010101u * h;
    // Reads in the order the MFMAs (row-block major) first use them: scale words, A block 0,
    // the B blocks, the other A blocks. The LDS counter tracks at most 15 reads, so a read
    // that an MFMA waits for must be among the first of those in flight.
    auto load = [&](int s, int f) {
      const int c0 = ((frag_chunk<EL>(s, h, 0)) ^ xsw) * 16;
      const int c1 = ((frag_chunk<EL>(s, h, 1)) ^ xsw) * 16;
      if (MXE && s == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = blk_row(i) + l32;
          asc[i] = SCW == 1 ? b.As[r] >> (8 * h)
                            : __builtin_amdgcn_perm(b.As[BM + r], b.As[r], perm_sel);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wn * WN + j * 32 + l32;
          bsc[j] = SCW == 1 ? b.Bs[r] >> (8 * h)
                            : __builtin_amdgcn_perm(b.Bs[BN + r], b.Bs[r], perm_sel);
        }
      }
      auto ra = [&](int i) {
        fa[f][i][0] = *(const uint4*)(a_buf + i * 32 * C::ROW_B + c0);
        if (TR::CPL == 2) fa[f][i][1] = *(const uint4*)(a_buf + i * 32 * C::ROW_B + c1);
      };
      ra(0);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        fb[f][j][0] = *(const uint4*)(b_buf + j * 32 * C::ROW_B + c0);
        if (TR::CPL == 2) fb[f][j][1] = *(const uint4*)(b_buf + j * 32 * C::ROW_B + c1);
      }
#pragma unroll
      for (int i = 1; i < FM; ++i) ra(i);
    };
    static_assert(!MXE || (SUB == 2 * SCW && SC_B == 4 * SCW), "one scale word per 128 elements");
    load(0, 0);
    // The reads of sub-step s + 1 go out after the first NEXT_AT MFMAs of s: issued before
    // them, they would sit ahead of s's own reads in the LDS counter, and the first MFMA would
    // wait for most of both sub-steps' reads (scheduling barriers pin the order).
    constexpr int NEXT_AT = 8;
    auto sub = [&](auto S_) {
      constexpr int s = decltype(S_)::value;
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0) after(-1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_step<EL, FM, FN, SCW == 1 ? 2 * s : 2 * (s & 1) + (s >> 1)>(
          fa[s & 1], fb[s & 1], asc, bsc, acc, [&](int n) {
        if (s + 1 < SUB && n == NEXT_AT - 1) {
          __builtin_amdgcn_sched_barrier(0);
          load(s + 1, (s + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        after(s * FM * FN + n);
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(SUB <= 4, "sub-steps unrolled below");
    sub(std::integral_constant<int, 0>{});
    if constexpr (SUB > 1) sub(std::integral_constant<int, 1>{});
    if constexpr (SUB > 2) sub(std::integral_constant<int, 2>{});
    if constexpr (SUB > 3) sub(std::integral_constant<int, 3>{});
  };

  if constexpr (EARLY_X) {
    // K loop over two buffers. Step kt: B phase (sub-steps 0 .. SUB - 2 from buffer kt % 2,
    // finishing the DMA of step kt + 1), then X(kt + 1), the reads of step kt + 1's sub-step 0,
    // and the E phase (the last sub-step of kt, starting the DMA of step kt + 2 into the buffer
    // kt just released). The steady state is unrolled by 2 so every buffer's role is static.
    after_step(-1);
    if (nk > 0) {
#pragma unroll
      for (int q = 0; q < DMA_PER_STEP; ++q) issue_one(step_addr(0), sm.buf[0], q);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    barrier_x();                                    // X(0)
    at_step0();
    if (nk > 1) {
      const StepAddr s1 = step_addr(1);
#pragma unroll
      for (int slot = 0; slot < MPS; ++slot) issue_slot(s1, sm.buf[1], slot);
    }
    if (nk > 0) load(sm.buf[0], 0, 0, 0);
    auto steady = [&](int kt, const Bufs<C>& cur, const Bufs<C>& nxt) {
      const StepAddr s1 = step_addr(kt + 1);
      phase_b(cur, kt, [&](int n) { issue_slot(s1, nxt, MPS + n); });
      barrier_x();                                  // X(kt + 1)
      if (kt + 1 < 4) after_step(kt + 1);
      load(nxt, kt + 1, 0, 0);
      const StepAddr s2 = step_addr(kt + 2);
      phase_e([&](int n) { issue_slot(s2, cur, n); });
    };
    int kt = 0;
    for (; kt + 4 <= nk; kt += 2) {
      steady(kt, sm.buf[0], sm.buf[1]);
      steady(kt + 1, sm.buf[1], sm.buf[0]);
    }
    for (; kt < nk; ++kt) {     // the last steps, buffers chosen at run time
      const bool has1 = kt + 1 < nk, has2 = kt + 2 < nk;
      const Bufs<C> cur = pick(sm, kt & 1), nxt = pick(sm, (kt + 1) & 1);
      const StepAddr s1 = step_addr(has1 ? kt + 1 : kt);
      phase_b(cur, kt, [&](int n) { if (has1) issue_slot(s1, nxt, MPS + n); });
      if (has1) {
        barrier_x();
        if (kt + 1 < 4) after_step(kt + 1);
        load(nxt, kt + 1, 0, 0);
      }
      const StepAddr s2 = step_addr(has2 ? kt + 2 : kt);
      phase_e([&](int n) { if (has2) issue_slot(s2, cur, n); });
    }
  } else {
    // K loop over a ring of ST buffers. Step kt: wait until this wave's DMA of kt has landed
    // (later steps' DMAs stay in flight), barrier (every wave's DMA of kt landed; every wave
    // done computing kt - 1), issue step kt + ST - 1 into the buffer kt - 1 used, compute kt.
    // The steady state is unrolled by ST so every buffer's role is static.
    after_step(-1);
#pragma unroll
    for (int q = 0; q < ST - 1; ++q)
      if (q < nk) issue_all(q, sm.buf[q]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    auto steady = [&](int kt, const Bufs<C>& cur, const Bufs<C>& nxt) {
      wait_vmcnt<(ST - 2) * DMA_PER_STEP>();
      lds_barrier();
      if (kt == 0) at_step0();
      else if (kt < 4) after_step(kt);
      const StepAddr sa = step_addr(kt + ST - 1);
      compute(cur, kt, [&](int n) { issue_at(sa, nxt, n); });
    };
    int kt = 0;
    for (; kt + 2 * ST - 1 <= nk; kt += ST) {
#pragma unroll
      for (int q = 0; q < ST; ++q) steady(kt + q, sm.buf[q], sm.buf[(q + ST - 1) % ST]);
    }
    for (; kt < nk; ++kt) {     // the last steps, buffers chosen at run time
      wait_vmcnt<0>();
      lds_barrier();
      if (kt == 0) at_step0();
      else if (kt < 4) after_step(kt);
      const bool more = kt + ST - 1 < nk;
      const Bufs<C> cur = pick(sm, kt % ST), nxt = pick(sm, (kt + ST - 1) % ST);
      const StepAddr sa = step_addr(more ? kt + ST - 1 : kt);
      compute(cur, kt, [&](int n) {
        if (more) issue_at(sa, nxt, n);
      });
    }
  }

  // ---- epilogue. Value 4g + r of block (i, j) is (row 32i + l32, column 32j + 8g + 4h + r) of
  // the wave's block (see mfma_step). One barrier: every wave is past the K loop (both operand
  // buffers are free) and the row table is complete. There is none at the end: the staging
  // uses buffer 1 only, the next tile's first DMA fills buffer 0, and that tile writes buffer 1
  // and the row table only after its first K step's barrier, which every wave reaches after
  // its epilogue.
  for (int s = max(nk, 1); s < 4; ++s) after_step(s);
  if (rt_lane) sm.row_w[tid] = rt_w;
  __syncthreads();
  {
  const int lane = opaque(threadIdx.x) & 63, h = lane >> 5, l32 = lane & 31;
  auto r_of = [&](int i) { return blk_row(i) + l32; };   // tile row of the lane in block row i
  if constexpr (!F32OUT) {
    // bf16 (or MXFP8 H) outputs: each wave stages 32 rows at a time through its own LDS region
    // (the operand buffers are free once every wave is past the K loop), four columns per
    // write, then stores whole row segments: H rows of the ring (up) or route-slot / shared
    // rows (down). MX H is staged as float32 and quantised 8 values per lane, the 4 lanes of a
    // 32-column block forming an aligned quad (the first stores the scale byte).
    constexpr bool MX = UP && is_mx<EL>();
    constexpr int VB = MX ? 4 : 2;                    // staged bytes per value
    constexpr int CW = UP ? WN / 2 : WN;              // output columns per wave
    constexpr int JB = CW / 32;                       // 32-column blocks per wave
    constexpr int STRIDE = CW * VB + 16;              // padded LDS row (bytes)
    constexpr int VPL = MX ? 8 : 16 / VB;             // values per lane in the store phase
    constexpr int LPR = CW / VPL;                     // lanes per row in the store phase
    constexpr int SRPI = 64 / LPR;                    // rows per store pass
    static_assert(!MX || LPR % 4 == 0, "whole 32-column blocks per row");
    static_assert(32 * STRIDE <= 16384, "a wave's 32-row pass fits a quarter of buffer 1");
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) u32x2 lds_u2;
    typedef __attribute__((address_space(3))) u32x4 lds_u4;
    // wave w's region: 16 KB at (w / 2) * 16 KB into the A half (w even) or the B half (w odd)
    // of operand buffer 1 (the 256 x 256 configuration's buffers, which every view borrows)
    char* region = ((wid & 1) ? (char*)sm.buf[1].B : (char*)sm.buf[1].A) + (wid >> 1) * 16384;
    const int col0 = UP ? nt * (BN / 2) + wn * (WN / 2) : nt * BN + wn * WN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float rw = 1.0f;                                  // routing weight of the lane's row
      if (!UP) rw = sm.row_w[min(r_of(i), BM - 1)];
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float val[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = 4 * g + r;
            val[r] = UP ? silu(acc[i][j][v]) * acc[i][j + FN / 2][v] : acc[i][j][v] * rw;
          }
          char* dst = region + l32 * STRIDE + (j * 32 + 8 * g + 4 * h) * VB;
          if constexpr (MX) {
            u32x4 q;
            q.x = __float_as_uint(val[0]); q.y = __float_as_uint(val[1]);
            q.z = __float_as_uint(val[2]); q.w = __float_as_uint(val[3]);
            *(lds_u4*)dst = q;
          } else {
            u32x2 q;
            q.x = pack_bf16x2(val[0], val[1]);
            q.y = pack_bf16x2(val[2], val[3]);
            *(lds_u2*)dst = q;
          }
        }
#pragma unroll
      for (int q = 0; q < 32 / SRPI; ++q) {
        const int rr = q * SRPI + lane / LPR;           // row within the pass
        const int c = (lane % LPR) * VPL;               // first column of the lane's values
        const int r = blk_row(i) + rr;                  // row within the tile
        const char* src = region + rr * STRIDE + c * VB;
        if constexpr (MX) {
          const u32x4 lo = *(const lds_u4*)src, hi = *(const lds_u4*)(src + 16);
          const float vals[8] = {__uint_as_float(lo.x), __uint_as_float(lo.y),
                                 __uint_as_float(lo.z), __uint_as_float(lo.w),
                                 __uint_as_float(hi.x), __uint_as_float(hi.y),
                                 __uint_as_float(hi.z), __uint_as_float(hi.w)};
          int se;
          const int64_t hr = ring_row0 + m0 + r;
          const bool st = r < rows_valid && col0 + c < N;
          if constexpr (EL == Elem::FP4) {
            const uint32_t codes = mx4_quad8_f32(vals, &se);   // streamed past the L2
            if (st)
              __builtin_nontemporal_store(
                  codes, (uint32_t*)((uint8_t*)p.H + hr * (p.Hld / 2) + (col0 + c) / 2));
          } else {
            const uint2 codes = quantize_quad8_f32(vals, &se);
            u32x2 cv;                                    // streamed past the L2, as bf16 H
            cv.x = codes.x;
            cv.y = codes.y;
            if (st)
              __builtin_nontemporal_store(cv, (u32x2*)((uint8_t*)p.H + hr * p.Hld + col0 + c));
          }
          if (st) {
            if ((c & 31) == 0)
              p.H_sc[mx_kmajor_scale(hr, (col0 + c) / 32, (int64_t)p.n_slots * p.mb)] =
                  (uint8_t)(se + 127);
          }
        } else {
          const u32x4 val = *(const lds_u4*)src;
          if (r < rows_valid && col0 + c < N) {
            bf16_t* dst;
            if (UP) dst = (bf16_t*)p.H + (ring_row0 + m0 + r) * p.Hld;
            else dst = (shared ? (bf16_t*)p.y_shared : (bf16_t*)p.y_slots) + (int64_t)sm.row_dst[r] * p.d;
            // H rows (read again only by the down stage) stream past the L2 so they do not
            // evict the operand tiles other workgroups of the XCD are reading; route-slot and
            // shared rows stay cached for the combine
            if constexpr (UP) __builtin_nontemporal_store(val, (u32x4*)(dst + col0 + c));
            else *(u32x4*)(dst + col0 + c) = val;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);                // one 32-row block of values live at a time
    }
  } else {
    // float32 outputs: each lane stores its four consecutive columns as one 16-byte vector
    // (N is a multiple of 32, so a group of four is wholly inside or outside the matrix).
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const int col0 = UP ? nt * (BN / 2) + wn * (WN / 2) : nt * BN + wn * WN;
    constexpr int JB = UP ? FN / 2 : FN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = r_of(i);
      if (r >= rows_valid) continue;
      float* dst_row;
      float rw = 1.0f;
      if (UP) {
        dst_row = (float*)p.H + (ring_row0 + m0 + r) * p.Hld;
      } else {
        dst_row = (shared ? (float*)p.y_shared : (float*)p.y_slots) + (int64_t)sm.row_dst[r] * p.d;
        rw = sm.row_w[r];
      }
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = col0 + j * 32 + 8 * g + 4 * h;
          f32x4v o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int v = 4 * g + q;
            o[q] = UP ? silu(acc[i][j][v]) * acc[i][j + FN / 2][v] : acc[i][j][v] * rw;
          }
          if (col < N) *(f32x4v*)(dst_row + col) = o;
        }
    }
  }
  }
}

// LDS of a tile workgroup: the STAGES operand buffers as separate objects (only the first
// STAGES are referenced), the MX scale words and the down stage's row table. Stages 0 and 1 are
// sized for 128-byte rows whatever the configuration's row: the epilogue stages each wave's
// outputs through 16 KB of buffer 1's A or B half.
#define MOK_TILE_LDS(C, EL, sm)                                                                  \
  constexpr int SCW_ = scale_words<EL>();                                                        \
  __shared__ uint4 a0_[C::BM][8], a1_[C::BM][8], b0_[C::BN][8], b1_[C::BN][8];                   \
  uint4(*a0)[C::CH] = (uint4(*)[C::CH])a0_;                                                      \
  uint4(*a1)[C::CH] = (uint4(*)[C::CH])a1_;                                                      \
  uint4(*b0)[C::CH] = (uint4(*)[C::CH])b0_;                                                      \
  uint4(*b1)[C::CH] = (uint4(*)[C::CH])b1_;                                                      \
  __shared__ uint4 a2[C::STAGES > 2 ? C::BM : 1][C::CH], a3[C::STAGES > 2 ? C::BM : 1][C::CH];   \
  __shared__ uint4 b2[C::STAGES > 2 ? C::BN : 1][C::CH], b3[C::STAGES > 2 ? C::BN : 1][C::CH];   \
  __shared__ uint32_t as0[C::BM * SCW_], as1[C::BM * SCW_], bs0[C::BN * SCW_],                  \
      bs1[C::BN * SCW_];                                                                         \
  __shared__ uint32_t as2[C::STAGES > 2 ? C::BM : 1], as3[C::STAGES > 2 ? C::BM : 1];            \
  __shared__ uint32_t bs2[C::STAGES > 2 ? C::BN : 1], bs3[C::STAGES > 2 ? C::BN : 1];            \
  __shared__ int32_t row_dst[C::BM];                                                             \
  __shared__ float row_w[C::BM];                                                                 \
  Lds<C> sm;                                                                                     \
  sm.buf[0].A = a0; sm.buf[0].B = b0; sm.buf[0].As = as0; sm.buf[0].Bs = bs0;                    \
  sm.buf[1].A = a1; sm.buf[1].B = b1; sm.buf[1].As = as1; sm.buf[1].Bs = bs1;                    \
  if constexpr (C::STAGES > 2) {                                                                 \
    sm.buf[2].A = a2; sm.buf[2].B = b2; sm.buf[2].As = as2; sm.buf[2].Bs = bs2;                  \
    sm.buf[3].A = a3; sm.buf[3].B = b3; sm.buf[3].As = as3; sm.buf[3].Bs = bs3;                  \
  }                                                                                              \
  sm.row_dst = row_dst;                                                                          \
  sm.row_w = row_w

// Stage kernel: the workgroups walk the stage's tiles; consecutive tile ids land on the same
// XCD (workgroups are dispatched round-robin over the 8 XCDs), so tiles that share operand
// rows share that XCD's L2.
template <Elem EL, bool UP, bool F32OUT, class C>
__global__ __launch_bounds__(C::NT, 1) void k_expert_stage(ExpertPass p) {
  MOK_TILE_LDS(C, EL, sm);
  const int cap = p.max_mb;
  const int32_t total = p.wl[UP ? WL_N_U : WL_N_D];
  const int4* tab = UP ? wl_utab(p.wl, cap) : wl_dtab(p.wl, cap, p.cap_u);
  const int G = gridDim.x;
  const int b = blockIdx.x;
  int32_t t = (b & 7) * (G >> 3) + (b >> 3);
  if (t >= total) return;
  // The next tile's entry and slot, and (per lane) its A rows, are parked in LDS: no value is
  // carried in registers from one tile to the next (across the epilogue, where the register
  // file is full), so none is spilled and reloaded with a wait that drains the epilogue's
  // stores.
  constexpr bool PRE = UP && !is_mx<EL>();
  __shared__ int32_t pre_lds[PRE ? C::A_SLABS : 1][C::NT];
  __shared__ int4 nxt_lds;
  __shared__ int nslot_lds;
  const int tid = threadIdx.x;
  int4 cur = tab[t];
  int slot = wl_slot(p.wl, cap)[cur.x];
  int32_t pre[C::A_SLABS];
  prefetch_a_rows<EL, UP, C>(p, cur, pre);
  if constexpr (PRE) route_rows<C>(p, pre);
  for (;;) {
    const int32_t tn = t + G;
    const bool more = tn < total;
    // The next tile's entry (before the first DMA), its slot and route ids (step 1) and their
    // pool rows (step 2) are fetched under this tile's first K steps, each from values that
    // landed by that step's barrier, so the next prologue waits on no global load. The epilogue's barrier
    // orders the LDS writes before the reads below; the next tile's first barriers order those
    // reads before the next writes.
    int4 nxt = cur;
    int nslot = slot;
    int32_t pn[C::A_SLABS];
    run_tile<EL, UP, F32OUT, C>(p, sm, cur, slot, pre, [&](int s) {
      if (!more) return;
      if (s < 0) {                              // the entry: scalar loads (uniform index)
        const __attribute__((address_space(4))) int32_t* tc = (const __attribute__((address_space(4))) int32_t*)(tab + tn);
        nxt = make_int4(tc[0], tc[1], tc[2], tc[3]);
      } else if (s == 1) {
        nslot = wl_slot(p.wl, cap)[nxt.x];
        if constexpr (PRE) prefetch_a_rows<EL, UP, C>(p, nxt, pn);
        if (tid == 0) nxt_lds = nxt;
      } else if (s == 2) {
        if constexpr (PRE) {
          route_rows<C>(p, pn);
#pragma unroll
          for (int q = 0; q < C::A_SLABS; ++q) pre_lds[q][tid] = pn[q];
        }
        if (tid == 0) nslot_lds = nslot;
      }
    });
    if (!more) break;
    if constexpr (PRE) {
#pragma unroll
      for (int q = 0; q < C::A_SLABS; ++q) pre[q] = pre_lds[q][tid];
    }
    const int4 c = nxt_lds;
    cur.x = __builtin_amdgcn_readfirstlane(c.x);
    cur.y = __builtin_amdgcn_readfirstlane(c.y);
    cur.z = __builtin_amdgcn_readfirstlane(c.z);
    cur.w = __builtin_amdgcn_readfirstlane(c.w);
    slot = __builtin_amdgcn_readfirstlane(nslot_lds);
    t = tn;
  }
}

// ------------------------------------------------------------------------- MXFP8 gather
// Pull-gather + quantise of rows [r_begin, r_end) (at most G_ROWS) of minibatch m: the token
// rows of the pool picked by route id (or the own rows, for the shared experts) become MXFP8
// rows of the minibatch's ring slot. Called by every thread of the workgroup. The rows' token
// indices are looked up once into LDS; then a wave quantises one 128-element K step of 8 rows
// per item, 8 lanes a row and 16 consecutive elements a lane (the 2 lanes of a 32-element block
// are an aligned pair), GQ_UNROLL items with their loads in flight together. Its scale bytes
// (K-step-major words of consecutive ring rows) are then contiguous.
// items in flight per lane: 2 in the gather launch (8 workgroups per CU), 8 in the ring loop
// (one workgroup per CU, whose registers are free outside the GEMM tiles)
constexpr int GQ_UNROLL_STAGE = 2, GQ_UNROLL_RING = 8;
template <int GQ_UNROLL, bool FP4>
MOK_DEV void gather_quantize_rows(const ExpertPass& p, int m, int r_begin, int r_end, int wave,
                                  int n_waves) {
  __shared__ int64_t tok_row[G_ROWS];
  const int cap = p.max_mb;
  const int32_t g = wl_group(p.wl, cap)[m], first = wl_row0(p.wl, cap)[m];
  const int rows = r_end - r_begin;
  const int t = wave * 64 + (threadIdx.x & 63);
  __syncthreads();                                   // the previous call's readers are done
  if (t < rows) {
    const int r = r_begin + t;
    tok_row[t] = (g >= p.E_l ? p.own_begin + first + r : (int64_t)(p.route_ids[first + r] / p.k)) * p.d;
  }
  __syncthreads();
  const int steps = p.d / 128;
  const int total = (rows + 7) / 8 * steps * 64;
  const int nt = 64 * n_waves;
  const int64_t ring0 = (int64_t)wl_slot(p.wl, cap)[m] * p.mb + r_begin;
  const int64_t R = (int64_t)p.n_slots * p.mb;
  const int n_iter = (total + GQ_UNROLL * nt - 1) / (GQ_UNROLL * nt);   // same for every lane
  for (int it = 0; it < n_iter; ++it) {
    uint4 raw[GQ_UNROLL][2];
    int rr[GQ_UNROLL], cc[GQ_UNROLL];
#pragma unroll
    for (int u = 0; u < GQ_UNROLL; ++u) {
      const int q = t + (it * GQ_UNROLL + u) * nt;
      const uint32_t unit = (uint32_t)q >> 6;       // 8 rows x one K step
      const int li = q & 63, rg = (int)(unit / (uint32_t)steps), j = (int)unit - rg * steps;
      const int r = rg * 8 + (li >> 3);
      const bool ok = q < total && r < rows;
      rr[u] = ok ? r : 0;
      cc[u] = ok ? j * 8 + (li & 7) : -1;            // 16-element chunk of the row
      const bf16_t* src = (const bf16_t*)p.x + tok_row[rr[u]] + 16 * max(cc[u], 0);
      raw[u][0] = ok ? *(const uint4*)src : make_uint4(0, 0, 0, 0);
      raw[u][1] = ok ? *(const uint4*)(src + 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < GQ_UNROLL; ++u) {
      int sh;
      // both lanes of a pair share cc's validity
      const int64_t hr = ring0 + rr[u];
      if constexpr (FP4) {
        const uint2 codes = mx4_pair16(raw[u][0], raw[u][1], &sh);
        if (cc[u] >= 0) *(uint2*)(p.A_codes + hr * (p.d / 2) + 8 * cc[u]) = codes;
      } else {
        const uint4 codes = quantize_pair16(raw[u][0], raw[u][1], &sh);
        if (cc[u] >= 0) *(uint4*)(p.A_codes + hr * p.d + 16 * cc[u]) = codes;
      }
      if (cc[u] >= 0 && (cc[u] & 1) == 0)
        p.A_sc[mx_kmajor_scale(hr, cc[u] / 2, R)] = (uint8_t)(sh + 127);
    }
  }
}

// Stage-ordered path: every minibatch's rows, before the up stage. The rows of all minibatches
// (in work-list order) are cut into one contiguous range per workgroup, of equal size to a row;
// a workgroup walks its range in pieces of at most 16 rows of one minibatch.
template <bool FP4>
__global__ __launch_bounds__(256) void k_gather_quantize(ExpertPass p) {
  constexpr int PIECE = 16;
  const int n_mb = p.wl[WL_N_MB];
  const int32_t* nr = wl_rows(p.wl, p.max_mb);
  const int32_t* rp = wl_rpre(p.wl, p.max_mb);
  const int64_t total = rp[n_mb], G = gridDim.x;
  const int32_t r_lo = (int32_t)(blockIdx.x * total / G), r_hi = (int32_t)((blockIdx.x + 1) * total / G);
  if (r_lo >= r_hi) return;
  int lo = 0, hi = n_mb;                            // rp[lo] <= r_lo < rp[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (rp[mid] <= r_lo) lo = mid; else hi = mid;
  }
  int m = lo;
  int32_t r = r_lo - rp[m];                         // row within minibatch m
  for (int32_t done = r_lo; done < r_hi;) {
    if (r >= nr[m]) {                               // next minibatch (workgroup-uniform)
      ++m;
      r = 0;
      continue;
    }
    const int32_t r1 = min(min(nr[m], r + PIECE), r + (r_hi - done));
    gather_quantize_rows<GQ_UNROLL_STAGE, FP4>(p, m, r, r1, threadIdx.x >> 6, 4);
    done += r1 - r;
    r = r1;
  }
}

// ------------------------------------------------------------------------- ring work loop
// Persistent loop over the ring order built by k_build_worklist: each workgroup takes the next
// item with a ticket (an integer atomic: which workgroup runs an item never changes what the
// item computes), waits until the item's inputs are complete, runs it and counts it complete.
// Waits are bounded: one that runs out sets ERR_WAIT in the error word and goes on, so the
// loop always drains. Completion is published with an agent-scope release (the workgroup's
// stores written back from its XCD's L2) and observed with an agent-scope acquire, since the
// producer and the consumer of a ring slot may sit on different XCDs.
constexpr uint32_t kSpinLimit = 1u << 20;   // ~1 s: far above any legitimate wait

// Spin until *ctr >= need. Gives up (setting ERR_WAIT) after kSpinLimit polls, or at once once
// another wait has given up, so a broken dependency costs about one limit in total. Run by a
// whole wave: every value it branches on is made wave-uniform first.
MOK_DEV void wait_count(const int32_t* ctr, int32_t need, int32_t* err) {
  for (uint32_t it = 0;; ++it) {
    const int32_t v = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (v >= need) return;
    if ((it & 255u) == 255u) {
      const int32_t e = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (e & (int32_t)ERR_WAIT) return;
    }
    if (it >= kSpinLimit) {
      // one lane sets the bit (the others or in 0)
      __hip_atomic_fetch_or(err, opaque(lane_id()) == 0 ? (int32_t)ERR_WAIT : 0, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// The loop's control flow is wave-uniform everywhere: wave 0 as a whole takes the ticket, waits
// and publishes completion (lane 0 contributes the atomic increments, the other lanes add 0), and
// every field of the item is read back with readfirstlane. A lane-divergent branch here would let
// the compiler merge the publish of one item with the ticket of the next across the loop's
// back-edge, leaving the rest of wave 0 to pass the item barrier without lane 0.
//
// XCD split (WL_AFFINE): a workgroup serves the queue of the XCD it runs on (read from the
// hardware), so every ring slot is produced and consumed under one L2. A producer's stores have
// reached that L2 once its vmcnt drains (the L1 writes through); consumers read ring data past
// their L1 (sc0). No fence beyond that is needed. Without the split, items move between XCDs:
// completion is published with an agent-scope release (the L2 written back) and observed with
// an agent-scope acquire (the L2 invalidated).
template <Elem EL, bool F32OUT, class C>
__global__ __launch_bounds__(C::NT, 1) void k_ring(ExpertPass p) {
  MOK_TILE_LDS(C, EL, sm);
  // The loop's own LDS words, reached through a base made afresh at each use: the tile buffers
  // fill the first 128 KB, so these sit past the 64 KB an LDS instruction's offset field
  // reaches and need an address register; held across the loop, those registers were spilled.
  struct RingLds {
    int4 item, nitem;
    int32_t nprev, drain, next_queue, pad;
  };
  __shared__ RingLds rl_;
  auto R = [&]() { return (RingLds*)((char*)&rl_ + opaque(0)); };
  const int cap = p.max_mb;
  int32_t* wl = p.wl;
  const int4* rt = wl_rtab(wl, cap, p.cap_u, p.cap_d);
  const int32_t* us = wl_ustart(wl, cap);
  const int32_t* ds = wl_dstart(wl, cap);
  const int32_t* gs = wl_gstart(wl, cap);
  const int32_t* prev = wl_prev(wl, cap);
  int32_t* done_u = wl_done(wl, cap, KIND_U);
  int32_t* done_d = wl_done(wl, cap, KIND_D);
  int32_t* done_g = wl_done(wl, cap, KIND_G);
  const bool affine = uniform(wl[WL_AFFINE]) != 0;
  uint32_t hw_xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(hw_xcc));
  int x = affine ? (int)(hw_xcc & (N_XCD - 1)) : 0;
  int32_t seg0 = uniform(wl[WL_XR + x]);
  int32_t seg1 = affine ? uniform(wl[WL_XR + x + 1]) : uniform(wl[WL_N_R]);
  int32_t* ticket = &wl[WL_TICKETS + x];
  bool draining = false;               // this workgroup runs queues no workgroup served
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // 1 in lane 0, else 0: the increment of a wave-wide atomic. Made afresh at each use (from the
  // lane id), so no register holds it across the loop.
  auto one = [&]() { return opaque(lane_id()) == 0 ? 1 : 0; };
  // The next item is fetched while the current tile runs (wave 0, after K-step barriers 0..3,
  // where each load issued before has landed): ticket, entry, its slot predecessor, parked in
  // LDS. A gather item has no K loop: the next item is then fetched in line.
  int32_t tk = 0;
  int4 ne = make_int4(-1, 0, 0, 0);
  auto fetch_step = [&](int s) {
    if (wid != 0) return;
    if (s == 0) {
      tk = __hip_atomic_fetch_add(ticket, one(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (s == 1) {
      const int32_t t = seg0 + __builtin_amdgcn_readfirstlane(tk);
      ne = make_int4(-1, 0, 0, 0);
      if (t < seg1) ne = rt[t];
    } else if (s == 2) {
      int4 v;
      v.x = __builtin_amdgcn_readfirstlane(ne.x);
      v.y = __builtin_amdgcn_readfirstlane(ne.y);
      v.z = __builtin_amdgcn_readfirstlane(ne.z);
      v.w = __builtin_amdgcn_readfirstlane(ne.w);
      R()->nitem = v;
      tk = v.x >= 0 ? prev[v.x] : -1;
    } else {
      R()->nprev = __builtin_amdgcn_readfirstlane(tk);
    }
  };
  for (int s = 0; s < 4; ++s) {
    fetch_step(s);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  // Completion of a GEMM item is published late: at the next item's first K-step barrier, where
  // every wave has waited for its earlier stores anyway (vmcnt counts in order), so the store
  // drain overlaps the next item's first loads. pend (wave 0) is the counter of the item run
  // last and not yet published. A workgroup never waits while it holds an unpublished item:
  // unless the next item's inputs are already complete (or there is no next item), it drains
  // its stores and publishes first, so no chain of waits can lead back to it.
  int32_t* pend = nullptr;
  auto publish = [&]() {                          // wave 0; every wave's stores are complete
    if (pend) {
      if (!affine) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_fetch_add(pend, one(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pend = nullptr;
    }
  };
  for (;;) {
    // the counters the next item waits on (wave 0)
    int32_t *c1 = nullptr, *c2 = nullptr;
    int32_t n1 = 0, n2 = 0;
    auto wait_deps = [&]() {
      if (c1) wait_count(c1, n1, &wl[WL_ERR]);
      if (c2) wait_count(c2, n2, &wl[WL_ERR]);
      if (!affine) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    };
    auto complete = [&](const int32_t* c, int32_t n) {
      return !c || __builtin_amdgcn_readfirstlane(
                       __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >= n;
    };
    if (wid == 0) {
      int4 e = R()->nitem;
      bool drain = pend != nullptr;
      if (e.x >= 0) {
        const int m = __builtin_amdgcn_readfirstlane(e.x);
        const int kind = __builtin_amdgcn_readfirstlane(e.y) >> KIND_SHIFT;
        const int pm = __builtin_amdgcn_readfirstlane(R()->nprev);
        if (kind == KIND_D) {
          c1 = &done_u[m];
          n1 = us[m + 1] - us[m];
        } else if (kind == KIND_U) {
          c1 = &done_g[m];
          n1 = gs[m + 1] - gs[m];
          if (pm >= 0) {
            c2 = &done_d[pm];
            n2 = ds[pm + 1] - ds[pm];
          }
        } else if (pm >= 0) {
          c1 = &done_u[pm];
          n1 = us[pm + 1] - us[pm];
        }
        if (!pend) {
          wait_deps();
        } else {
          // a gather item publishes in line: drain for it too
          drain = kind == KIND_G || !complete(c1, n1) || !complete(c2, n2);
          if (!drain && !affine) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
      }
      RingLds* r = R();
      r->item = e;                                // every lane of wave 0 stores the same value
      r->drain = drain ? 1 : 0;
    }
    __syncthreads();
    int4 e;
    {
      const RingLds* r = R();
      e.x = __builtin_amdgcn_readfirstlane(r->item.x);
      e.y = __builtin_amdgcn_readfirstlane(r->item.y);
      e.z = __builtin_amdgcn_readfirstlane(r->item.z);
      e.w = __builtin_amdgcn_readfirstlane(r->item.w);
    }
    if (__builtin_amdgcn_readfirstlane(R()->drain)) {
      // every wave's stores of the pending item have reached L2; publish, then wait
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (wid == 0) {
        publish();
        if (e.x >= 0) wait_deps();
      }
      __syncthreads();
    }
    if (e.x < 0) {
      // queue x is exhausted. Without the split that ends the loop. With it, a queue is served
      // only by the workgroups the hardware placed on its XCD; should an XCD get none (a
      // placement other than round-robin), the last workgroup to finish its own queue runs
      // each queue whose ticket was never taken, from first item to last. Those items depend
      // only on items of the same queue, so one workgroup on any XCD computes them correctly.
      if (!affine) break;
      if (wid == 0) {
        bool last = draining;
        if (!draining) {
          const int32_t before = __builtin_amdgcn_readfirstlane(__hip_atomic_fetch_add(
              &wl[WL_EXITS], one(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          last = before == (int32_t)gridDim.x - 1;
        }
        int q = -1;
        if (last) {
          for (int y = N_XCD - 1; y >= 0; --y) {
            const int32_t taken = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                &wl[WL_TICKETS + y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (taken == 0 && uniform(wl[WL_XR + y]) < uniform(wl[WL_XR + y + 1])) q = y;
          }
        }
        R()->next_queue = q;              // every lane of wave 0 stores the same value
      }
      __syncthreads();
      const int q = __builtin_amdgcn_readfirstlane(R()->next_queue);
      if (q < 0) break;
      draining = true;
      x = q;
      seg0 = uniform(wl[WL_XR + q]);
      seg1 = uniform(wl[WL_XR + q + 1]);
      ticket = &wl[WL_TICKETS + q];
      for (int s = 0; s < 4; ++s) {
        fetch_step(s);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      continue;
    }
    const int kind = e.y >> KIND_SHIFT;
    e.y &= (1 << KIND_SHIFT) - 1;
    int32_t* ctr = kind == KIND_U ? done_u : (kind == KIND_D ? done_d : done_g);
    // after the first K-step barrier of a tile every wave's earlier stores are complete
    auto hook = [&](int s) {
      if (s < 0) return;
      if (s == 0 && wid == 0) publish();
      fetch_step(s);
    };
    if (kind == KIND_U) {
      int32_t pre[C::A_SLABS];
      prefetch_a_rows<EL, true, C>(p, e, pre);
      if constexpr (!is_mx<EL>()) route_rows<C>(p, pre);
      run_tile<EL, true, F32OUT, C, true>(p, sm, e, wl_slot(p.wl, p.max_mb)[e.x], pre, hook);
      if (wid == 0) pend = &ctr[e.x];
    } else if (kind == KIND_D) {
      int32_t pre[C::A_SLABS];
      run_tile<EL, false, F32OUT, C, true>(p, sm, e, wl_slot(p.wl, p.max_mb)[e.x], pre, hook);
      if (wid == 0) pend = &ctr[e.x];
    } else {
      if constexpr (is_mx<EL>()) {
        const int r0 = e.y * G_ROWS, r1 = min(e.w & 0xFFFF, r0 + G_ROWS);
        gather_quantize_rows<GQ_UNROLL_RING, EL == Elem::FP4>(p, e.x, r0, r1, wid, C::NW);
      }
      for (int s = 0; s < 4; ++s) {
        fetch_step(s);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      // every wave's stores have reached L2; then one publish covers the workgroup's item
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (wid == 0) {
        pend = &ctr[e.x];
        publish();
      }
    }
  }
}

// ------------------------------------------------------------------------- combine
// y[t] = S[t] + sum_{j ascending} P[t*k + j], float32 accumulator, one rounding. One thread
// per 16 B of a row: the k + 1 rows of a token are read once, y is written once. KC > 0: k ==
// KC known at compile time, so all k + 1 loads are in flight together; KC == 0: any k.
// The route slot rows and S are read once here: non-temporal loads keep them from displacing
// cached lines (measured: 42 against 45 us on the EP1 layer).
typedef unsigned int cmb_u32x4 __attribute__((ext_vector_type(4)));
MOK_DEV uint4 cmb_ld(const void* p) {
  const cmb_u32x4 v = __builtin_nontemporal_load((const cmb_u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <class OT, int KC>
__global__ __launch_bounds__(256) void k_combine(const OT* __restrict__ S, const OT* __restrict__ P,
                                                 OT* __restrict__ y, int64_t n_tok, int k_rt, int d) {
  constexpr int V = 16 / sizeof(OT);
  const int k = KC > 0 ? KC : k_rt;
  const int64_t per_row = d / V;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n_tok * per_row) return;
  const int64_t t = q / per_row, c = (q % per_row) * V;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0f;
  uint4 pv[KC > 0 ? KC : 1];
  if constexpr (KC > 0) {
#pragma unroll
    for (int j = 0; j < KC; ++j) pv[j] = cmb_ld(P + (t * k + j) * d + c);
  }
  if (S) {  // no shared expert: S = 0
    const uint4 s = cmb_ld(S + t * d + c);
    const OT* sv = (const OT*)&s;
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = load_as_f32<OT>(sv + v);
  }
#pragma unroll
  for (int j = 0; j < k; ++j) {
    if constexpr (KC == 0) pv[0] = *(const uint4*)(P + (t * k + j) * d + c);
    const OT* pp = (const OT*)&pv[KC > 0 ? j : 0];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] += load_as_f32<OT>(pp + v);
  }
  uint4 o;
  OT* ov = (OT*)&o;
#pragma unroll
  for (int v = 0; v < V; ++v) ov[v] = f32_to<OT>(acc[v]);
  *(uint4*)(y + t * d + c) = o;
}

template <class OT>
static void launch_combine_t(dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                             const void* S, const void* P, void* y, int64_t n_tok, int k, int d) {
  const OT *Sp = (const OT*)S, *Pp = (const OT*)P;
  OT* yp = (OT*)y;
  switch (k) {
    case 1: launch_k(k_combine<OT, 1>, grid, dim3(256), 0, s, e0, e1, Sp, Pp, yp, n_tok, k, d); break;
    case 2: launch_k(k_combine<OT, 2>, grid, dim3(256), 0, s, e0, e1, Sp, Pp, yp, n_tok, k, d); break;
    case 4: launch_k(k_combine<OT, 4>, grid, dim3(256), 0, s, e0, e1, Sp, Pp, yp, n_tok, k, d); break;
    case 6: launch_k(k_combine<OT, 6>, grid, dim3(256), 0, s, e0, e1, Sp, Pp, yp, n_tok, k, d); break;
    case 8: launch_k(k_combine<OT, 8>, grid, dim3(256), 0, s, e0, e1, Sp, Pp, yp, n_tok, k, d); break;
    default: launch_k(k_combine<OT, 0>, grid, dim3(256), 0, s, e0, e1, Sp, Pp, yp, n_tok, k, d);
  }
}

hipError_t launch_combine(const void* y_shared, const void* y_slots, void* y, int64_t n_tok,
                          int k, int d, bool f32, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int V = f32 ? 4 : 8;
  const int64_t n = n_tok * (d / V);
  if (n == 0) return mark_empty(s, e0, e1), hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (f32) launch_combine_t<float>(grid, s, e0, e1, y_shared, y_slots, y, n_tok, k, d);
  else launch_combine_t<bf16_t>(grid, s, e0, e1, y_shared, y_slots, y, n_tok, k, d);
  return hipGetLastError();
}

// ------------------------------------------------------------------------- launch
// event i of the stage-event array (stage s: 2s start, 2s + 1 stop), NULL if absent
static hipEvent_t ev_at(void* const* ev, int i) { return ev ? (hipEvent_t)ev[i] : nullptr; }
constexpr int EV_UP = 2 * 3, EV_DOWN = 2 * 4, EV_GATHER = 2 * 6;

template <Elem EL, bool F32OUT>
static hipError_t launch_stages_t(const ExpertPass& p, hipStream_t s, void* const* ev) {
  typedef typename CfgOf<EL>::type C;
  if (is_mx<EL>() && !p.ring)
    launch_k(k_gather_quantize<EL == Elem::FP4>, dim3(p.grid * 8), dim3(256), 0, s,
             ev_at(ev, EV_GATHER), ev_at(ev, EV_GATHER + 1), p);
  if (p.ring || p.loop) {
    launch_k(k_ring<EL, F32OUT, C>, dim3(p.grid), dim3(C::NT), 0, s, ev_at(ev, EV_UP),
             ev_at(ev, EV_UP + 1), p);
    mark_empty(s, ev_at(ev, EV_DOWN), ev_at(ev, EV_DOWN + 1));
    return hipGetLastError();
  }
  launch_k(k_expert_stage<EL, true, F32OUT, C>, dim3(p.grid), dim3(C::NT), 0, s,
           ev_at(ev, EV_UP), ev_at(ev, EV_UP + 1), p);
  launch_k(k_expert_stage<EL, false, F32OUT, C>, dim3(p.grid), dim3(C::NT), 0, s,
           ev_at(ev, EV_DOWN), ev_at(ev, EV_DOWN + 1), p);
  return hipGetLastError();
}

void gemm_tile_caps(int max_mb, int mb, int I, int I_sh, int d, bool gather_items, int* cap_u,
                    int* cap_d, int* cap_g) {
  const int64_t mt = (mb + Big::BM - 1) / Big::BM;
  const int64_t nU = std::max((I + Big::BN / 2 - 1) / (Big::BN / 2), (I_sh + Big::BN / 2 - 1) / (Big::BN / 2));
  const int64_t nD = (d + Big::BN - 1) / Big::BN;
  *cap_u = (int)std::min<int64_t>(INT32_MAX / 8, (int64_t)max_mb * mt * nU);
  *cap_d = (int)std::min<int64_t>(INT32_MAX / 8, (int64_t)max_mb * mt * nD);
  *cap_g = gather_items ? (int)std::min<int64_t>(INT32_MAX / 8, (int64_t)max_mb * ((mb + G_ROWS - 1) / G_ROWS)) : 0;
}

hipError_t launch_plan_worklist(const int32_t* idx, int64_t n_tok, int64_t tokens_per_rank,
                                int32_t* rank_counts, int32_t* blk_counts, const ExpertPass& p,
                                hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const bool mx = p.elem == Elem::FP8 || p.elem == Elem::FP4;
  WlBuild wb = {};
  wb.wl = p.wl;
  wb.E_l = p.E_l;
  wb.T_own = p.T_own;
  wb.mb = p.mb;
  wb.bm = Big::BM;
  wb.nU_r = (p.I + Big::BN / 2 - 1) / (Big::BN / 2);
  wb.nU_s = (p.I_sh + Big::BN / 2 - 1) / (Big::BN / 2);
  wb.nD = (p.d + Big::BN - 1) / Big::BN;
  wb.gather = p.ring && mx;
  wb.ring = p.ring;
  wb.loop = p.loop;
  wb.ks_u = p.d / 64;
  wb.ks_dr = p.I / 64;
  wb.ks_ds = p.I_sh / 64;
  wb.xcd_split = p.xcd_split;
  wb.n_slots = p.n_slots;
  wb.cap = p.max_mb;
  wb.cap_u = p.cap_u;
  wb.cap_d = p.cap_d;
  wb.cap_r = p.cap_r;
  wb.route_cap = p.route_cap;
  return launch_plan(idx, n_tok, p.k, p.e0, p.E_l, tokens_per_rank, (int32_t*)p.counts,
                     (int32_t*)p.offsets, rank_counts, (int32_t*)p.route_ids, blk_counts,
                     p.route_cap, s, ev0, ev1, &wb);
}

hipError_t launch_expert_stages(const ExpertPass& p, hipStream_t s, void* const* ev) {
  const bool mx = p.elem == Elem::FP8 || p.elem == Elem::FP4;
  if (!(mx && !p.ring))                  // the GATHER stage launches nothing
    mark_empty(s, ev_at(ev, EV_GATHER), ev_at(ev, EV_GATHER + 1));
  if (p.elem == Elem::BF16) return launch_stages_t<Elem::BF16, false>(p, s, ev);
  if (p.elem == Elem::F32) return launch_stages_t<Elem::F32, true>(p, s, ev);
  if (p.elem == Elem::FP4) return launch_stages_t<Elem::FP4, false>(p, s, ev);
  return launch_stages_t<Elem::FP8, false>(p, s, ev);
}

}  // namespace mok
