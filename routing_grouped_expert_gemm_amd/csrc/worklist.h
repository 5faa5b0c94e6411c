// The device work list of the expert stages: its layout, and the builder that the plan's last
// workgroup runs once the per-expert counts and region offsets are known (no host sync).
#pragma once
#include <stdint.h>

#include "device_common.h"

namespace mok {

// ------------------------------------------------------------------------- work list
// int32 block layout (offsets in ints): header; per minibatch: group, first row, rows, the
// prefix sums of its gather, up and down items, three completion counters, its ring slot, the
// minibatch that used that slot before it (-1: none), the prefix of its rows, and (ring) the
// item prefix sums in XCD-major order; then, 16-byte aligned, one int4 per
// up tile and per down tile {minibatch, tile within it, first row, group << 16 | rows} so that a
// workgroup finds its tile with a single load, and (ring work loop only) the ring order of all
// items, the item kind in bits 28+ of the second field.
// Header: counts, the error word, and for the ring loop the per-XCD split (WL_AFFINE set): XCD
// x owns minibatches x, x + 8, x + 16, ... (positions [XB[x], XB[x+1]) of the XCD-major order)
// and ring items [XR[x], XR[x+1]), and takes them with its own ticket TICKETS[x]; without the
// split every workgroup uses TICKETS[0] over all items. CAPS: the capacities the layout was cut
// for (minibatches, up tiles, down tiles, ring items), so that a reader can find the tables.
constexpr int WL_N_MB = 0, WL_N_U = 1, WL_N_D = 2, WL_ERR = 4, WL_N_R = 5, WL_AFFINE = 6,
              WL_XB = 8, WL_XR = 17, WL_TICKETS = 26, WL_EXITS = 34, WL_CAPS = 44, WL_HDR = 48;
constexpr int N_XCD = 8;        // XCDs of an MI355X, each with its own L2
constexpr int XB_N = 4;         // N tiles per block of the stage tables' tile order: up
constexpr int XB_ND = 8;        // ... down
constexpr uint32_t ERR_OVERFLOW = 1u, ERR_WAIT = 2u;
constexpr int KIND_U = 0, KIND_D = 1, KIND_G = 2, KIND_SHIFT = 28;
constexpr int G_ROWS = 64;      // rows of one gather + quantise item of the ring loop
MOK_DEV int32_t* wl_group(int32_t* wl, int cap) { return wl + WL_HDR; }
MOK_DEV int32_t* wl_row0(int32_t* wl, int cap) { return wl + WL_HDR + cap; }
MOK_DEV int32_t* wl_rows(int32_t* wl, int cap) { return wl + WL_HDR + 2 * cap; }
MOK_DEV int32_t* wl_ustart(int32_t* wl, int cap) { return wl + WL_HDR + 3 * cap; }
MOK_DEV int32_t* wl_dstart(int32_t* wl, int cap) { return wl + WL_HDR + 4 * cap + 1; }
MOK_DEV int32_t* wl_gstart(int32_t* wl, int cap) { return wl + WL_HDR + 5 * cap + 2; }
MOK_DEV int32_t* wl_done(int32_t* wl, int cap, int kind) { return wl + WL_HDR + (6 + kind) * cap + 3; }
MOK_DEV int32_t* wl_slot(int32_t* wl, int cap) { return wl + WL_HDR + 9 * cap + 3; }
MOK_DEV int32_t* wl_prev(int32_t* wl, int cap) { return wl + WL_HDR + 10 * cap + 3; }
MOK_DEV int32_t* wl_rpre(int32_t* wl, int cap) { return wl + WL_HDR + 11 * cap + 3; }   // cap + 1
// ring order: prefix sums of gather, up and down items over the minibatches in XCD-major order
MOK_DEV int32_t* wl_pg(int32_t* wl, int cap) { return wl + WL_HDR + 12 * cap + 4; }     // cap + 1
MOK_DEV int32_t* wl_pu(int32_t* wl, int cap) { return wl + WL_HDR + 13 * cap + 5; }     // cap + 1
MOK_DEV int32_t* wl_pd(int32_t* wl, int cap) { return wl + WL_HDR + 14 * cap + 6; }     // cap + 1
MOK_HOSTDEV size_t wl_tab_off(int cap) { return ((size_t)WL_HDR + 15 * (size_t)cap + 7 + 3) & ~(size_t)3; }
MOK_DEV int4* wl_utab(int32_t* wl, int cap) { return (int4*)(wl + wl_tab_off(cap)); }
MOK_DEV int4* wl_dtab(int32_t* wl, int cap, int cap_u) { return (int4*)(wl + wl_tab_off(cap)) + cap_u; }
MOK_DEV int4* wl_rtab(int32_t* wl, int cap, int cap_u, int cap_d) {
  return (int4*)(wl + wl_tab_off(cap)) + cap_u + cap_d;
}


// What the builder needs besides the plan's counts and offsets.
struct WlBuild {
  int32_t* wl;              // the work list to build (null: none)
  int E_l, T_own, mb, bm;   // local experts, own tokens, minibatch rows, GEMM tile rows
  int nU_r, nU_s, nD;       // N tiles of an up tile row (routed, shared) and of a down tile row
  int gather, ring, xcd_split, n_slots;   // gather items (MX ring), ring order, XCD split
  int loop;                 // stage order run by the persistent loop (stage tables + rt)
  int ks_u, ks_dr, ks_ds;   // K steps of an up tile, a routed and a shared down tile (weights)
  int cap, cap_u, cap_d, cap_r;           // capacities of the layout
  int64_t route_cap;        // rows of route_ids
};

// Exclusive scan of four values at once over a workgroup of 1024 threads (sh: 132 ints).
MOK_DEV int4 block_excl_scan4_1024(int4 v, int32_t* sh, int4* total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int4 inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ax = __shfl_up(inc.x, off, 64), ay = __shfl_up(inc.y, off, 64);
    const int az = __shfl_up(inc.z, off, 64), aw = __shfl_up(inc.w, off, 64);
    if (lane >= off) { inc.x += ax; inc.y += ay; inc.z += az; inc.w += aw; }
  }
  if (lane == 63) { sh[4 * w] = inc.x; sh[4 * w + 1] = inc.y; sh[4 * w + 2] = inc.z; sh[4 * w + 3] = inc.w; }
  __syncthreads();
  if (w == 0) {
    int4 wt = make_int4(0, 0, 0, 0);
    if (lane < 16) wt = make_int4(sh[4 * lane], sh[4 * lane + 1], sh[4 * lane + 2], sh[4 * lane + 3]);
    int4 wi = wt;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int ax = __shfl_up(wi.x, off, 64), ay = __shfl_up(wi.y, off, 64);
      const int az = __shfl_up(wi.z, off, 64), aw = __shfl_up(wi.w, off, 64);
      if (lane >= off) { wi.x += ax; wi.y += ay; wi.z += az; wi.w += aw; }
    }
    if (lane < 16) {
      sh[64 + 4 * lane] = wi.x - wt.x; sh[64 + 4 * lane + 1] = wi.y - wt.y;
      sh[64 + 4 * lane + 2] = wi.z - wt.z; sh[64 + 4 * lane + 3] = wi.w - wt.w;
    }
    if (lane == 15) { sh[128] = wi.x; sh[129] = wi.y; sh[130] = wi.z; sh[131] = wi.w; }
  }
  __syncthreads();
  const int4 r = make_int4(sh[64 + 4 * w] + inc.x - v.x, sh[64 + 4 * w + 1] + inc.y - v.y,
                           sh[64 + 4 * w + 2] + inc.z - v.z, sh[64 + 4 * w + 3] + inc.w - v.w);
  *total = make_int4(sh[128], sh[129], sh[130], sh[131]);
  __syncthreads();                                  // sh is reused by the next call
  return r;
}

// LDS of the builder: scan scratch, the minibatch prefix over the routed experts, and 18
// tables of up to WL_MBL + 1 entries (the per-minibatch tables while a forward has at most
// WL_MBL minibatches, so they are built in LDS and written out once; beyond that they are
// built in place in global memory), plus the staging of the tile placement.
constexpr int WL_MBL = 1024;
constexpr int WL_LDS_INTS = 160 + 19 * (WL_MBL + 1);

// One workgroup of 1024 threads builds the work list from cnt[E_l] and off[E_l + 1] (the
// plan's per-expert counts and region offsets, in LDS). Minibatches: routed experts ascending
// (rows ascending within each plan region), then the shared experts' minibatches over the own
// tokens. Every count comes from the plan on the device; nothing returns to the host.
//
// Ring order (ring): block b holds the gather items of minibatch b + 1 (MX only; b itself with
// a single slot), the up tiles of b, then the down tiles of minibatch b - lag; the first
// minibatch's gather items open the order. A down item needs every up tile of its minibatch;
// an up item needs its gather items and the down items of the minibatch that used its ring
// slot before it; a gather item needs that previous minibatch's up items. With lag < slots and
// the gather lead < slots every dependency of an item lies earlier in this order.
//
// With at least 8 slots the ring is split by XCD: XCD x runs minibatches x, x + 8, x + 16, ...
// on its own slots (n_slots / 8 of them, lag half of that) in the order above. A slot's
// producer and consumer then always share one L2, and the handover needs no L2 write-back or
// invalidation. Otherwise (fewer slots) one order covers all minibatches on all slots and
// every handover is made coherent device-wide.
MOK_DEV void build_worklist(const WlBuild& P, const int32_t* cnt, const int32_t* off,
                            int32_t* lds) {
  const int t = threadIdx.x;
  int32_t* wl = P.wl;
  const int cap = P.cap, E_l = P.E_l, mb = P.mb, bm = P.bm;
  int32_t* sh = lds;
  int32_t* mbp = lds + 160;                          // [E_l + 1] first minibatch of each expert
  auto la = [&](int i) { return lds + 160 + (1 + i) * (WL_MBL + 1); };
  // routed minibatches: expert e's region is cut into ceil(count / mb) pieces of mb rows
  const int32_t nm = t < E_l ? (cnt[t] + mb - 1) / mb : 0;
  int32_t n_routed;
  const int32_t ex = block_excl_scan_1024(nm, sh, &n_routed);
  if (t < E_l) mbp[t] = ex;
  if (t == 0) mbp[E_l] = n_routed;
  const int32_t n_sh = (P.nU_s > 0 && P.T_own > 0) ? (P.T_own + mb - 1) / mb : 0;
  const int32_t n_mb = min(cap, n_routed + n_sh);
  const bool in_lds = n_mb <= WL_MBL;
  int32_t* grp = in_lds ? la(0) : wl_group(wl, cap);
  int32_t* r0 = in_lds ? la(1) : wl_row0(wl, cap);
  int32_t* nr = in_lds ? la(2) : wl_rows(wl, cap);
  int32_t* us = in_lds ? la(3) : wl_ustart(wl, cap);
  int32_t* ds = in_lds ? la(4) : wl_dstart(wl, cap);
  int32_t* gs = in_lds ? la(5) : wl_gstart(wl, cap);
  int32_t* rp = in_lds ? la(6) : wl_rpre(wl, cap);
  int32_t* pg = in_lds ? la(7) : wl_pg(wl, cap);
  int32_t* pu = in_lds ? la(8) : wl_pu(wl, cap);
  int32_t* pd = in_lds ? la(9) : wl_pd(wl, cap);
  __syncthreads();
  for (int m = t; m < n_mb; m += 1024) {
    int32_t g, first, rows;
    if (m < n_routed) {
      int lo = 0, hi = E_l;                          // mbp[lo] <= m < mbp[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (mbp[mid] <= m) lo = mid; else hi = mid;
      }
      const int i = m - mbp[lo];
      g = lo;
      first = off[lo] + i * mb;
      rows = min(mb, cnt[lo] - i * mb);
    } else {
      const int i = m - n_routed;
      g = E_l;
      first = i * mb;
      rows = min(mb, P.T_own - i * mb);
    }
    grp[m] = g;
    r0[m] = first;
    nr[m] = rows;
  }
  for (int m = t; m < cap; m += 1024) {
    wl_done(wl, cap, KIND_U)[m] = 0;
    wl_done(wl, cap, KIND_D)[m] = 0;
    wl_done(wl, cap, KIND_G)[m] = 0;
  }
  __syncthreads();
  // item prefix sums: tiles of a minibatch = ceil(rows / bm) * n-tiles of its stage
  int4 carry = make_int4(0, 0, 0, 0);               // up, down, gather items, rows
  for (int c0 = 0; c0 < n_mb; c0 += 1024) {
    const int m = c0 + t;
    int4 v = make_int4(0, 0, 0, 0);
    if (m < n_mb) {
      const int32_t mt = (nr[m] + bm - 1) / bm;
      v = make_int4(mt * (grp[m] < E_l ? P.nU_r : P.nU_s), mt * P.nD,
                    P.gather ? (nr[m] + G_ROWS - 1) / G_ROWS : 0, nr[m]);
    }
    int4 tot;
    const int4 e = block_excl_scan4_1024(v, sh, &tot);
    if (m < n_mb) {
      us[m] = carry.x + e.x;
      ds[m] = carry.y + e.y;
      gs[m] = carry.z + e.z;
      rp[m] = carry.w + e.w;
    }
    carry.x += tot.x; carry.y += tot.y; carry.z += tot.z; carry.w += tot.w;
  }
  // more local routes than route_ids holds (a token naming one expert twice) also overflows:
  // no tile then reads past the plan
  const bool overflow = n_routed + n_sh > cap || carry.x > P.cap_u || carry.y > P.cap_d ||
                        (P.ring && (int64_t)carry.x + carry.y + carry.z > P.cap_r) ||
                        (P.loop && (int64_t)carry.x + carry.y > P.cap_r) ||
                        (int64_t)off[E_l] > P.route_cap;
  const bool affine = P.ring && P.xcd_split && P.n_slots >= N_XCD;
  if (t == 0) {
    us[n_mb] = carry.x;
    ds[n_mb] = carry.y;
    gs[n_mb] = carry.z;
    rp[n_mb] = overflow ? 0 : carry.w;
    wl[WL_N_MB] = n_mb;
    wl[WL_N_U] = overflow ? 0 : carry.x;
    wl[WL_N_D] = overflow ? 0 : carry.y;
    wl[WL_N_R] = overflow ? 0 : P.ring ? carry.x + carry.y + carry.z : P.loop ? carry.x + carry.y : 0;
    wl[WL_ERR] = overflow ? ERR_OVERFLOW : 0;
    wl[WL_AFFINE] = (affine || (P.loop && P.xcd_split && in_lds)) ? 1 : 0;
    wl[WL_CAPS] = cap;
    wl[WL_CAPS + 1] = P.cap_u;
    wl[WL_CAPS + 2] = P.cap_d;
    wl[WL_CAPS + 3] = P.cap_r;
  }
  if (t < N_XCD) wl[WL_TICKETS + t] = 0;
  if (t == 0) wl[WL_EXITS] = 0;
  // Ring order. With at least 8 slots the ring is split by XCD: minibatch m belongs to XCD
  // m % 8 as its (m / 8)-th minibatch, so the 8 XCDs run neighbouring minibatches -- mostly of
  // the same expert -- at the same time, and weights that one XCD reads from HBM the others
  // find in the chip's last-level cache (the MALL, shared by all XCDs). Without the split one
  // order spans all minibatches. Positions: XCD-major order p = base(x) + j for m = x + 8 j
  // (p = m without the split), and prefix sums of each item kind over p.
  __syncthreads();
  auto n_of = [&](int x) { return affine ? (n_mb - x + N_XCD - 1) / N_XCD : (x == 0 ? n_mb : 0); };
  auto base_of = [&](int x) {
    int b = 0;
    for (int y = 0; y < x; ++y) b += n_of(y);
    return b;
  };
  auto m_of = [&](int pp) {                         // the minibatch at XCD-major position pp
    if (!affine) return pp;
    int x = 0, b = 0;
    while (x < N_XCD - 1 && pp >= b + n_of(x)) b += n_of(x++);
    return x + N_XCD * (pp - b);
  };
  if (P.ring && !overflow) {
    int4 c = make_int4(0, 0, 0, 0);                 // gather, up, down
    for (int c0 = 0; c0 < n_mb; c0 += 1024) {
      const int pp = c0 + t;
      int4 v = make_int4(0, 0, 0, 0);
      if (pp < n_mb) {
        const int m = m_of(pp);
        v = make_int4(gs[m + 1] - gs[m], us[m + 1] - us[m], ds[m + 1] - ds[m], 0);
      }
      int4 tot;
      const int4 e = block_excl_scan4_1024(v, sh, &tot);
      if (pp < n_mb) {
        pg[pp] = c.x + e.x;
        pu[pp] = c.y + e.y;
        pd[pp] = c.z + e.z;
      }
      c.x += tot.x; c.y += tot.y; c.z += tot.z;
    }
    if (t == 0) {
      pg[n_mb] = c.x;
      pu[n_mb] = c.y;
      pd[n_mb] = c.z;
    }
  }
  __syncthreads();
  if (t <= N_XCD) {
    const int b = t < N_XCD ? base_of(t) : n_mb;
    wl[WL_XB + t] = b;
    if (!P.loop || overflow) wl[WL_XR + t] = (P.ring && !overflow) ? pg[b] + pu[b] + pd[b] : 0;
  }
  if (in_lds) {                                     // the tables the stages read
    for (int m = t; m <= n_mb; m += 1024) {
      if (m < n_mb) {
        wl_group(wl, cap)[m] = grp[m];
        wl_row0(wl, cap)[m] = r0[m];
        wl_rows(wl, cap)[m] = nr[m];
      }
      wl_ustart(wl, cap)[m] = us[m];
      wl_dstart(wl, cap)[m] = ds[m];
      wl_gstart(wl, cap)[m] = gs[m];
      wl_rpre(wl, cap)[m] = rp[m];
      if (P.ring && !overflow) {
        wl_pg(wl, cap)[m] = pg[m];
        wl_pu(wl, cap)[m] = pu[m];
        wl_pd(wl, cap)[m] = pd[m];
      }
    }
  }
  if (overflow) return;
  // Stage-ordered tables: when the shared experts' down tiles are the longer ones (K =
  // n_shared * I_shared > I), the down table lists them first, so that the longest tiles start
  // first and the stage ends evenly.
  const bool shared_first = P.nU_s > P.nU_r;
  const int32_t d_sh0 = ds[min(n_routed, n_mb)], d_sh = carry.y - d_sh0;
  // Tile order in the stage tables, per group (routed expert, or the shared experts): blocks of
  // XB consecutive N tiles (XB_N up, XB_ND down), and in each block the group's M tiles in
  // order, each with the block's N tiles. The 32 workgroups of an XCD take 32 consecutive
  // entries: with 8 or more M tiles in a group, an up round runs 8 M tiles x 4 N tiles and reads
  // 12 operand tiles per K step from the XCD's L2, not the 18 of 2 M tiles x 16 N tiles
  // (minibatch-major order).
  int4* ut = wl_utab(wl, P.cap);
  int4* dt = wl_dtab(wl, P.cap, P.cap_u);
  int4* rt = wl_rtab(wl, P.cap, P.cap_u, P.cap_d);
  const int mpm = (mb + bm - 1) / bm;               // M tiles of a whole minibatch
  auto dshift = [&](int m) {
    return !shared_first ? ds[m] : (m >= n_routed ? ds[m] - d_sh0 : ds[m] + d_sh);
  };
  // Stage tables (the ring loop reads only its own). Per chunk of 1024 minibatches: one thread
  // per minibatch puts its placement in LDS, then one thread per tile finds its minibatch by a
  // binary search over the chunk's tile prefix sums in LDS and writes the entry.
  if (!P.ring) {
    int32_t* c_pu = la(10);
    int32_t* c_pd = la(11);
    int32_t* c_first = la(12);
    int32_t* c_gw = la(13);
    int32_t* c_bu = la(14);
    int32_t* c_bd = la(15);
    int32_t* c_mt = la(16);
    int32_t* c_mo = la(17);
    for (int c0 = 0; c0 < n_mb; c0 += 1024) {
      const int nc = min(1024, n_mb - c0);
      __syncthreads();                                 // the previous chunk's readers are done
      if (t < nc) {
        const int m = c0 + t;
        const int32_t g = grp[m];
        // the group's minibatches [f, f_end): all but the last hold mb rows
        const int f = g < E_l ? mbp[g] : n_routed;
        const int f_end = g < E_l ? mbp[g + 1] : n_mb;
        c_first[t] = r0[m];
        c_gw[t] = (g << 16) | nr[m];
        c_bu[t] = us[f];
        c_bd[t] = dshift(f);
        c_mt[t] = (f_end - 1 - f) * mpm + (nr[f_end - 1] + bm - 1) / bm;   // the group's M tiles
        c_mo[t] = (m - f) * mpm;                                            // ... before m
      }
      if (t < nc) {
        c_pu[t] = us[c0 + t];
        c_pd[t] = ds[c0 + t];
      }
      if (t == 0) {                                    // the chunk's end (nc may be 1024)
        c_pu[nc] = us[c0 + nc];
        c_pd[nc] = ds[c0 + nc];
      }
      __syncthreads();
      auto place = [&](const int32_t* ps, int nN_r, int nN_s, const int32_t* bases, int4* tab,
                       int XB) {
        for (int32_t i = ps[0] + t; i < ps[nc]; i += 1024) {
          int lo = 0, hi = nc;                         // ps[lo] <= i < ps[hi]
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (ps[mid] <= i) lo = mid; else hi = mid;
          }
          const int l = i - ps[lo], gw = c_gw[lo];
          const int mt_m = ((gw & 0xFFFF) + bm - 1) / bm;
          const int mt = l % mt_m, nt = l / mt_m, nN = (gw >> 16) < E_l ? nN_r : nN_s;
          const int nb = nt / XB, w = min(XB, nN - nb * XB);
          tab[bases[lo] + nb * c_mt[lo] * XB + (c_mo[lo] + mt) * w + (nt - nb * XB)] =
              make_int4(c0 + lo, l, c_first[lo], gw);
        }
      };
      place(c_pu, P.nU_r, P.nU_s, c_bu, ut, XB_N);
      place(c_pd, P.nD, P.nD, c_bd, dt, XB_ND);
    }
  }
  if (P.loop) {
    // The stage order run by the persistent loop. The minibatches are cut, in order, into 8
    // contiguous ranges of about equal work (K steps of their tiles), one per XCD (with the
    // split; else one range); XCD x's queue holds the up tiles of its range, then their down
    // tiles, so a down tile depends only on up tiles earlier in its own queue, produced under
    // the same L2. Within a queue each expert's tiles keep the stage tables' blocked order,
    // restricted to the expert's M tiles in the range: blocks of XB N tiles, each with those
    // M tiles in order (an expert that straddles a cut is split by M tiles).
    const bool split = P.xcd_split && in_lds;
    __syncthreads();                                 // the stage tables are complete
    if (!split) {
      // one queue: the up table, then the down table
      for (int32_t i = t; i < carry.x; i += 1024) {
        int4 e = ut[i];
        e.y |= KIND_U << KIND_SHIFT;
        rt[i] = e;
      }
      for (int32_t i = t; i < carry.y; i += 1024) {
        int4 e = dt[i];
        e.y |= KIND_D << KIND_SHIFT;
        rt[carry.x + i] = e;
      }
      if (t <= N_XCD) wl[WL_XR + t] = t == 0 ? 0 : carry.x + carry.y;
    } else {
      int32_t* ub = la(10);                          // per minibatch: queue base of its up tiles
      int32_t* db = la(11);                          // ... of its down tiles
      int32_t* mg = la(12);                          // first minibatch of its expert in its range
      int32_t* mtx = la(13);                         // M tiles of its expert in its range
      int32_t* xm = la(14);                          // its XCD
      int32_t* xs = la(15);                          // per XCD: up count, down count, first m
      // work of minibatch m in K steps, and its exclusive prefix over m (n_mb <= 1024 here)
      int32_t wm = 0;
      if (t < n_mb) {
        const int32_t nu = us[t + 1] - us[t], nd = ds[t + 1] - ds[t];
        wm = nu * P.ks_u + nd * (grp[t] < E_l ? P.ks_dr : P.ks_ds);
      }
      int32_t w_tot;
      const int32_t wp = block_excl_scan_1024(wm, sh, &w_tot);
      if (t < N_XCD) { xs[t] = 0; xs[N_XCD + t] = 0; xs[2 * N_XCD + t] = n_mb; }
      if (t < n_mb) mtx[t] = 0;
      __syncthreads();
      // the XCD of m's work midpoint (non-decreasing in m: contiguous ranges)
      int x = 0;
      if (t < n_mb) {
        const int64_t mid2 = 2 * (int64_t)wp + wm;
        x = w_tot > 0 ? (int)min((int64_t)(N_XCD - 1), mid2 * N_XCD / (2 * (int64_t)w_tot)) : 0;
        xm[t] = x;
        atomicAdd(&xs[x], us[t + 1] - us[t]);          // integer sums: order-independent
        atomicAdd(&xs[N_XCD + x], ds[t + 1] - ds[t]);
        atomicMin(&xs[2 * N_XCD + x], t);
      }
      __syncthreads();
      if (t < n_mb) {
        const int g = grp[t];
        const int f = g < E_l ? mbp[g] : n_routed;     // the expert's first minibatch
        const int m_g = max(f, xs[2 * N_XCD + x]);
        mg[t] = m_g;
        atomicAdd(&mtx[m_g], (nr[t] + bm - 1) / bm);
        int32_t seg = 0;
        for (int y = 0; y < x; ++y) seg += xs[y] + xs[N_XCD + y];
        const int mf = xs[2 * N_XCD + x];
        ub[t] = seg + (us[m_g] - us[mf]);
        db[t] = seg + xs[x] + (ds[m_g] - ds[mf]);
      }
      if (t <= N_XCD) {
        int32_t b = 0;
        for (int y = 0; y < t; ++y) b += xs[y] + xs[N_XCD + y];
        wl[WL_XR + t] = b;
      }
      __syncthreads();
      // entry (m, l): M tile mt and N tile nt of minibatch m; its place in the expert's part of
      // the queue: block nb of XB N tiles holds the part's MT M tiles x w N tiles
      auto place_q = [&](const int4* tab, int32_t n, int kind, int XB) {
        for (int32_t i = t; i < n; i += 1024) {
          int4 e = tab[i];
          const int m = e.x, l = e.y;
          const int g = grp[m];
          const int mt_m = (nr[m] + bm - 1) / bm;
          const int mt = l % mt_m, nt = l / mt_m;
          const int nN = kind == KIND_U ? (g < E_l ? P.nU_r : P.nU_s) : P.nD;
          const int nb = nt / XB, w = min(XB, nN - nb * XB);
          const int MT = mtx[mg[m]];
          const int32_t rank = nb * MT * XB + ((m - mg[m]) * mpm + mt) * w + (nt - nb * XB);
          e.y |= kind << KIND_SHIFT;
          rt[(kind == KIND_U ? ub[m] : db[m]) + rank] = e;
        }
      };
      place_q(ut, carry.x, KIND_U, XB_N);
      place_q(dt, carry.y, KIND_D, XB_ND);
    }
  }
  int32_t* slot = wl_slot(wl, cap);
  int32_t* prev = wl_prev(wl, cap);
  for (int m = t; m < n_mb; m += 1024) {
    const int32_t g = grp[m], rw = nr[m], first = r0[m];
    const int4 ent = make_int4(m, 0, first, (g << 16) | rw);
    const int32_t nu = us[m + 1] - us[m], nd = ds[m + 1] - ds[m], ng = gs[m + 1] - gs[m];
    // this minibatch: the j-th of its XCD's n_x, on S slots starting at slot s0, order lag L
    int S = P.n_slots, s0 = 0, j = m, pb = 0, nx = n_mb, mstep = 1;
    if (affine) {
      const int x = m % N_XCD;
      S = P.n_slots / N_XCD;
      s0 = x * S;
      j = m / N_XCD;
      pb = base_of(x);
      nx = n_of(x);
      mstep = N_XCD;
    }
    const int L = S >= 2 ? S / 2 : 0;
    slot[m] = s0 + j % S;
    prev[m] = j >= S ? m - mstep * S : -1;
    if (P.ring) {
      // block b of the XCD's order: gather items of b + G, up tiles of b, down tiles of b - L
      // (G = 1 with two or more slots: a minibatch's rows are quantised a block before its up
      // tiles need them; the first minibatch's gather items open the order)
      const int G = S >= 2 ? 1 : 0;
      auto at = [&](int i) { return pb + min(max(i, 0), nx); };
      const int32_t pos_g = pg[at(j)] + pu[at(j - G)] + pd[at(j - G - L)];
      const int32_t pos_u = pg[at(j + G + 1)] + pu[at(j)] + pd[at(j - L)];
      const int32_t pos_d = pg[at(j + L + G + 1)] + pu[at(j + L + 1)] + pd[at(j)];
      for (int l = 0; l < ng; ++l) { int4 e = ent; e.y = (KIND_G << KIND_SHIFT) | l; rt[pos_g + l] = e; }
      for (int l = 0; l < nu; ++l) { int4 e = ent; e.y = (KIND_U << KIND_SHIFT) | l; rt[pos_u + l] = e; }
      for (int l = 0; l < nd; ++l) { int4 e = ent; e.y = (KIND_D << KIND_SHIFT) | l; rt[pos_d + l] = e; }
    }
  }
}

}  // namespace mok
