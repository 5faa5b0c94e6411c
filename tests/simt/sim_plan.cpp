// Runs the plan's two kernels (count; scatter + work-list workgroup) on the CPU emulation of a
// workgroup (simt.h) for the inputs in DIR/in.bin and writes the outputs to DIR/out.bin.
// kernels_gen.h is the kernels' own source text (plan.hip, worklist.h and the helpers they use
// from device_common.h), assembled by tests/test_plan_emulated.py.
#include "kernels_gen.h"
using namespace mok;

// the host side's chunking (plan_chunk in plan.hip)
static int64_t plan_chunk_h(int64_t n_routes, int E_l) {
  int64_t nb_max = 256;
  while (nb_max > 1 && nb_max * nb_max * E_l > ((int64_t)1 << 23)) nb_max /= 2;
  const int64_t per = PLAN_THREADS * nb_max;
  return PLAN_THREADS * std::max<int64_t>(1, (n_routes + per - 1) / per);
}

int main(int argc, char** argv) {
  std::string dir = argv[1];
  FILE* f = fopen((dir + "/in.bin").c_str(), "rb");
  int64_t hdr[24];
  if (fread(hdr, 8, 24, f) != 24) return 2;
  const int64_t T = hdr[0]; const int k = hdr[1], e0 = hdr[2], E_l = hdr[3];
  const int64_t tpr = hdr[4];
  WlBuild wb{};
  wb.E_l = E_l; wb.T_own = hdr[5]; wb.mb = hdr[6]; wb.bm = hdr[7]; wb.nU_r = hdr[8];
  wb.nU_s = hdr[9]; wb.nD = hdr[10]; wb.gather = hdr[11]; wb.ring = hdr[12]; wb.xcd_split = hdr[13];
  wb.n_slots = hdr[14]; wb.cap = hdr[15]; wb.cap_u = hdr[16]; wb.cap_d = hdr[17]; wb.cap_r = hdr[18];
  const int64_t route_cap = hdr[19];
  wb.loop = hdr[20]; wb.ks_u = hdr[21]; wb.ks_dr = hdr[22]; wb.ks_ds = hdr[23];
  wb.route_cap = route_cap;
  const int64_t n_routes = T * k;
  std::vector<int32_t> idx(std::max<int64_t>(1, n_routes));
  if (n_routes && fread(idx.data(), 4, n_routes, f) != (size_t)n_routes) return 3;
  fclose(f);
  const int64_t chunk = plan_chunk_h(n_routes, E_l);
  const int64_t nb = n_routes == 0 ? 1 : (n_routes + chunk - 1) / chunk;
  const int64_t R = T / tpr;
  // whole chunks per source rank: the scatter writes the rank counts as chunk sums
  const bool rank_sums = chunk % k == 0 && tpr % (chunk / k) == 0;
  // exactly sized heap buffers, so that the address sanitizer sees any overrun
  int32_t* blk_counts = (int32_t*)malloc(4 * nb * E_l);
  int32_t* counts = (int32_t*)malloc(4 * E_l);
  int32_t* offsets = (int32_t*)malloc(4 * (E_l + 1));
  int32_t* route_ids = (int32_t*)malloc(4 * route_cap);
  int32_t* rank_counts = (int32_t*)malloc(4 * E_l * R);
  const size_t wl_ints = wl_tab_off(wb.cap) + 4 * ((size_t)wb.cap_u + wb.cap_d + wb.cap_r);
  int32_t* wl = (int32_t*)malloc(4 * wl_ints);
  memset(wl, 0x7f, 4 * wl_ints);
  memset(route_ids, 0x7f, 4 * route_cap);
  memset(rank_counts, 0x7f, 4 * E_l * R);
  wb.wl = wl;
  const int32_t* idxp = idx.data();
  launch((unsigned)nb, PLAN_THREADS, sizeof(int32_t) * E_l, [&] {
    k_plan_count(idxp, n_routes, chunk, e0, E_l, blk_counts, rank_counts, (int64_t)E_l * R);
  });
  const int un = std::max(plan_scatter_ints(E_l), WL_LDS_INTS);
  const size_t sh = sizeof(int32_t) * (size_t)(plan_sums_ints(E_l) + std::max(un, 160));
  launch((unsigned)(nb + 1), PLAN_THREADS, sh, [&] {
    k_plan_scatter(idxp, n_routes, chunk, (int)nb, e0, E_l, blk_counts, counts, offsets,
                   route_ids, rank_counts, k, tpr, R, route_cap, wb, rank_sums ? 1 : 0);
  });
  FILE* o = fopen((dir + "/out.bin").c_str(), "wb");
  int64_t oh[4] = {nb, (int64_t)wl_ints, route_cap, E_l * R};
  fwrite(oh, 8, 4, o);
  fwrite(counts, 4, E_l, o);
  fwrite(offsets, 4, E_l + 1, o);
  fwrite(route_ids, 4, route_cap, o);
  fwrite(rank_counts, 4, E_l * R, o);
  fwrite(wl, 4, wl_ints, o);
  fclose(o);
  printf("nb %ld chunk %ld wl_ints %zu\n", (long)nb, (long)chunk, wl_ints);
  return 0;
}
