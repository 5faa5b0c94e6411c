// libmok C ABI (include/mok.h): argument validation, workspace layout, launch sequence.
// Every entry point validates everything before its first launch and never synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "mok.h"
#include "launch.h"

using namespace mok;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int status_of(hipError_t e) { return e == hipSuccess ? MOK_OK : MOK_EHIP; }

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Workspace layout of one forward. The work list sits at offset 0 so the device error word
// can be found from the workspace pointer alone.
struct Layout {
  bool use_ring = false, loop = false;
  int64_t route_cap = 1;   // rows of route_ids
  int n_slots = 0, max_mb = 0, Hld = 0, cap_u = 0, cap_d = 0, cap_g = 0, cap_r = 0;
  size_t wl = 0, logits = 0, idx = 0, w = 0, counts = 0, offsets = 0, rank_counts = 0,
         route_ids = 0, blk_counts = 0, H = 0, H_sc = 0, A_codes = 0, A_sc = 0,
         wq = 0, total = 0;
  // MX weight codes / scales sub-offsets (relative to wq)
  size_t wg_q = 0, wu_q = 0, wd_q = 0, sg_q = 0, su_q = 0, sd_q = 0;
  size_t wg_s = 0, wu_s = 0, wd_s = 0, sg_s = 0, su_s = 0, sd_s = 0;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int validate_moe(const mok_moe_args* a) {
  if (!a) return MOK_EINVAL;
  if (a->dtype < MOK_FP32 || a->dtype > MOK_MXFP4) return MOK_EINVAL;
  if (a->d <= 0 || a->E <= 0 || a->E > 1024 || a->k < 1 || a->k > a->E || a->k > 64)
    return MOK_EINVAL;
  if (a->I <= 0 || a->e0 < 0 || a->E_l < 1 || a->e0 + a->E_l > a->E) return MOK_EINVAL;
  if (a->T_pool < 0 || a->tokens_per_rank < 1 || a->T_pool % a->tokens_per_rank) return MOK_EINVAL;
  if (a->T_pool * (int64_t)a->k >= (int64_t)1 << 31) return MOK_EINVAL;
  // the GEMMs address pool rows with 32-bit byte offsets from the pool base
  const int64_t x_es = a->dtype == MOK_FP32 ? 4 : 2;
  if (a->T_pool * (int64_t)a->d * x_es >= (int64_t)1 << 32) return MOK_EUNSUPPORTED;
  if ((int64_t)std::max(a->I, a->n_shared * a->I_shared) * a->d * x_es >= (int64_t)1 << 32)
    return MOK_EUNSUPPORTED;
  if (a->own_begin < 0 || a->T_own < 0 || a->own_begin + a->T_own > a->T_pool) return MOK_EINVAL;
  if (a->n_shared < 0) return MOK_EINVAL;
  const int mb = a->minibatch_rows;
  if (mb != 128 && mb != 256 && mb != 512 && mb != 1024) return MOK_EINVAL;
  if (a->ring_rows < mb || a->ring_rows % mb) return MOK_EINVAL;
  // tile divisibility: K steps of 128 bytes per row (fp32 32, bf16 64, fp8 128, fp4 256
  // elements); down tiles of 128 columns, up tiles of 64 columns
  const int kstep = a->dtype == MOK_FP32 ? 32
                  : a->dtype == MOK_BF16 ? 64
                  : a->dtype == MOK_MXFP8 ? 128 : 256;
  if (a->d % 128 || a->d % kstep || a->I % 64 || a->I % kstep) return MOK_EINVAL;
  if (a->n_shared > 0) {
    if (a->I_shared <= 0 || a->I_shared % 64 || a->I_shared % kstep) return MOK_EINVAL;
    if (!a->ws_gate || !a->ws_up || !a->ws_down || !a->y_shared) return MOK_EINVAL;
  } else if (a->y_shared) {
    return MOK_EINVAL;
  }
  if (!a->x || !a->w_gate || !a->w_up || !a->w_down || !a->y_slots) return MOK_EINVAL;
  const bool given = a->topk_idx_in != nullptr;
  if (given != (a->topk_w_in != nullptr)) return MOK_EINVAL;
  if (given == (a->w_router != nullptr)) return MOK_EINVAL;
  const bool full = a->E_l == a->E;
  if (full) {
    if (!a->y || a->own_begin != 0 || (a->n_shared > 0 && a->T_own != a->T_pool)) return MOK_EINVAL;
  } else if (a->y) {
    return MOK_EINVAL;
  }
  return MOK_OK;
}

Layout layout_moe(const mok_moe_args* a) {
  Layout L;
  const int mb = a->minibatch_rows;
  const int64_t n_cap = a->T_pool * (int64_t)std::min(a->k, a->E_l);
  L.route_cap = std::max<int64_t>(1, n_cap);
  const int I_sh = a->n_shared * a->I_shared;
  const int64_t max_mb = ceil_div(n_cap, mb) + a->E_l + (I_sh > 0 ? ceil_div(a->T_own, mb) : 0);
  L.max_mb = (int)std::max<int64_t>(1, max_mb);
  L.loop = (a->flags & MOK_FLAG_STAGE_LOOP) != 0;
  L.use_ring = !(a->flags & MOK_FLAG_NO_RING) && !L.loop;
  L.n_slots = L.use_ring ? a->ring_rows / mb : L.max_mb;
  L.Hld = std::max(a->I, I_sh);
  const size_t es = a->dtype == MOK_FP32 ? 4 : 2;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  const bool mx = a->dtype == MOK_MXFP8 || a->dtype == MOK_MXFP4;
  // bytes of n MX codes: one a byte (MXFP8), two a byte (MXFP4)
  auto cb = [&](size_t n) { return a->dtype == MOK_MXFP4 ? n / 2 : n; };
  gemm_tile_caps(L.max_mb, mb, a->I, I_sh, a->d, L.use_ring && mx, &L.cap_u, &L.cap_d, &L.cap_g);
  L.cap_r = L.use_ring ? L.cap_u + L.cap_d + L.cap_g : L.loop ? L.cap_u + L.cap_d : 0;
  L.wl = take(sizeof(int32_t) * worklist_ints(L.max_mb, L.cap_u, L.cap_d, L.cap_r));
  const bool route = a->w_router != nullptr;
  L.logits = (route && !a->logits_out) ? take(sizeof(float) * a->T_pool * a->E) : 0;
  L.idx = (route && !a->topk_idx_out) ? take(sizeof(int32_t) * a->T_pool * a->k) : 0;
  L.w = (route && !a->topk_w_out) ? take(sizeof(float) * a->T_pool * a->k) : 0;
  L.counts = take(sizeof(int32_t) * a->E_l);
  L.offsets = take(sizeof(int32_t) * (a->E_l + 1));
  L.rank_counts = 0;
  L.route_ids = a->route_ids_out ? 0 : take(sizeof(int32_t) * std::max<int64_t>(1, n_cap));
  const int64_t nb = plan_n_blocks(a->T_pool * a->k, a->E_l);
  L.blk_counts = take(sizeof(int32_t) * nb * a->E_l);
  const int64_t ring_rows = (int64_t)L.n_slots * mb;
  if (mx) {
    L.H = take(cb((size_t)ring_rows * L.Hld));
    L.H_sc = take((size_t)ring_rows * (L.Hld / 32));
    L.A_codes = take(cb((size_t)ring_rows * a->d));
    L.A_sc = take((size_t)ring_rows * (a->d / 32));
    const size_t el = (size_t)a->E_l * a->I * a->d;
    L.wg_q = take(cb(el)); L.wu_q = take(cb(el)); L.wd_q = take(cb(el));
    L.wg_s = take(el / 32); L.wu_s = take(el / 32); L.wd_s = take(el / 32);
    const size_t sl = (size_t)I_sh * a->d;
    L.sg_q = take(cb(sl)); L.su_q = take(cb(sl)); L.sd_q = take(cb(sl));
    L.sg_s = take(sl / 32); L.su_s = take(sl / 32); L.sd_s = take(sl / 32);
  } else {
    L.H = take((size_t)ring_rows * L.Hld * es);
  }
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char* mok_status_string(int s) {
  switch (s) {
    case MOK_OK: return "MOK_OK";
    case MOK_EINVAL: return "MOK_EINVAL: invalid argument";
    case MOK_EUNSUPPORTED: return "MOK_EUNSUPPORTED: not supported by this build";
    case MOK_EWORKSPACE: return "MOK_EWORKSPACE: workspace missing or too small";
    case MOK_EHIP: return "MOK_EHIP: HIP runtime error";
    default: return "unknown mok status";
  }
}

const char* mok_version(void) { return "mok 0.1.0 gfx950"; }

int mok_route(const void* x, const void* w_router, int64_t T, int32_t d, int32_t E, int32_t k,
              int32_t io_dtype, float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  if (T < 0 || d < 1 || E < 1 || E > 1024 || k < 1 || k > E || k > 64) return MOK_EINVAL;
  if (io_dtype != MOK_FP32 && io_dtype != MOK_BF16) return MOK_EINVAL;
  if (T == 0) return MOK_OK;
  if (!x || !w_router || !logits || !topk_idx || !topk_w) return MOK_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  return status_of(launch_route(x, w_router, T, d, E, k, io_dtype == MOK_BF16, logits, topk_idx,
                                topk_w, s));
}

int mok_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx,
             float* topk_w, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 64) return MOK_EINVAL;
  if (T == 0) return MOK_OK;
  if (!logits || !topk_idx || !topk_w) return MOK_EINVAL;
  return status_of(launch_topk(logits, T, E, k, topk_idx, topk_w, (hipStream_t)stream));
}

int mok_dispatch_plan_workspace_bytes(int64_t T_pool, int32_t k, int32_t E_l, size_t* bytes) {
  if (!bytes || T_pool < 0 || k < 1 || E_l < 1 || E_l > 1024) return MOK_EINVAL;
  const int64_t nb = plan_n_blocks(T_pool * k, E_l);
  *bytes = align_up(sizeof(int32_t) * nb * E_l);
  return MOK_OK;
}

int mok_dispatch_plan(const int32_t* topk_idx, int64_t T_pool, int32_t k, int32_t E, int32_t e0,
                      int32_t E_l, int32_t tokens_per_rank, int32_t* counts, int32_t* offsets,
                      int32_t* rank_counts, int32_t* route_ids, void* ws, size_t ws_bytes,
                      void* stream) {
  if (T_pool < 0 || k < 1 || E < 1 || k > E || e0 < 0 || E_l < 1 || E_l > 1024 || e0 + E_l > E)
    return MOK_EINVAL;
  if (tokens_per_rank < 1 || T_pool % tokens_per_rank) return MOK_EINVAL;
  if (T_pool * (int64_t)k >= (int64_t)1 << 31) return MOK_EINVAL;
  if ((T_pool > 0 && !topk_idx) || !counts || !offsets || !rank_counts || !route_ids)
    return MOK_EINVAL;
  size_t need = 0;
  mok_dispatch_plan_workspace_bytes(T_pool, k, E_l, &need);
  if (!ws || ws_bytes < need) return MOK_EWORKSPACE;
  int32_t* blk_counts = (int32_t*)ws;
  const int64_t cap = std::max<int64_t>(1, T_pool * std::min(k, E_l));
  return status_of(launch_plan(topk_idx, T_pool, k, e0, E_l, tokens_per_rank, counts, offsets,
                               rank_counts, route_ids, blk_counts, cap, (hipStream_t)stream));
}

int mok_moe_workspace_bytes(const mok_moe_args* a, size_t* bytes) {
  if (!bytes) return MOK_EINVAL;
  int st = validate_moe(a);
  if (st != MOK_OK) return st;
  *bytes = layout_moe(a).total;
  return MOK_OK;
}

int mok_moe_forward(const mok_moe_args* a, void* stream) {
  int st = validate_moe(a);
  if (st != MOK_OK) return st;
  const Layout L = layout_moe(a);
  if (!a->workspace || a->workspace_bytes < L.total) return MOK_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)a->workspace;
  auto at = [&](size_t off) { return (void*)(ws + off); };
  const int k = a->k;
  // stage events: tied to the stage's first and last kernels (a stage that launches nothing
  // records them as markers)
  void* const* ev = a->stage_events;
  auto ev_start = [&](int stage) { return ev ? (hipEvent_t)ev[2 * stage] : nullptr; };
  auto ev_stop = [&](int stage) { return ev ? (hipEvent_t)ev[2 * stage + 1] : nullptr; };
  auto mark = [&](int stage) { mark_empty(s, ev_start(stage), ev_stop(stage)); };

  // stage 1: routing
  const int32_t* idx = a->topk_idx_in;
  const float* w = a->topk_w_in;
  if (a->w_router) {
    float* logits = a->logits_out ? a->logits_out : (float*)at(L.logits);
    int32_t* oidx = a->topk_idx_out ? a->topk_idx_out : (int32_t*)at(L.idx);
    float* ow = a->topk_w_out ? a->topk_w_out : (float*)at(L.w);
    if (a->T_pool > 0) {
      hipError_t e = launch_route(a->x, a->w_router, a->T_pool, a->d, a->E, k,
                                  a->dtype != MOK_FP32, logits, oidx, ow, s,
                                  ev_start(MOK_STAGE_ROUTE), ev_stop(MOK_STAGE_ROUTE));
      if (e != hipSuccess) return MOK_EHIP;
    } else {
      mark(MOK_STAGE_ROUTE);
    }
    idx = oidx;
    w = ow;
  } else {
    mark(MOK_STAGE_ROUTE);
  }

  // stage 2: plan (and the expert stages' work list)
  int32_t* counts = a->counts_out ? a->counts_out : (int32_t*)at(L.counts);
  int32_t* offsets = a->offsets_out ? a->offsets_out : (int32_t*)at(L.offsets);
  int32_t* route_ids = a->route_ids_out ? a->route_ids_out : (int32_t*)at(L.route_ids);

  // stages 3-5
  ExpertPass p = {};
  p.elem = a->dtype == MOK_FP32 ? Elem::F32
         : a->dtype == MOK_BF16 ? Elem::BF16
         : a->dtype == MOK_MXFP8 ? Elem::FP8 : Elem::FP4;
  p.out_f32 = a->dtype == MOK_FP32;
  p.d = a->d;
  p.k = k;
  p.I = a->I;
  p.E_l = a->E_l;
  p.e0 = a->e0;
  p.I_sh = a->n_shared * a->I_shared;
  p.I_seg = a->n_shared > 0 ? a->I_shared : 1;
  p.own_begin = a->own_begin;
  p.T_own = a->n_shared > 0 ? a->T_own : 0;
  p.mb = a->minibatch_rows;
  p.n_slots = L.n_slots;
  p.Hld = L.Hld;
  p.max_mb = L.max_mb;
  p.cap_u = L.cap_u;
  p.cap_d = L.cap_d;
  p.cap_r = L.cap_r;
  p.ring = L.use_ring;
  p.loop = L.loop;
  p.route_cap = L.route_cap;
  const int cus = device_cus();
  p.grid = ((cus + 7) / 8) * 8;            // one 256 x 256 tile workgroup per CU
  // the ring's per-XCD queues pay off on the whole chip (8 XCDs of 32 CUs, dispatched
  // round-robin); on a partition of it one queue serves every workgroup
  p.xcd_split = cus == 256;
  p.x = a->x;
  p.route_ids = route_ids;
  p.topk_w = w;
  p.counts = counts;
  p.offsets = offsets;
  p.H = at(L.H);
  p.wl = (int32_t*)at(L.wl);
  p.y_slots = a->y_slots;
  p.y_shared = a->y_shared;
  if (launch_plan_worklist(idx, a->T_pool, a->tokens_per_rank, a->rank_counts_out,
                           (int32_t*)at(L.blk_counts), p, s, ev_start(MOK_STAGE_PLAN),
                           ev_stop(MOK_STAGE_PLAN)) != hipSuccess)
    return MOK_EHIP;
  if (a->dtype == MOK_MXFP8 || a->dtype == MOK_MXFP4) {
    const bool fp4 = a->dtype == MOK_MXFP4;
    char* q = ws;
    uint8_t* wg_q = (uint8_t*)(q + L.wg_q); uint8_t* wu_q = (uint8_t*)(q + L.wu_q);
    uint8_t* wd_q = (uint8_t*)(q + L.wd_q); uint8_t* sg_q = (uint8_t*)(q + L.sg_q);
    uint8_t* su_q = (uint8_t*)(q + L.su_q); uint8_t* sd_q = (uint8_t*)(q + L.sd_q);
    uint8_t* wg_s = (uint8_t*)(q + L.wg_s); uint8_t* wu_s = (uint8_t*)(q + L.wu_s);
    uint8_t* wd_s = (uint8_t*)(q + L.wd_s); uint8_t* sg_s = (uint8_t*)(q + L.sg_s);
    uint8_t* su_s = (uint8_t*)(q + L.su_s); uint8_t* sd_s = (uint8_t*)(q + L.sd_s);
    const int64_t rI = (int64_t)a->E_l * a->I, rD = (int64_t)a->E_l * a->d;
    const bool sh = p.I_sh > 0;
    hipEvent_t q0 = ev_start(MOK_STAGE_QUANT), q1 = ev_stop(MOK_STAGE_QUANT);
    // scales K-step major per matrix (the layout the GEMMs' scale loads read)
    hipError_t e = launch_quantize_mx(a->w_gate, rI, a->d, wg_q, wg_s, fp4, s, q0, nullptr, a->I);
    if (e == hipSuccess)
      e = launch_quantize_mx(a->w_up, rI, a->d, wu_q, wu_s, fp4, s, nullptr, nullptr, a->I);
    if (e == hipSuccess)
      e = launch_quantize_mx(a->w_down, rD, a->I, wd_q, wd_s, fp4, s, nullptr, sh ? nullptr : q1,
                             a->d);
    if (e == hipSuccess && sh) {
      e = launch_quantize_mx(a->ws_gate, p.I_sh, a->d, sg_q, sg_s, fp4, s, nullptr, nullptr,
                             p.I_sh);
      if (e == hipSuccess)
        e = launch_quantize_mx(a->ws_up, p.I_sh, a->d, su_q, su_s, fp4, s, nullptr, nullptr,
                               p.I_sh);
      if (e == hipSuccess)
        e = launch_quantize_mx(a->ws_down, (int64_t)a->n_shared * a->d, a->I_shared, sd_q, sd_s,
                               fp4, s, nullptr, q1, a->d);
    }
    if (e != hipSuccess) return MOK_EHIP;
    p.wg = wg_q; p.wu = wu_q; p.wd = wd_q; p.sg = sg_q; p.su = su_q; p.sd = sd_q;
    p.wg_sc = wg_s; p.wu_sc = wu_s; p.wd_sc = wd_s; p.sg_sc = sg_s; p.su_sc = su_s; p.sd_sc = sd_s;
    p.H_sc = (uint8_t*)at(L.H_sc);
    p.A_codes = (uint8_t*)at(L.A_codes);
    p.A_sc = (uint8_t*)at(L.A_sc);
  } else {
    p.wg = a->w_gate; p.wu = a->w_up; p.wd = a->w_down;
    p.sg = a->ws_gate; p.su = a->ws_up; p.sd = a->ws_down;
    mark(MOK_STAGE_QUANT);
  }
  if (launch_expert_stages(p, s, ev) != hipSuccess) return MOK_EHIP;

  // combine (full layer only)
  if (a->E_l == a->E) {
    if (launch_combine(a->y_shared, a->y_slots, a->y, a->T_pool, k, a->d, p.out_f32, s,
                       ev_start(MOK_STAGE_COMBINE), ev_stop(MOK_STAGE_COMBINE)) != hipSuccess)
      return MOK_EHIP;
  } else {
    mark(MOK_STAGE_COMBINE);
  }
  return MOK_OK;
}

int mok_moe_workspace_region(const mok_moe_args* a, int32_t region, size_t* offset,
                             size_t* bytes, int64_t* rows) {
  if (!offset || !bytes || !rows) return MOK_EINVAL;
  int st = validate_moe(a);
  if (st != MOK_OK) return st;
  const Layout L = layout_moe(a);
  const bool mx = a->dtype == MOK_MXFP8 || a->dtype == MOK_MXFP4;
  const int64_t ring = (int64_t)L.n_slots * a->minibatch_rows;
  const size_t half = a->dtype == MOK_MXFP4 ? 2 : 1;   // MX codes a byte
  const int64_t I_sh = (int64_t)a->n_shared * a->I_shared;
  const int64_t el = (int64_t)a->E_l * a->I * a->d, sl = I_sh * a->d;
  const size_t es = a->dtype == MOK_FP32 ? 4 : 2;
  size_t off = 0, n = 0;
  int64_t R = 0;
  switch (region) {
    case MOK_REGION_WORKLIST:
      off = L.wl; n = sizeof(int32_t) * worklist_ints(L.max_mb, L.cap_u, L.cap_d, L.cap_r);
      R = 1; break;
    case MOK_REGION_H:
      off = L.H; n = (size_t)ring * L.Hld * (mx ? 1 : es) / half; R = ring; break;
    case MOK_REGION_H_SCALES: off = L.H_sc; n = (size_t)ring * (L.Hld / 32); R = ring; break;
    case MOK_REGION_A_CODES: off = L.A_codes; n = (size_t)ring * a->d / half; R = ring; break;
    case MOK_REGION_A_SCALES: off = L.A_sc; n = (size_t)ring * (a->d / 32); R = ring; break;
    case MOK_REGION_WG_CODES: off = L.wg_q; n = el / half; R = a->I; break;
    case MOK_REGION_WG_SCALES: off = L.wg_s; n = el / 32; R = a->I; break;
    case MOK_REGION_WU_CODES: off = L.wu_q; n = el / half; R = a->I; break;
    case MOK_REGION_WU_SCALES: off = L.wu_s; n = el / 32; R = a->I; break;
    case MOK_REGION_WD_CODES: off = L.wd_q; n = el / half; R = a->d; break;
    case MOK_REGION_WD_SCALES: off = L.wd_s; n = el / 32; R = a->d; break;
    case MOK_REGION_SG_CODES: off = L.sg_q; n = sl / half; R = I_sh; break;
    case MOK_REGION_SG_SCALES: off = L.sg_s; n = sl / 32; R = I_sh; break;
    case MOK_REGION_SU_CODES: off = L.su_q; n = sl / half; R = I_sh; break;
    case MOK_REGION_SU_SCALES: off = L.su_s; n = sl / 32; R = I_sh; break;
    case MOK_REGION_SD_CODES: off = L.sd_q; n = sl / half; R = a->d; break;
    case MOK_REGION_SD_SCALES: off = L.sd_s; n = sl / 32; R = a->d; break;
    default: return MOK_EINVAL;
  }
  // the MX regions exist only in an MXFP8 forward, the shared ones only with shared experts
  if (!mx && region >= MOK_REGION_H_SCALES) return MOK_EINVAL;
  if (region >= MOK_REGION_SG_CODES && I_sh == 0) return MOK_EINVAL;
  *offset = off;
  *bytes = n;
  *rows = R;
  return MOK_OK;
}

int mok_quantize_mxfp8(const void* src_bf16, int64_t rows, int32_t K, uint8_t* codes,
                       uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOK_EINVAL;
  if (rows == 0) return MOK_OK;
  if (!src_bf16 || !codes || !scales) return MOK_EINVAL;
  return status_of(launch_quantize_mx(src_bf16, rows, K, codes, scales, false,
                                      (hipStream_t)stream));
}

int mok_quantize_mxfp4(const void* src_bf16, int64_t rows, int32_t K, uint8_t* codes,
                       uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOK_EINVAL;
  if (rows == 0) return MOK_OK;
  if (!src_bf16 || !codes || !scales) return MOK_EINVAL;
  return status_of(launch_quantize_mx(src_bf16, rows, K, codes, scales, true,
                                      (hipStream_t)stream));
}

int mok_quantize_mxfp8_f32(const float* src, int64_t rows, int32_t K, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOK_EINVAL;
  if (rows == 0) return MOK_OK;
  if (!src || !codes || !scales) return MOK_EINVAL;
  return status_of(launch_quantize_mx_f32(src, rows, K, codes, scales, false, (hipStream_t)stream));
}

int mok_quantize_mxfp4_f32(const float* src, int64_t rows, int32_t K, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOK_EINVAL;
  if (rows == 0) return MOK_OK;
  if (!src || !codes || !scales) return MOK_EINVAL;
  return status_of(launch_quantize_mx_f32(src, rows, K, codes, scales, true, (hipStream_t)stream));
}

int mok_get_device_error(const void* workspace, uint32_t* err, void* stream) {
  if (!workspace || !err) return MOK_EINVAL;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOK_EHIP;
  int32_t v[5] = {0};
  if (hipMemcpy(v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return MOK_EHIP;
  *err = (uint32_t)v[4];
  return MOK_OK;
}

}  // extern "C"
