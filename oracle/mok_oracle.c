/*
 * CPU oracle for the MoE-layer forward -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct C. Only the tests, the smoke check and the benchmark's CPU
 * baseline load it; the product path never does. It shares no code, header or table with
 * the HIP library.
 *
 * Sources (the three pages on Mixture-of-Kittens, MoK):
 *   [P1-Overlap] "Overlapping compute and communication in MoE" section of the MoK write-up:
 *                DeepSeek-V3-style layer; a router projection picks the top-k routed experts
 *                and gives each a router weight; each picked expert runs up/gate projections,
 *                SwiGLU and a down projection; shared and routed outputs are combined with the
 *                router weights.
 *   [P1-Sched]   "Scheduling" section of the same write-up: the pull schedule {src_rank,
 *                src_index}, whose row index is the slot in the local destination buffer, is
 *                built with no sort by walking the routing results; its outputs are the token
 *                count per local expert, the count per (local expert, source rank), region
 *                offsets and the table.
 *   [P2-Method]  the Telegram summary, "Method and experiments": once each expert knows its
 *                tokens (e.g. after sorting) it pulls them; worked example T0->E2, T1->E7,
 *                T2->E2, T3->E5 and expert 2 takes [0,2,9,15], 5 takes [3,8], 7 takes [1,4,5,6].
 *   [P3]         the news summary: deterministic output, BF16 and MXFP8 support.
 *   MXFP8 itself is the OCP Microscaling Formats (MX) v1.0 specification (E4M3 elements,
 *   E8M0 shared scale per block of 32); the pages only name the format.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC (no FTZ). OpenMP
 * splits only independent rows; every element's arithmetic order is the sequential one
 * written here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ router logits
 * [P1-Overlap] router projection. The summation order is fixed so that the routing
 * decision (an integer) is reproducible: logits[t,e] = fma chain over i = 0..d-1 in
 * ascending order, starting from +0, in float32. */
void orc_router_logits(const float* x, const float* w_router, int64_t T, int32_t d,
                       int32_t E, float* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int32_t i = 0; i < d; ++i) acc = fmaf(x[t * d + i], w_router[(int64_t)e * d + i], acc);
      logits[t * E + e] = acc;
    }
  }
}

/* ------------------------------------------------------------------ top-k + weights
 * [P1-Overlap] top-k experts per token and a router weight for each.
 * Selection is on the logits (softmax is strictly increasing, so it picks the same
 * experts); a larger logit wins, equal logits go to the lower expert index (+0 == -0).
 * Slot j holds the j-th pick. Weights: the softmax over all E experts renormalised over
 * the k picks, which equals the softmax over the k picked logits:
 *   w_j = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0), in double, rounded to float. */
void orc_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx,
              float* topk_w) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    double lv[1024];
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict '>' keeps the lower index on ties */
      }
      taken[best] = 1;
      topk_idx[t * k + j] = best;
      lv[j] = (double)l[best];
    }
    double sum = 0.0;
    for (int32_t j = 0; j < k; ++j) sum += exp(lv[j] - lv[0]);
    for (int32_t j = 0; j < k; ++j) topk_w[t * k + j] = (float)(exp(lv[j] - lv[0]) / sum);
    free(taken);
  }
}

/* ------------------------------------------------------------------ dispatch plan
 * [P1-Sched] pull schedule for the local experts [e0, e0+E_l) of one rank.
 * Routes are numbered r = t*k + j (token t of the pool, slot j); the source rank of token t
 * is t / tokens_per_rank and its source index t % tokens_per_rank.
 * Walk the routing results in ascending r; every route whose expert is local is counted per
 * local expert and per (local expert, source rank). The region offsets are the exclusive
 * prefix sum of the per-expert counts. A second walk in the same order writes each local
 * route into the next free row of its expert's region, so rows within a region are in
 * ascending r = ascending (source rank, source index): no sort, a scan ("no sort needed").
 * route_ids[row] = r, from which {src_rank, src_index} = {(r/k)/tpr, (r/k)%tpr}.
 * Returns the number of local routes. */
int64_t orc_dispatch_plan(const int32_t* topk_idx, int64_t T, int32_t k, int32_t e0,
                          int32_t E_l, int32_t tokens_per_rank, int32_t* counts,
                          int32_t* offsets, int32_t* rank_counts, int32_t* route_ids) {
  const int64_t R = T / tokens_per_rank;
  for (int32_t e = 0; e < E_l; ++e) counts[e] = 0;
  for (int64_t q = 0; q < (int64_t)E_l * R; ++q) rank_counts[q] = 0;
  for (int64_t r = 0; r < T * k; ++r) {
    int32_t le = topk_idx[r] - e0;
    if (le < 0 || le >= E_l) continue;
    int64_t src_rank = (r / k) / tokens_per_rank;
    counts[le] += 1;
    rank_counts[(int64_t)le * R + src_rank] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E_l; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E_l > 0 ? E_l : 1));
  for (int32_t e = 0; e < E_l; ++e) next[e] = offsets[e];
  for (int64_t r = 0; r < T * k; ++r) {
    int32_t le = topk_idx[r] - e0;
    if (le < 0 || le >= E_l) continue;
    route_ids[next[le]++] = (int32_t)r;
  }
  free(next);
  return offsets[E_l];
}

/* ------------------------------------------------------------------ MXFP8 (OCP MX v1.0)
 * Element type E4M3 ("FN": bias 7, no infinities, max normal 448 = 1.75 * 2^8, min normal
 * 2^-6, subnormals m * 2^-9). One E8M0 scale per block of 32 consecutive elements along K.
 * Shared exponent s = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest normal),
 * clamped to [-127, 127]; amax == 0 gives s = -127. Scale byte = s + 127.
 * Element: a = |v| * 2^-s, rounded to nearest (ties to even mantissa) on the E4M3 grid,
 * then saturated to 448; the sign is kept (so -0 encodes as 0x80). */

static double e4m3_decode_mag(int code7) {
  int ex = (code7 >> 3) & 15, man = code7 & 7;
  if (ex == 0) return ldexp((double)man, -9);
  return ldexp(1.0 + man / 8.0, ex - 7);
}

/* Round a >= 0 to the E4M3 grid (RNE) and saturate; returns the 7-bit magnitude code. */
static int e4m3_encode_mag(double a) {
  if (a >= 448.0) return 0x7E;
  if (a == 0.0) return 0;
  int e = (int)floor(log2(a));
  /* log2 of a double can be off by one ulp near powers of two; fix e so 2^e <= a < 2^(e+1) */
  while (ldexp(1.0, e) > a) --e;
  while (ldexp(1.0, e + 1) <= a) ++e;
  if (e < -6) e = -6;                          /* subnormal binade shares the 2^-9 step */
  double quantum = ldexp(1.0, e - 3);
  double q = nearbyint(a / quantum) * quantum; /* default rounding mode: ties to even */
  if (q >= 448.0) return 0x7E;
  if (q == 0.0) return 0;
  if (q < ldexp(1.0, -6)) return (int)(q / ldexp(1.0, -9)); /* subnormal, exponent field 0 */
  int qe = (int)floor(log2(q));
  while (ldexp(1.0, qe) > q) --qe;
  while (ldexp(1.0, qe + 1) <= q) ++qe;
  int man = (int)((q / ldexp(1.0, qe) - 1.0) * 8.0);
  return ((qe + 7) << 3) | man;
}

uint8_t orc_e4m3_encode(float v, int32_t s) {
  double a = fabs((double)v) * ldexp(1.0, -s);
  int mag = e4m3_encode_mag(a);
  return (uint8_t)((signbit(v) ? 0x80 : 0) | mag);
}

float orc_e4m3_decode(uint8_t code) {
  double m = e4m3_decode_mag(code & 0x7F);
  return (float)((code & 0x80) ? -m : m);
}

int32_t orc_mx_shared_exponent(float amax) {
  if (amax == 0.0f) return -127;
  int ex;
  frexp((double)amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
  int s = (ex - 1) - 8;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return s;
}

void orc_mxfp8_quantize(const float* src, int64_t rows, int32_t K, uint8_t* codes,
                        uint8_t* scales) {
  const int32_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t b = 0; b < nb; ++b) {
      const float* v = src + r * K + (int64_t)b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
      }
      int32_t s = orc_mx_shared_exponent(amax);
      scales[r * nb + b] = (uint8_t)(s + 127);
      for (int i = 0; i < 32; ++i) codes[r * K + (int64_t)b * 32 + i] = orc_e4m3_encode(v[i], s);
    }
  }
}

void orc_mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t K,
                          float* out) {
  const int32_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t i = 0; i < K; ++i) {
      int s = (int)scales[r * nb + i / 32] - 127;
      out[r * K + i] = (float)ldexp((double)orc_e4m3_decode(codes[r * K + i]), s);
    }
}

/* ------------------------------------------------------------------ MXFP4 (OCP MX v1.0)
 * Element type E2M1 (FP4: sign, 2 exponent bits with bias 1, 1 mantissa bit; no infinities or
 * NaN). Its finite magnitudes are 0, 0.5 (the one subnormal), 1, 1.5, 2, 3, 4, 6; the largest
 * normal is 6 = 1.5 * 2^2, so the element's emax is 2. One E8M0 scale per block of 32 along K.
 * Shared exponent s = floor(log2(amax)) - 2, clamped to [-127, 127]; amax == 0 gives -127.
 * Element: a = |v| * 2^-s, rounded to the nearest E2M1 magnitude (a tie goes to the one with an
 * even mantissa bit), then saturated to 6; the sign is kept (-0 encodes as 0x8).
 * The MX format names the scale and the elements; how two 4-bit codes share a byte is a
 * storage choice: here element 2i is the low nibble of byte i and element 2i+1 the high one. */

static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Nearest magnitude by exhaustive search over the 8 codes; ties to the even code (the even
 * codes are the ones whose mantissa bit is 0). */
static int e2m1_encode_mag(double a) {
  if (a >= 6.0) return 7;
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    double dc = fabs(kE2M1[c] - a), db = fabs(kE2M1[best] - a);
    if (dc < db || (dc == db && (c & 1) == 0 && (best & 1) == 1)) best = c;
  }
  return best;
}

uint8_t orc_e2m1_encode(float v, int32_t s) {
  double a = fabs((double)v) * ldexp(1.0, -s);
  return (uint8_t)((signbit(v) ? 0x8 : 0) | e2m1_encode_mag(a));
}

float orc_e2m1_decode(uint8_t code) {
  double m = kE2M1[code & 7];
  return (float)((code & 8) ? -m : m);
}

int32_t orc_mx4_shared_exponent(float amax) {
  if (amax == 0.0f) return -127;
  int ex;
  frexp((double)amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
  int s = (ex - 1) - 2;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return s;
}

/* codes [rows, K/2] (two elements a byte, as above), scales [rows, K/32] */
void orc_mxfp4_quantize(const float* src, int64_t rows, int32_t K, uint8_t* codes,
                        uint8_t* scales) {
  const int32_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t b = 0; b < nb; ++b) {
      const float* v = src + r * K + (int64_t)b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
      }
      int32_t s = orc_mx4_shared_exponent(amax);
      scales[r * nb + b] = (uint8_t)(s + 127);
      for (int i = 0; i < 32; i += 2) {
        uint8_t lo = orc_e2m1_encode(v[i], s), hi = orc_e2m1_encode(v[i + 1], s);
        codes[r * (K / 2) + ((int64_t)b * 32 + i) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

void orc_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t K,
                          float* out) {
  const int32_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t i = 0; i < K; ++i) {
      int s = (int)scales[r * nb + i / 32] - 127;
      uint8_t byte = codes[r * (K / 2) + i / 2];
      uint8_t c = (i & 1) ? (byte >> 4) : (byte & 15);
      out[r * K + i] = (float)ldexp((double)orc_e2m1_decode(c), s);
    }
}
