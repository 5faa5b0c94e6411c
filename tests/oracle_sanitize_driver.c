/* Drives every function of oracle/mok_oracle.c on small inputs, edge cases included, so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer checks the oracle's own memory
 * accesses and arithmetic. Prints one summary line; any sanitizer report aborts the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_router_logits(const float*, const float*, int64_t, int32_t, int32_t, float*);
void orc_topk(const float*, int64_t, int32_t, int32_t, int32_t*, float*);
int64_t orc_dispatch_plan(const int32_t*, int64_t, int32_t, int32_t, int32_t, int32_t, int32_t*,
                          int32_t*, int32_t*, int32_t*);
uint8_t orc_e4m3_encode(float, int32_t);
float orc_e4m3_decode(uint8_t);
int32_t orc_mx_shared_exponent(float);
void orc_mxfp8_quantize(const float*, int64_t, int32_t, uint8_t*, uint8_t*);
void orc_mxfp8_dequantize(const uint8_t*, const uint8_t*, int64_t, int32_t, float*);
uint8_t orc_e2m1_encode(float, int32_t);
float orc_e2m1_decode(uint8_t);
int32_t orc_mx4_shared_exponent(float);
void orc_mxfp4_quantize(const float*, int64_t, int32_t, uint8_t*, uint8_t*);
void orc_mxfp4_dequantize(const uint8_t*, const uint8_t*, int64_t, int32_t, float*);

static float frand(unsigned* s) {
  *s = *s * 1664525u + 1013904223u;
  return ((float)(*s >> 8) / 16777216.0f - 0.5f) * 6.0f;
}

int main(void) {
  unsigned seed = 1;
  enum { T = 37, D = 64, E = 9, K = 3, TPR = 37 };
  float* x = malloc(sizeof(float) * T * D);
  float* w = malloc(sizeof(float) * E * D);
  float* lg = malloc(sizeof(float) * T * E);
  for (int i = 0; i < T * D; ++i) x[i] = frand(&seed);
  for (int i = 0; i < E * D; ++i) w[i] = frand(&seed);
  orc_router_logits(x, w, T, D, E, lg);
  lg[0] = lg[1];                                    /* a tie */
  int32_t* idx = malloc(sizeof(int32_t) * T * E);
  float* tw = malloc(sizeof(float) * T * E);
  orc_topk(lg, T, E, K, idx, tw);
  orc_topk(lg, T, E, E, idx, tw);                   /* k = E */
  orc_topk(lg, T, E, K, idx, tw);
  int32_t counts[E], offsets[E + 1], rank_counts[E], route_ids[T * K];
  int64_t n = orc_dispatch_plan(idx, T, K, 0, E, TPR, counts, offsets, rank_counts, route_ids);
  int64_t n2 = orc_dispatch_plan(idx, T, K, 4, 2, TPR, counts, offsets, rank_counts, route_ids);
  int64_t n0 = orc_dispatch_plan(idx, 0, K, 0, E, TPR, counts, offsets, rank_counts, route_ids);
  /* MX codecs: random, zero, tiny and huge blocks */
  enum { R = 5, KK = 96 };
  float* v = malloc(sizeof(float) * R * KK);
  float* back = malloc(sizeof(float) * R * KK);
  for (int i = 0; i < R * KK; ++i) v[i] = frand(&seed);
  for (int i = 0; i < KK; ++i) v[i] = 0.0f;
  for (int i = KK; i < 2 * KK; ++i) v[i] = ldexpf(v[i], -140);
  for (int i = 2 * KK; i < 3 * KK; ++i) v[i] = ldexpf(v[i], 120);
  uint8_t* c8 = malloc((size_t)R * KK);
  uint8_t* c4 = malloc((size_t)R * KK / 2);
  uint8_t* sc = malloc((size_t)R * KK / 32);
  orc_mxfp8_quantize(v, R, KK, c8, sc);
  orc_mxfp8_dequantize(c8, sc, R, KK, back);
  orc_mxfp4_quantize(v, R, KK, c4, sc);
  orc_mxfp4_dequantize(c4, sc, R, KK, back);
  int acc = 0;
  for (int c = 0; c < 256; ++c) acc += (int)orc_e4m3_decode((uint8_t)c) != 0;
  for (int c = 0; c < 16; ++c) acc += (int)orc_e2m1_decode((uint8_t)c) != 0;
  for (int s = -127; s <= 127; s += 7) {
    acc += orc_e4m3_encode(1.0f, s) + orc_e2m1_encode(-3.0f, s);
    acc += orc_mx_shared_exponent(ldexpf(1.0f, s)) + orc_mx4_shared_exponent(ldexpf(1.5f, s));
  }
  acc += orc_mx_shared_exponent(0.0f) + orc_mx4_shared_exponent(1e-45f);
  printf("oracle sanitize run ok: routes %lld %lld %lld, check %d\n", (long long)n,
         (long long)n2, (long long)n0, acc);
  free(x); free(w); free(lg); free(idx); free(tw); free(v); free(back); free(c8); free(c4);
  free(sc);
  return 0;
}
