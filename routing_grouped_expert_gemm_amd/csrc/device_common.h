// Device-side helpers shared by the libmok kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOK_DEV __device__ __forceinline__
#define MOK_HOSTDEV __host__ __device__ __forceinline__

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

MOK_DEV float bf16_to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// float32 -> bf16, round to nearest even (NaN stays NaN): gfx950's v_cvt_pk_bf16_f32.
MOK_DEV bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two values in one 32-bit word (a in the low half), with one v_cvt_pk_bf16_f32.
MOK_DEV uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <class T> MOK_DEV float load_as_f32(const T* p);
template <> MOK_DEV float load_as_f32<float>(const float* p) { return *p; }
template <> MOK_DEV float load_as_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <class T> MOK_DEV T f32_to(float v);
template <> MOK_DEV float f32_to<float>(float v) { return v; }
template <> MOK_DEV bf16_t f32_to<bf16_t>(float v) { return f32_to_bf16(v); }

MOK_DEV int lane_id() { return __lane_id(); }

// v unchanged, but opaque to the optimiser: expressions of it are not hoisted or shared across
// this point.
MOK_DEV int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Block-wide exclusive scan of one int per thread (1024 threads = 16 waves). Returns the
// exclusive prefix; *total receives the sum. Each wave scans its 64 values with shuffles, wave
// 0 scans the 16 wave totals, and every lane adds its wave's base: two barriers.
MOK_DEV int32_t block_excl_scan_1024(int32_t v, int32_t* sh, int32_t* total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t a = __shfl_up(incl, off, 64);
    if (lane >= off) incl += a;
  }
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int32_t wt = lane < 16 ? sh[lane] : 0;
    int32_t wi = wt;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int32_t a = __shfl_up(wi, off, 64);
      if (lane >= off) wi += a;
    }
    if (lane < 16) sh[16 + lane] = wi - wt;        // exclusive wave bases
    if (lane == 15) sh[32] = wi;                    // block total
  }
  __syncthreads();
  const int32_t r = sh[16 + w] + incl - v;
  *total = sh[32];
  __syncthreads();                                  // sh is reused by the next call
  return r;
}

// Values every lane of the wave holds identically, moved to scalar registers.
MOK_DEV int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <class T>
MOK_DEV T* uniform_ptr(T* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

MOK_DEV uint64_t ballot(bool p) { return __ballot(p); }

MOK_DEV uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

MOK_DEV uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, kWave);
  hi = __shfl_xor(hi, m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// silu(z) = z / (1 + e^-z), with the hardware exp2 and reciprocal (~1 ulp each)
MOK_DEV float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ----------------------------------------------------------------------- MXFP8 (OCP MX)
// Shared exponent of a block from its absolute maximum: floor(log2(amax)) - EMAX, clamped to
// [-127, 127]; amax == 0 -> -127. EMAX is the exponent of the element type's largest normal: 8
// for E4M3 (448 = 1.75 * 2^8), 2 for E2M1 (6 = 1.5 * 2^2). Exact integer arithmetic on the
// float's fields.
template <int EMAX = 8>
MOK_DEV int mx_shared_exp(float amax) {
  uint32_t u = __float_as_uint(amax) & 0x7FFFFFFFu;
  if (u == 0) return -127;
  int e;
  if ((u >> 23) == 0) {                 // float32 subnormal: value = m * 2^-149
    e = 31 - __clz(u) - 149;           // floor(log2(m)) - 149
  } else {
    e = (int)(u >> 23) - 127;
  }
  int s = e - EMAX;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// E4M3 ("FN") code of v * 2^-s: round to nearest, ties to even, saturate to 448, keep sign.
// Integer-only: the float32's bits are re-rounded at the bit position of E4M3's step.
MOK_DEV uint32_t e4m3_encode(float v, int s) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a == 0) return sign;
  // unbiased exponent and 24-bit significand of |v| (subnormal floats handled)
  int ex;
  uint32_t sig;
  if ((a >> 23) == 0) {
    int lz = __clz(a) - 8;             // shift the leading one to bit 23
    sig = a << lz;
    ex = -126 - lz;
  } else {
    sig = (a & 0x7FFFFFu) | 0x800000u;
    ex = (int)(a >> 23) - 127;
  }
  int e = ex - s;                      // exponent of |v| * 2^-s
  if (e > 8) return sign | 0x7Eu;      // >= 512 -> saturate
  // step of the E4M3 grid in this binade: 2^(e-3) for e >= -6, 2^-9 below
  int step_e = (e >= -6 ? e : -6) - 3;
  // |v|*2^-s = sig * 2^(e-23); quantum index q = sig * 2^(e-23-step_e)
  int sh = 23 + step_e - e;            // right shift amount (>= 3)
  uint32_t q;
  if (sh >= 25) {
    q = 0;                             // below half a step: sig < 2^24 <= 2^(sh-1)
  } else {
    uint32_t kept = sig >> sh;
    uint32_t rem = sig & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1);
    q = kept + ((rem > half || (rem == half && (kept & 1u))) ? 1u : 0u);
  }
  // value = q * 2^step_e; encode
  if (q == 0) return sign;
  if (q < 8) return sign | q;          // only possible with step 2^-9: subnormal, field 0
  // normal: value = q * 2^step_e with q in [8, 16]; q == 16 carries into the next binade
  int ef = step_e + 3 + 7;             // exponent field for q in [8, 16)
  if (q == 16) { q = 8; ef += 1; }
  if (ef > 15 || (ef == 15 && q > 14)) return sign | 0x7Eu;  // > 448 -> 448
  return sign | ((uint32_t)ef << 3) | (q - 8);
}

// Eight consecutive elements (one 16-byte load of bf16) of a 32-element block held by one lane;
// the block's four lanes are an aligned quad (lanes 4g .. 4g + 3). The shared exponent comes
// from the quad's amax; each element is |v| * 2^-s clamped to 448, then rounded to nearest even
// on the E4M3 grid by the hardware conversion (for a value that rounds past 448, rounding the
// clamped value gives 448 as well, so the clamp implements the saturation rule). 2^-s is
// applied with ldexp, which is exact wherever the result can round to a nonzero code.
// Returns the 8 codes (little-endian) and the block's shared exponent.
MOK_DEV uint2 quantize_quad8(const uint4 raw, int* s_out) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(w[q] << 16);
    v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  const int s = mx_shared_exp(amax);
  float y[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) y[q] = fminf(fmaxf(__builtin_amdgcn_ldexpf(v[q], -s), -448.0f), 448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  *s_out = s;
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// The same rules for sixteen bf16 values per lane, the 2 lanes of an aligned pair holding one
// 32-element block (the even lane the first half): the 16 codes, and the block's exponent.
MOK_DEV uint4 quantize_pair16(const uint4 raw0, const uint4 raw1, int* s_out) {
  const uint32_t w[8] = {raw0.x, raw0.y, raw0.z, raw0.w, raw1.x, raw1.y, raw1.z, raw1.w};
  float v[16];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    v[2 * q] = __uint_as_float(w[q] << 16);
    v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fabsf(v[q]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  const int s = mx_shared_exp(amax);
  uint32_t c[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      y[r] = fminf(fmaxf(__builtin_amdgcn_ldexpf(v[4 * q + r], -s), -448.0f), 448.0f);
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
    c[q] = (uint32_t)word;
  }
  *s_out = s;
  return make_uint4(c[0], c[1], c[2], c[3]);
}

// quantize_quad8 for eight float32 values already in registers (same rules).
MOK_DEV uint2 quantize_quad8_f32(const float (&v)[8], int* s_out) {
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  const int s = mx_shared_exp(amax);
  float y[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) y[q] = fminf(fmaxf(__builtin_amdgcn_ldexpf(v[q], -s), -448.0f), 448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  *s_out = s;
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// ----------------------------------------------------------------------- MXFP4 (OCP MX)
// E2M1 codes (sign in bit 3) of y = v * 2^-s, which the caller forms exactly: the nearest of
// the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a tie going to the even code, and everything
// past 6 saturating to 6. gfx950's conversion (v_cvt_scalef32_pk_fp4_f32, scale 1) implements
// exactly this rule: checked against comparisons with the midpoints (0.25, 0.75, 1.25, 1.75,
// 2.5, 3.5, 5; the even neighbour decides a tie) on every bf16 pattern times 2^k (k = -12 ..
// 12) and on every float32 within 2^20 ulps of a midpoint, 0 or 6, both signs, with no
// difference. Two elements a byte, element 2i in the low nibble of byte i.
MOK_DEV uint32_t pack_e2m1x8(const float (&y)[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// MXFP4 of eight values held by one lane of an aligned quad (a 32-element block over 4 lanes):
// the 8 codes (4 bytes) and the block's shared exponent (emax 2). v * 2^-s is exact (ldexp of
// a value whose result can reach a nonzero code is a normal float).
MOK_DEV uint32_t mx4_quad8_f32(const float (&v)[8], int* s_out) {
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  const int s = mx_shared_exp<2>(amax);
  float y[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) y[q] = __builtin_amdgcn_ldexpf(v[q], -s);
  *s_out = s;
  return pack_e2m1x8(y);
}

MOK_DEV uint32_t mx4_quad8(const uint4 raw, int* s_out) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(w[q] << 16);
    v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
  }
  return mx4_quad8_f32(v, s_out);
}

// Sixteen bf16 values a lane, the 2 lanes of an aligned pair holding one 32-element block:
// the 16 codes (8 bytes) and the block's shared exponent.
MOK_DEV uint2 mx4_pair16(const uint4 raw0, const uint4 raw1, int* s_out) {
  const uint32_t w[8] = {raw0.x, raw0.y, raw0.z, raw0.w, raw1.x, raw1.y, raw1.z, raw1.w};
  float v[16];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    v[2 * q] = __uint_as_float(w[q] << 16);
    v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fabsf(v[q]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  const int s = mx_shared_exp<2>(amax);
  float lo[8], hi[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    lo[q] = __builtin_amdgcn_ldexpf(v[q], -s);
    hi[q] = __builtin_amdgcn_ldexpf(v[8 + q], -s);
  }
  *s_out = s;
  return make_uint2(pack_e2m1x8(lo), pack_e2m1x8(hi));
}
