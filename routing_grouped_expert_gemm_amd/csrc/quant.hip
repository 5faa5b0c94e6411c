// MX operands (OCP Microscaling Formats v1.0: one E8M0 scale per block of 32 along K). The
// news summary of MoK says the kernel supports BF16 and MXFP8; MXFP4 is the 4-bit member of the
// same family (the MoK write-up mentions earlier MXFP8 and NVFP4 training kernels). The rules
// come from the OCP specification: shared exponent floor(log2(amax)) - emax (8 for E4M3, 2 for
// E2M1), elements rounded to nearest-even on the element grid and saturated at its maximum
// (448, 6).
//
// HBM streams: four lanes per 32-element block, each lane 16 bytes of bf16 in, 8 code bytes out,
// the quad's first lane writing the scale byte; a wave covers 1 KB of contiguous input.
#include "device_common.h"
#include "launch.h"

namespace mok {

// Row-major scales (the mok_quantize_mx* layout): four lanes per 32-element block, 8 elements a
// lane. K-step-major scales (the GEMMs' operands): a wave quantises one 128-element K step of 8
// consecutive rows, 8 lanes a row and 16 elements a lane (two lanes a block), so its 32 scale
// bytes -- 8 K-step-major words of consecutive rows -- are contiguous, and each lane reads 32
// bytes and writes 16 (MXFP8) or 8 (MXFP4). FP4: E2M1 codes, two a byte (MXFP4).
template <bool KMAJOR, bool FP4>
__global__ __launch_bounds__(256) void k_quantize_mx(const bf16_t* __restrict__ src, int64_t rows,
                                                     int K, int64_t R, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int64_t n_chunks = KMAJOR ? (rows + 7) / 8 * (K / 128) * 64 : rows * (K / 8);
  const int64_t stride = (int64_t)gridDim.x * 256;
  // every lane of a wave runs the same number of iterations (the quad / pair shuffles need the
  // whole group): lanes past the end load and store nothing
  const int64_t n_iter = (n_chunks + stride - 1) / stride;
  int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int64_t it = 0; it < n_iter; ++it, q += stride) {
    if constexpr (KMAJOR) {
      const uint32_t unit = (uint32_t)(q >> 6);   // 8 rows x one K step (< 2^31 units)
      const uint32_t steps = (uint32_t)K / 128, li = (uint32_t)q & 63;
      const uint32_t rg = unit / steps;
      const int j = (int)(unit - rg * steps);
      const int64_t row = (int64_t)rg * 8 + (li >> 3);
      const int c16 = j * 8 + (int)(li & 7);      // the lane's 16-element chunk of the row
      const bool ok = q < n_chunks && row < rows;
      const int64_t at = row * K + 16 * c16;
      uint4 r0 = make_uint4(0, 0, 0, 0), r1 = r0;
      if (ok) {
        r0 = *(const uint4*)(src + at);
        r1 = *(const uint4*)(src + at + 8);
      }
      int sh;
      if constexpr (FP4) {
        const uint2 c = mx4_pair16(r0, r1, &sh);
        if (ok) *(uint2*)(codes + at / 2) = c;
      } else {
        const uint4 c = quantize_pair16(r0, r1, &sh);
        if (ok) *(uint4*)(codes + at) = c;
      }
      if (ok && (c16 & 1) == 0) {
        const int64_t g = (uint32_t)row / (uint32_t)R;   // matrix g, its row row - g R
        scales[g * R * (K / 32) + mx_kmajor_scale(row - g * R, c16 >> 1, R)] = (uint8_t)(sh + 127);
      }
    } else {
      const bool ok = q < n_chunks;
      const int64_t at = q * 8;
      const uint4 raw = ok ? *(const uint4*)(src + at) : make_uint4(0, 0, 0, 0);
      int sh;
      if constexpr (FP4) {
        const uint32_t c = mx4_quad8(raw, &sh);
        if (ok) *(uint32_t*)(codes + at / 2) = c;
      } else {
        const uint2 c = quantize_quad8(raw, &sh);
        if (ok) *(uint2*)(codes + at) = c;
      }
      if (ok && (q & 3) == 0) scales[at >> 5] = (uint8_t)(sh + 127);
    }
  }
}

// Float32 rows, row-major scales: the encoders the gate/up epilogue applies to H in float32
// (quantize_quad8_f32, mx4_quad8_f32), four lanes a 32-element block, 8 elements a lane.
template <bool FP4>
__global__ __launch_bounds__(256) void k_quantize_mx_f32(const float* __restrict__ src, int64_t rows,
                                                         int K, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  const int64_t n_chunks = rows * (K / 8);
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t n_iter = (n_chunks + stride - 1) / stride;   // the same for every lane
  int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int64_t it = 0; it < n_iter; ++it, q += stride) {
    const bool ok = q < n_chunks;
    const int64_t at = q * 8;
    float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (ok) {
      const float4 a = *(const float4*)(src + at), b = *(const float4*)(src + at + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    int sh;
    if constexpr (FP4) {
      const uint32_t c = mx4_quad8_f32(v, &sh);
      if (ok) *(uint32_t*)(codes + at / 2) = c;
    } else {
      const uint2 c = quantize_quad8_f32(v, &sh);
      if (ok) *(uint2*)(codes + at) = c;
    }
    if (ok && (q & 3) == 0) scales[at >> 5] = (uint8_t)(sh + 127);
  }
}

hipError_t launch_quantize_mx_f32(const float* src, int64_t rows, int K, uint8_t* codes,
                                  uint8_t* scales, bool fp4, hipStream_t s) {
  const int64_t n_chunks = rows * (K / 8);
  if (n_chunks == 0) return hipSuccess;
  const int64_t want = (n_chunks + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  if (fp4)
    launch_k(k_quantize_mx_f32<true>, dim3(grid), dim3(256), 0, s, nullptr, nullptr, src, rows, K,
             codes, scales);
  else
    launch_k(k_quantize_mx_f32<false>, dim3(grid), dim3(256), 0, s, nullptr, nullptr, src, rows, K,
             codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const void* src_bf16, int64_t rows, int K, uint8_t* codes,
                              uint8_t* scales, bool fp4, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1, int64_t scales_kmajor) {
  const int64_t n_chunks = scales_kmajor > 0 ? (rows + 7) / 8 * (K / 128) * 64 : rows * (K / 8);
  if (n_chunks == 0) return mark_empty(s, e0, e1), hipSuccess;
  if (scales_kmajor > 0 && (rows >= INT32_MAX || n_chunks / 64 >= INT32_MAX))
    return hipErrorInvalidValue;                  // the K-major index math is 32-bit
  const int64_t want = (n_chunks + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  const bf16_t* src = (const bf16_t*)src_bf16;
  const int64_t R = scales_kmajor > 0 ? scales_kmajor : 0;
  if (scales_kmajor > 0 && fp4)
    launch_k(k_quantize_mx<true, true>, dim3(grid), dim3(256), 0, s, e0, e1, src, rows, K, R,
             codes, scales);
  else if (scales_kmajor > 0)
    launch_k(k_quantize_mx<true, false>, dim3(grid), dim3(256), 0, s, e0, e1, src, rows, K, R,
             codes, scales);
  else if (fp4)
    launch_k(k_quantize_mx<false, true>, dim3(grid), dim3(256), 0, s, e0, e1, src, rows, K, R,
             codes, scales);
  else
    launch_k(k_quantize_mx<false, false>, dim3(grid), dim3(256), 0, s, e0, e1, src, rows, K, R,
             codes, scales);
  return hipGetLastError();
}

}  // namespace mok
