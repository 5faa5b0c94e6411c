// MXFP8 operands (OCP Microscaling Formats v1.0: E4M3 elements, one E8M0 scale per block of
// 32 along K). The news summary of MoK says the kernel supports BF16 and MXFP8; the format's
// rules come from the OCP specification: shared exponent floor(log2(amax)) - 8, elements
// rounded to nearest-even on the E4M3 grid and saturated at 448.
//
// HBM streams: four lanes per 32-element block, each lane 16 bytes of bf16 in, 8 code bytes out,
// the quad's first lane writing the scale byte; a wave covers 1 KB of contiguous input.
#include "device_common.h"
#include "launch.h"

namespace mok {

__global__ __launch_bounds__(256) void k_quantize_mxfp8(const bf16_t* __restrict__ src,
                                                        int64_t n_chunks,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  // every lane of a wave runs the same number of iterations (the quad shuffles need the whole
  // quad): lanes past the end load and store nothing
  const int64_t n_iter = (n_chunks + stride - 1) / stride;
  int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int64_t it = 0; it < n_iter; ++it, q += stride) {
    const bool ok = q < n_chunks;
    const uint4 raw = ok ? *(const uint4*)(src + q * 8) : make_uint4(0, 0, 0, 0);
    int sh;
    const uint2 c = quantize_quad8(raw, &sh);
    if (ok) {
      *(uint2*)(codes + q * 8) = c;
      if ((q & 3) == 0) scales[q >> 2] = (uint8_t)(sh + 127);
    }
  }
}

hipError_t launch_quantize_mxfp8(const void* src_bf16, int64_t rows, int K, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int64_t n_chunks = rows * (K / 8);
  if (n_chunks == 0) return mark_empty(s, e0, e1), hipSuccess;
  const int64_t want = (n_chunks + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  launch_k(k_quantize_mxfp8, dim3(grid), dim3(256), 0, s, e0, e1, (const bf16_t*)src_bf16,
           n_chunks, codes, scales);
  return hipGetLastError();
}

}  // namespace mok
