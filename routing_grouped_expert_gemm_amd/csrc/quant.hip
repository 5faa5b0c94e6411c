// MXFP8 operands (OCP Microscaling Formats v1.0: E4M3 elements, one E8M0 scale per block of
// 32 along K). The news summary of MoK says the kernel supports BF16 and MXFP8; the format's
// rules come from the OCP specification: shared exponent floor(log2(amax)) - 8, elements
// rounded to nearest-even on the E4M3 grid and saturated at 448.
//
// Both kernels are HBM streams: each thread turns one 32-element block (64 B of bf16) into
// 32 code bytes and one scale byte; neighbouring threads take neighbouring blocks.
#include "device_common.h"
#include "launch.h"

namespace mok {

__global__ __launch_bounds__(256) void k_quantize_mxfp8(const bf16_t* __restrict__ src,
                                                        int64_t n_blocks,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < n_blocks; b += stride)
    quantize_block32(src + b * 32, codes + b * 32, scales + b);
}

hipError_t launch_quantize_mxfp8(const void* src_bf16, int64_t rows, int K, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s) {
  const int64_t n_blocks = rows * (K / 32);
  if (n_blocks == 0) return hipSuccess;
  const int64_t want = (n_blocks + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(k_quantize_mxfp8, dim3(grid), dim3(256), 0, s, (const bf16_t*)src_bf16,
                     n_blocks, codes, scales);
  return hipGetLastError();
}

}  // namespace mok
