// Standalone MXFP8 quantiser (used for the weights before a MXFP8 forward): every lane
// encodes one 32-element block, so a wave reads 64 consecutive blocks (4 KB) and writes
// 2 KB of codes plus 64 scale bytes, all coalesced.
#include <algorithm>

#include "launch.h"
#include "mx.h"

namespace mok {

__global__ __launch_bounds__(256) void k_quantize_mx(const uint16_t* __restrict__ src,
                                                     int64_t nblocks, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  for (int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x; b < nblocks;
       b += int64_t(gridDim.x) * 256)
    scales[b] = mx_block_bf16(src + b * 32, codes + b * 32);
}

mok_status_t launch_quantize_mx(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes,
                                uint8_t* scales, hipStream_t st) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return MOK_OK;
  const unsigned grid = unsigned(std::min<int64_t>((nblocks + 255) / 256, 65536));
  hipLaunchKernelGGL(k_quantize_mx, dim3(grid), dim3(256), 0, st, src, nblocks, codes, scales);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_E_LAUNCH;
}

}  // namespace mok
