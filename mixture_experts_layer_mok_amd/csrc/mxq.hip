// Standalone MXFP8 quantiser (the weights before a MXFP8 forward): one wave per row,
// blocks of 32 along the row, the same row quantiser the forward's dispatch uses.
#include <algorithm>

#include "launch.h"
#include "mx.h"

namespace mok {

__global__ __launch_bounds__(256) void k_quantize_mx(const uint16_t* __restrict__ src,
                                                     int64_t rows, int cols,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int64_t nw = int64_t(gridDim.x) * 4;
  for (int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6); r < rows; r += nw)
    wave_quant_row<false>(codes + r * cols, scales + r * (cols / 32), src + r * cols, cols);
}

mok_status_t launch_quantize_mx(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes,
                                uint8_t* scales, hipStream_t st) {
  if (rows == 0) return MOK_OK;
  const unsigned grid = unsigned(std::min<int64_t>((rows + 3) / 4, 65536));
  hipLaunchKernelGGL(k_quantize_mx, dim3(grid), dim3(256), 0, st, src, rows, int(cols), codes,
                     scales);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_E_LAUNCH;
}

}  // namespace mok
