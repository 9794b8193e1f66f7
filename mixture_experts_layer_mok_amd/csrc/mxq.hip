// Standalone MXFP8 quantisers for the weights, run before the layer:
//   k_quantize_mx   blocks of 32 along each row (the forward's operands): one wave per
//                   row, the same row quantiser the forward's dispatch uses;
//   k_quantize_mx_t blocks of 32 down each column, written transposed (the backward's
//                   operands, whose contraction runs over the stored rows).
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

// src [batch][rows][cols] bf16 -> codes [batch][cols][ldc] (code of src[b][r][c] at
// codes[b][c][r]) and scales [batch][cols][lds] (one per 32 consecutive r).  Thread
// (b, c, block q) reads the block's 32 values down column c (neighbouring threads read
// neighbouring columns: each load instruction reads contiguous bytes), takes the shared
// exponent of their largest magnitude and writes 32 codes and one scale.  The scaling
// and the conversion are those of the row quantiser (mx_shared_exp, e4m3x2), so the
// codes are those of mok_quantize_mx applied to the transposed matrix.
__global__ __launch_bounds__(256) void k_quantize_mx_t(const uint16_t* __restrict__ src,
                                                       int64_t batch, int rows, int cols,
                                                       uint8_t* __restrict__ codes, int64_t ldc,
                                                       uint8_t* __restrict__ scales,
                                                       int64_t lds) {
  const int nq = rows / 32;
  const int64_t n = batch * int64_t(nq) * cols;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * 256) {
    const int c = int(i % cols);
    const int64_t bq = i / cols;
    const int q = int(bq % nq);
    const int64_t b = bq / nq;
    const uint16_t* s0 = src + (b * rows + int64_t(q) * 32) * cols + c;
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      v[r] = bf16_to_f32(s0[int64_t(r) * cols]);
      amax = fmaxf(amax, fabsf(v[r]));
    }
    const int e = mx_shared_exp(amax);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = e4m3x2(ldexpf(v[4 * k], -e), ldexpf(v[4 * k + 1], -e)) |
             (e4m3x2(ldexpf(v[4 * k + 2], -e), ldexpf(v[4 * k + 3], -e)) << 16);
    uint8_t* d = codes + (b * cols + c) * ldc + int64_t(q) * 32;
    v4u* d16 = reinterpret_cast<v4u*>(d);
    d16[0] = v4u{w[0], w[1], w[2], w[3]};
    d16[1] = v4u{w[4], w[5], w[6], w[7]};
    scales[(b * cols + c) * lds + q] = uint8_t(e + 127);
  }
}

mok_status_t launch_quantize_mx_t(const uint16_t* src, int64_t batch, int32_t rows, int32_t cols,
                                  uint8_t* codes, int64_t ldc, uint8_t* scales, int64_t lds,
                                  hipStream_t st) {
  const int64_t n = batch * int64_t(rows / 32) * cols;
  if (n == 0) return MOK_OK;
  const unsigned grid = unsigned(std::min<int64_t>((n + 255) / 256, 65536));
  hipLaunchKernelGGL(k_quantize_mx_t, dim3(grid), dim3(256), 0, st, src, batch, int(rows),
                     int(cols), codes, ldc, scales, lds);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_E_LAUNCH;
}

// Weight scales with a row stride of K / 32 bytes, repacked to the tile's stride of one
// dword per 128-wide K step (used when K % 128 == 64); the pad byte is 127 (scale 1)
// and is never multiplied.
__global__ __launch_bounds__(256) void k_mx_repack(const uint8_t* __restrict__ src, int64_t rows,
                                                   int src_ld, uint8_t* __restrict__ dst,
                                                   int dst_ld) {
  const int64_t n = rows * dst_ld;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / dst_ld;
    const int c = int(i - r * dst_ld);
    dst[i] = c < src_ld ? src[r * src_ld + c] : uint8_t(127);
  }
}

void launch_mx_repack(const uint8_t* src, int64_t rows, int src_ld, uint8_t* dst, int dst_ld,
                      hipStream_t st) {
  const unsigned g = unsigned(std::min<int64_t>((rows * dst_ld + 255) / 256, 4096));
  if (g) hipLaunchKernelGGL(k_mx_repack, dim3(g), dim3(256), 0, st, src, rows, src_ld, dst, dst_ld);
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
