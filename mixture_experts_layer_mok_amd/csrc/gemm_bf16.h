// bf16 grouped-GEMM tile for gfx950: one workgroup (4 waves) computes a 128 x 256
// fp32 tile C = A * B^T with A [rows, K] and B [256 rows, K] both K-contiguous, using
// v_mfma_f32_32x32x16_bf16.  Each wave owns 64 rows x 128 columns (2 x 4 MFMA blocks).
//
// The 256 B rows come from two 128-row halves (B0, B1) so the same tile serves
//   GEMM1: B0 = W_gate rows, B1 = W_up rows of the same 128 intermediate columns
//          (the SwiGLU epilogue pairs gate and up values held by the same lane);
//   GEMM2: B0, B1 = two consecutive 128-row blocks of W_down.
//
// Global -> LDS: 16-byte chunks, 8 threads per 128-byte row segment (coalesced), double
// buffered through registers so the next K step's loads are in flight during the
// current step's MFMAs.  LDS rows are 64 bf16 = 8 chunks; chunk c of row r is stored at
// position c ^ (r & 7), so the 32 rows read by one MFMA operand fetch spread over all
// banks and the 8 threads writing one row segment hit 8 distinct chunk positions.
// Rows past the valid range are clamped to the last valid row (always in bounds);
// their results are never stored.
#pragma once
#include "device.h"

namespace mok {

struct TileSmem {
  v4u a[2][kBM * 8];   // 2 x 16 KB
  v4u b[2][256 * 8];   // 2 x 32 KB
};

__device__ __forceinline__ int lds_chunk(int r, int c) { return r * 8 + (c ^ (r & 7)); }

struct TileAcc {
  f32x16_t c[2][4];
};

// Row pointers of this thread's load assignments.
struct TileSrc {
  const uint16_t* pa[4];
  const uint16_t* pb[8];
};

__device__ __forceinline__ void tile_src_init(TileSrc& s, const uint16_t* A, int64_t lda,
                                              int rows_valid, const uint16_t* B0,
                                              const uint16_t* B1, int64_t ldb, int nb0, int nb1,
                                              int N) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = min(p * 32 + (t >> 3), rows_valid - 1);
    s.pa[p] = A + int64_t(r) * lda + c * 8;
  }
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = p * 32 + (t >> 3);
    if (r < 128) {
      s.pb[p] = B0 + int64_t(min(nb0 + r, N - 1)) * ldb + c * 8;
    } else {
      s.pb[p] = B1 + int64_t(min(nb1 + r - 128, N - 1)) * ldb + c * 8;
    }
  }
}

struct TileRegs {
  v4u a[4];
  v4u b[8];
};

__device__ __forceinline__ void tile_load(TileRegs& r, const TileSrc& s, int k0) {
#pragma unroll
  for (int p = 0; p < 4; ++p) r.a[p] = *reinterpret_cast<const v4u*>(s.pa[p] + k0);
#pragma unroll
  for (int p = 0; p < 8; ++p) r.b[p] = *reinterpret_cast<const v4u*>(s.pb[p] + k0);
}

__device__ __forceinline__ void tile_store(TileSmem& sm, int buf, const TileRegs& r) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int p = 0; p < 4; ++p) sm.a[buf][lds_chunk(p * 32 + (t >> 3), c)] = r.a[p];
#pragma unroll
  for (int p = 0; p < 8; ++p) sm.b[buf][lds_chunk(p * 32 + (t >> 3), c)] = r.b[p];
}

// B row (within the 256-row tile) of MFMA block j for wave column wn.
__device__ __forceinline__ int brow_of(int j, int wn) {
  return (j < 2) ? (wn * 64 + j * 32) : (128 + wn * 64 + (j - 2) * 32);
}

__device__ __forceinline__ void tile_compute(const TileSmem& sm, int buf, TileAcc& acc) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int r32 = lane & 31;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = ks * 2 + (lane >> 5);
    v4u a[2], b[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = sm.a[buf][lds_chunk(wm * 64 + i * 32 + r32, c)];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = sm.b[buf][lds_chunk(brow_of(j, wn) + r32, c)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc.c[i][j] = mfma32x32x16(a[i], b[j], acc.c[i][j]);
  }
}

// Full K loop.  K is a multiple of kBK.
__device__ __forceinline__ void tile_gemm(TileSmem& sm, const TileSrc& src, int K, TileAcc& acc) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.f;
  const int nk = K / kBK;
  TileRegs regs;
  tile_load(regs, src, 0);
  tile_store(sm, 0, regs);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nk) tile_load(regs, src, (kb + 1) * kBK);
    tile_compute(sm, buf, acc);
    if (kb + 1 < nk) tile_store(sm, buf ^ 1, regs);
    __syncthreads();
  }
}

// Row (within the 128-row tile) held by accumulator element v of block i for this lane.
__device__ __forceinline__ int acc_row(int i, int v) {
  const int lane = threadIdx.x & 63;
  const int wm = (threadIdx.x >> 6) >> 1;
  return wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

}  // namespace mok
