// Integer geometry of the GEMM tile's direct-to-LDS loads, shared by the kernels and by
// a host-side bounds check (tile_bounds_check.cpp) that verifies every offset the
// kernels can form stays inside its operand.
#pragma once
#include <stdint.h>

#ifndef MOK_HD
#if defined(__HIPCC__)
#define MOK_HD __host__ __device__
#else
#define MOK_HD
#endif
#endif

namespace mok {
namespace geom {

// The tile's workgroup has 8 waves; each operand stage is 256 rows x 8 chunks of 16
// bytes, loaded by 4 direct-to-LDS loads per wave.  Tile row loaded by load p (0..3) of
// wave w (0..7), lane l (0..63): rows (8p + w) * 8 + l/8.
constexpr int kLoads = 4;
constexpr int kWaves = 8;
MOK_HD inline int dma_row(int p, int w, int l) { return (p * 8 + w) * 8 + (l >> 3); }
// Logical 16-byte chunk of that lane (inverse of the LDS swizzle at its position).
MOK_HD inline int dma_chunk(int w, int l) { return (l & 7) ^ ((l >> 3) & 7) ^ (w & 1); }

// Byte offset of the A chunk from the tile's first A row (rows past rows_valid are
// clamped to the last valid row).
MOK_HD inline int64_t a_offset(int p, int w, int l, int rows_valid, int64_t lda) {
  int r = dma_row(p, w, l);
  if (r > rows_valid - 1) r = rows_valid - 1;
  return (int64_t(r) * lda + dma_chunk(w, l) * 8) * 2;
}

// B tile row layouts.
//   kSplit: tile rows 0..127 are rows nb0.. of B0, rows 128..255 rows nb1.. of B1
//           (GEMM2: two consecutive 128-row blocks of W_down).
//   kPaired: every 32-row MFMA block b holds rows nb0 + 16 b .. +15 of B0 (gate) in its
//           first 16 rows and the same rows of B1 (up) in its last 16, so one MFMA
//           output block holds 16 gate columns and their 16 up columns (GEMM1).
enum BLayout { kSplit = 0, kPaired = 1 };

// Matrix (0 = B0, 1 = B1) and row (clamped to N - 1) of B tile row r (0..255).
MOK_HD inline int b_matrix_of_row(int layout, int r) {
  return layout == kPaired ? ((r >> 4) & 1) : (r < 128 ? 0 : 1);
}
MOK_HD inline int b_row_of_row(int layout, int r, int nb0, int nb1, int N) {
  int rb;
  if (layout == kPaired) rb = nb0 + (r >> 5) * 16 + (r & 15);
  else rb = (r < 128) ? nb0 + r : nb1 + r - 128;
  return rb > N - 1 ? N - 1 : rb;
}

// Matrix and row of the B chunk of load p, wave w, lane l.  For the paired layout the
// half of the 32-row block, (r / 16) % 2, is (w / 2) % 2: wave-uniform; for the split
// layout the matrix is fixed per load p.
MOK_HD inline int b_matrix(int layout, int p, int w) {
  return layout == kPaired ? ((w >> 1) & 1) : (p < 2 ? 0 : 1);
}
MOK_HD inline int b_row(int layout, int p, int w, int l, int nb0, int nb1, int N) {
  return b_row_of_row(layout, dma_row(p, w, l), nb0, nb1, N);
}
// Byte offset of the B chunk from the start of its weight matrix (rows clamped to N - 1).
MOK_HD inline int64_t b_offset(int layout, int p, int w, int l, int nb0, int nb1, int N,
                               int64_t ldb) {
  return (int64_t(b_row(layout, p, w, l, nb0, nb1, N)) * ldb + dma_chunk(w, l) * 8) * 2;
}

// K-major operands (the backward reads weights and routed-row matrices as stored, with
// K running over their rows): a stage holds 64 K rows of 256 tile columns, 32 chunks of
// 16 bytes per row, logical chunk c of stage row kk at position c ^ (4 (kk & 3)).  Load p
// of wave w, lane l fills stage row (8p + w) * 2 + l / 32 at position l % 32; kk & 3
// depends on w and l only.
MOK_HD inline int km_row(int p, int w, int l) { return (p * 8 + w) * 2 + (l >> 5); }
MOK_HD inline int km_chunk(int w, int l) { return (l & 31) ^ (4 * (((w << 1) + (l >> 5)) & 3)); }
// First tile column of that chunk, clamped so that its 8 columns stay below N (columns
// past N are never stored).
MOK_HD inline int km_col(int w, int l, int n0, int N) {
  const int c = n0 + 8 * km_chunk(w, l);
  return c > N - 8 ? N - 8 : c;
}

// MXFP8 tiles: one K step is 128 code bytes per row (8 chunks: the same direct-to-LDS
// geometry, with rows of ld / 2 two-byte units) plus one dword of 4 e8m0 scales per
// row.  Lanes of waves 0-3 load the scale dword of A tile row (w % 4) * 64 + l, lanes
// of waves 4-7 that of B tile row (w % 4) * 64 + l.  Scale rows are s_ld bytes apart
// (a multiple of 4); the dword of step ks sits at byte 4 ks of its row.
MOK_HD inline int mx_scale_row(int w, int l) { return (w & 3) * 64 + l; }
MOK_HD inline int64_t mx_a_scale_offset(int w, int l, int rows_valid, int64_t s_ld) {
  int r = mx_scale_row(w, l);
  if (r > rows_valid - 1) r = rows_valid - 1;
  return int64_t(r) * s_ld;
}
MOK_HD inline int64_t mx_b_scale_offset(int layout, int w, int l, int nb0, int nb1, int N,
                                        int64_t s_ld) {
  return int64_t(b_row_of_row(layout, mx_scale_row(w, l), nb0, nb1, N)) * s_ld;
}
// On a half step (K % 128 == 64, the last step) only chunks 0..3 of each row load.
MOK_HD inline bool mx_chunk_in_half(int w, int l) { return dma_chunk(w, l) < 4; }

}  // namespace geom
}  // namespace mok
