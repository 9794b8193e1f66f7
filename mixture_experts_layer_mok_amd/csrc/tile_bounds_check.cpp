// Host-side check that every direct-to-LDS offset the GEMM tile forms stays inside its
// operand, for given hidden (D) and intermediate (I) sizes, over every tile shape the
// kernels launch: GEMM1 (A = [rows, D], B0 = W_gate, B1 = W_up: [I, D], columns n0..n0+127
// of both), GEMM2 (A = [rows, I], B0 = B1 = W_down: [D, I], columns n0..n0+255), any
// row count 1..256, and that the paired layout covers each gate/up row exactly once.  Built with the host compiler only; exits non-zero on a violation.
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "tile_geom.h"

static const int kBK = 64, kBM = 256, kBN1 = 128, kBN2 = 256;

static int check(const char* what, int layout, int K, int64_t lda, int64_t ldb, int N, int n0,
                 int nb1, int rows) {
  const int64_t a_bytes = int64_t(rows) * lda * 2;
  const int64_t b_bytes = int64_t(N) * ldb * 2;
  const int64_t k_last = int64_t(K - kBK) * 2;  // largest scalar (K step) offset
  int bad = 0;
  for (int p = 0; p < mok::geom::kLoads; ++p)
    for (int w = 0; w < mok::geom::kWaves; ++w)
      for (int l = 0; l < 64; ++l) {
        const int64_t oa = mok::geom::a_offset(p, w, l, rows, lda);
        const int64_t ob = mok::geom::b_offset(layout, p, w, l, n0, nb1, N, ldb);
        if (oa < 0 || oa + k_last + 16 > a_bytes || oa >= (int64_t(1) << 32)) ++bad;
        if (ob < 0 || ob + k_last + 16 > b_bytes || ob >= (int64_t(1) << 32)) ++bad;
      }
  if (bad) std::printf("%s: %d bad offsets (K=%d N=%d n0=%d rows=%d)\n", what, bad, K, N, n0, rows);
  return bad;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s D I\n", argv[0]);
    return 2;
  }
  const int D = std::atoi(argv[1]), I = std::atoi(argv[2]);
  int bad = 0;
  for (int rows = 1; rows <= kBM; ++rows) {
    for (int n0 = 0; n0 < I; n0 += kBN1)
      bad += check("gemm1", mok::geom::kPaired, D, D, D, I, n0, n0, rows);
    for (int n0 = 0; n0 < D; n0 += kBN2)
      bad += check("gemm2", mok::geom::kSplit, I, I, I, D, n0, n0 + 128, rows);
    // backward: dH (A = dY rows, B = W_down^T [I, D]), dX (A = [da|db] rows, B =
    // [W_gate|W_up]^T [D, 2I]), dW (A, B = expert panels of width TKP, K <= panel width)
    for (int n0 = 0; n0 < I; n0 += kBN2)
      bad += check("dh", mok::geom::kSplit, D, D, D, I, n0, n0 + 128, rows);
    for (int n0 = 0; n0 < D; n0 += kBN2)
      bad += check("dx", mok::geom::kSplit, 2 * I, 2 * I, 2 * I, D, n0, n0 + 128, rows);
    const int TKP = 4096;
    for (int K : {64, 1024, 4096})
      for (int n0 = 0; n0 < I; n0 += kBN2)
        bad += check("dw", mok::geom::kSplit, K, TKP, TKP, I, n0, n0 + 128, rows);
  }
  // paired layout: tile rows of block b cover intermediate columns n0 + 16 b .. +15 of
  // both matrices, each exactly once (unclamped case)
  for (int b = 0; b < 8; ++b)
    for (int m = 0; m < 2; ++m)
      for (int q = 0; q < 16; ++q) {
        int hits = 0;
        for (int p = 0; p < mok::geom::kLoads; ++p)
          for (int w = 0; w < mok::geom::kWaves; ++w)
            for (int l = 0; l < 64; l += 8)
              if (mok::geom::b_matrix(mok::geom::kPaired, p, w) == m &&
                  mok::geom::b_row(mok::geom::kPaired, p, w, l, 0, 0, 1 << 20) == b * 16 + q &&
                  (mok::geom::dma_row(p, w, l) >> 5) == b)
                ++hits;
        if (hits != 1) ++bad;
      }
  // every tile row is loaded exactly once (8 lanes per row, one per chunk)
  {
    int seen[256][8] = {};
    for (int p = 0; p < mok::geom::kLoads; ++p)
      for (int w = 0; w < mok::geom::kWaves; ++w)
        for (int l = 0; l < 64; ++l) seen[mok::geom::dma_row(p, w, l)][mok::geom::dma_chunk(w, l)]++;
    for (int r = 0; r < 256; ++r)
      for (int c = 0; c < 8; ++c)
        if (seen[r][c] != 1) ++bad;
  }
  std::printf("D=%d I=%d: %s\n", D, I, bad ? "VIOLATIONS" : "ok");
  return bad ? 1 : 0;
}
