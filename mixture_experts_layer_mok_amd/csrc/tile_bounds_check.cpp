// Host-side check that every direct-to-LDS offset the GEMM tile forms stays inside its
// operand, for given hidden (D) and intermediate (I) sizes, over every tile shape the
// kernels launch: GEMM1 (A = [rows, D], B0 = W_gate, B1 = W_up: [I, D], columns n0..n0+127
// of both), GEMM2 (A = [rows, I], B0 = B1 = W_down: [D, I], columns n0..n0+255), any
// row count 1..256, and that the paired layout covers each gate/up row exactly once.
// The MXFP8 tile (1-byte codes, 128-byte K steps, a last half step when K % 128 == 64,
// one scale dword per row and step) is checked the same way: every code load stays
// inside its own row's K bytes, every scale load inside its row of scales, and every
// valid offset below 2^31 (the range of its buffer resource; setting bit 31 makes a load
// out of range).  The backward's K-major operands are checked too: weight offsets over
// every K step, the column clamps of routed-row loads, and that each staged K row gets
// all of its chunks once, and so are the MXFP8 backward's two scaled tiles (dH over D,
// dX over 2I).  Built with the host compiler only; exits non-zero on a violation.
#include <cstdio>
#include <cstdlib>
#include <algorithm>
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

// K-major weight operand: a matrix of Kmat rows of N columns (ld = N); the tile reads
// columns n0 .. n0 + 255 (clamped below N) of K rows k0 + 0..63 for every step k0.
static int check_km_weights(const char* what, int Kmat, int N, int n0) {
  const int64_t bytes = int64_t(Kmat) * N * 2;
  int bad = 0;
  for (int k0 = 0; k0 < Kmat; k0 += kBK)
    for (int p = 0; p < mok::geom::kLoads; ++p)
      for (int w = 0; w < mok::geom::kWaves; ++w)
        for (int l = 0; l < 64; ++l) {
          const int c = mok::geom::km_col(w, l, n0, N);
          const int64_t off =
              (int64_t(mok::geom::km_row(p, w, l)) * N + c) * 2 + int64_t(k0) * N * 2;
          if (c < 0 || c + 8 > N || off < 0 || off + 16 > bytes || off >= (int64_t(1) << 32)) ++bad;
        }
  if (bad) std::printf("%s: %d bad offsets (Kmat=%d N=%d n0=%d)\n", what, bad, Kmat, N, n0);
  return bad;
}

// K-major routed rows: a lane reads 16 bytes at column col0 + km_col(n0, N) of a source
// row of ld elements; the columns must stay inside [col0, col0 + N) and the row.
static int check_km_rows(const char* what, int64_t ld, int col0, int N, int n0) {
  int bad = 0;
  for (int w = 0; w < mok::geom::kWaves; ++w)
    for (int l = 0; l < 64; ++l) {
      const int c = col0 + mok::geom::km_col(w, l, n0, N);
      if (c < col0 || c + 8 > col0 + N || c + 8 > ld) ++bad;
    }
  if (bad) std::printf("%s: %d bad columns (ld=%lld N=%d n0=%d)\n", what, bad, (long long)ld, N, n0);
  return bad;
}

static int check_mx(const char* what, int layout, int K, int64_t lda, int64_t as_ld, int rows,
                    int64_t ldb, int64_t bs_ld, int N, int n0, int nb1) {
  const int nk = (K + 127) / 128;
  const bool half_last = K % 128 != 0;
  int bad = 0;
  for (int ks = 0; ks < nk; ++ks) {
    const bool half = half_last && ks == nk - 1;
    for (int w = 0; w < mok::geom::kWaves; ++w)
      for (int l = 0; l < 64; ++l) {
        const int64_t adj = (half && !mok::geom::mx_chunk_in_half(w, l)) ? -64 : 0;
        for (int p = 0; p < mok::geom::kLoads; ++p) {
          const int ra = std::min(mok::geom::dma_row(p, w, l), rows - 1);
          const int64_t oa = mok::geom::a_offset(p, w, l, rows, lda / 2) + adj + 128 * ks;
          if (oa < ra * lda || oa + 16 > ra * lda + K || oa + 16 > (int64_t(1) << 31)) ++bad;
          const int rb = mok::geom::b_row(layout, p, w, l, n0, nb1, N);
          const int64_t ob = mok::geom::b_offset(layout, p, w, l, n0, nb1, N, ldb / 2) + adj +
                             128 * ks;
          if (rb < 0 || rb >= N || ob < rb * ldb || ob + 16 > rb * ldb + K ||
              ob + 16 > (int64_t(1) << 31))
            ++bad;
        }
        if (4 * ks + 4 > as_ld || 4 * ks + 4 > bs_ld || as_ld % 4 || bs_ld % 4) ++bad;
        const int64_t sa = mok::geom::mx_a_scale_offset(w, l, rows, as_ld) + 4 * ks;
        if (sa < 0 || sa + 4 > int64_t(rows) * as_ld) ++bad;
        const int64_t sb = mok::geom::mx_b_scale_offset(layout, w, l, n0, nb1, N, bs_ld) + 4 * ks;
        if (sb < 0 || sb + 4 > int64_t(N) * bs_ld) ++bad;
      }
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
    // backward: dH's A = dY rows (K = D), dX's A = [da|db] rows (K = 2I); their B
    // operands are K-major weights, and dW reads K-major routed rows (below)
    for (int n0 = 0; n0 < I; n0 += kBN2)
      bad += check("dh", mok::geom::kSplit, D, D, D, I, n0, n0 + 128, rows);
    for (int n0 = 0; n0 < D; n0 += kBN2)
      bad += check("dx", mok::geom::kSplit, 2 * I, 2 * I, 2 * I, D, n0, n0 + 128, rows);
    // MXFP8 forward: padded scale rows for X / H, the caller's K / 32 weight scales when
    // K % 128 == 0 and a padded repack otherwise
    {
      const int64_t xs_ld = (D + 127) / 128 * 4, hs_ld = (I + 127) / 128 * 4;
      const int64_t wgs_ld = D % 128 ? xs_ld : D / 32, wds_ld = I % 128 ? hs_ld : I / 32;
      for (int n0 = 0; n0 < I; n0 += kBN1)
        bad += check_mx("gemm1-mx", mok::geom::kPaired, D, D, xs_ld, rows, D, wgs_ld, I, n0, n0);
      for (int n0 = 0; n0 < D; n0 += kBN2)
        bad += check_mx("gemm2-mx", mok::geom::kSplit, I, I, hs_ld, rows, I, wds_ld, D, n0,
                        n0 + 128);
      // MXFP8 backward: dH (A = quantised dY rows [rows, D] with X-style padded scales,
      // B = W_down^T codes [I, D] with D / 32 or repacked scales) and dX (A = quantised
      // [da | db] rows [rows, 2I], B = [W_gate; W_up]^T codes [D, 2I], scales 2I / 32)
      const int64_t wdts_ld = D % 128 ? xs_ld : D / 32, ab_ld = 2 * I / 32;
      for (int n0 = 0; n0 < I; n0 += kBN2)
        bad += check_mx("dh-mx", mok::geom::kSplit, D, D, xs_ld, rows, D, wdts_ld, I, n0,
                        n0 + 128);
      for (int n0 = 0; n0 < D; n0 += kBN2)
        bad += check_mx("dx-mx", mok::geom::kSplit, 2 * I, 2 * I, ab_ld, rows, 2 * I, ab_ld, D,
                        n0, n0 + 128);
    }
  }
  // K-major weights: dH reads W_down [D rows, I columns], dX W_gate / W_up [I rows, D
  // columns] (K = 2I: the steps of each matrix stay inside it)
  for (int n0 = 0; n0 < I; n0 += kBN2) bad += check_km_weights("dh-wd", D, I, n0);
  for (int n0 = 0; n0 < D; n0 += kBN2) bad += check_km_weights("dx-wgu", I, D, n0);
  // dW: dY / X rows (D columns), g h rows (I), da / db halves of [da | db] rows (2I)
  for (int n0 = 0; n0 < D; n0 += kBN2) bad += check_km_rows("dw-x", D, 0, D, n0);
  for (int n0 = 0; n0 < I; n0 += kBN2) {
    bad += check_km_rows("dw-gh", I, 0, I, n0);
    bad += check_km_rows("dw-da", 2 * I, 0, I, n0);
    bad += check_km_rows("dw-db", 2 * I, I, I, n0);
  }
  // K-major stage: each stage row gets its 32 chunks once, logical chunks a permutation
  for (int kk = 0; kk < 64; ++kk) {
    unsigned seen = 0;
    int loads = 0;
    for (int p = 0; p < mok::geom::kLoads; ++p)
      for (int w = 0; w < mok::geom::kWaves; ++w)
        for (int l = 0; l < 64; ++l)
          if (mok::geom::km_row(p, w, l) == kk) {
            ++loads;
            seen |= 1u << mok::geom::km_chunk(w, l);
          }
    if (loads != 32 || seen != 0xFFFFFFFFu) ++bad;
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
