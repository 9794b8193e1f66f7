// Backward of the MoE layer on one GPU's share (bf16 in, fp32 weight gradients).
//
// What is computed (Leiphone article on MoK, section 02: the backward reverses the two
// transfers, pulling dY by the schedule's table and pushing dX contributions back to
// their tokens; news brief, design decisions: the router-weight gradient is formed
// inside the SwiGLU backward), per routed row r of expert e (token t, slot j, gate g):
//   u = dY[t] W_down[e]                      dH GEMM, against W_down transposed
//   dG[t,j] = <u, h>                          in the dH epilogue (no second pass over o)
//   da, db  = SwiGLU backward of g u          in the dH epilogue
//   dx_r = da W_gate[e] + db W_up[e]          dX GEMM, against [W_gate | W_up] transposed
//   dX[t] = sum over local slots j (ascending) of dx_r          fixed order
//   dW_down[e] = sum_r (g dY[t])^T h,  dW_gate[e] = sum_r da^T x,  dW_up[e] = sum_r db^T x
// The dW contractions run over the expert's rows; both operands are read from per-expert
// transposed panels (rows of the expert as columns, zero padded to a multiple of 64) so
// that every MFMA operand is K-contiguous, and each dW tile has one owner and one K
// order: no atomics, bitwise reproducible.
//
// This file holds the path as separate kernels.  The gate/up pre-activations a, b come
// from the forward where it still holds them and are recomputed otherwise (replay of
// GEMM1), following the reverse ring traversal: after a fused forward the ring slots
// hold the last S minibatches (the dH epilogue reads their a, b there), and only
// minibatches whose slot was recycled, mb < n_mb - S, are replayed into a row buffer.  An unfused forward that saves for
// the backward writes a, b of every row, and nothing is replayed.
#include <algorithm>

#include "tile_ops.h"

namespace mok {

struct BwdParams {
  Ptrs P;
  BwdArgs a;
  int T, D, I, k, nl, mt_max, nDt, nIt, nNdh, n_mb_max, S;
  int64_t TKP;
  int64_t slot_bytes, slot_ab;
  int ab_saved;  // 1: the forward wrote a, b of every row (unfused); 0: ring only (fused)
  int per_mt;    // forward tiles per m-tile (GEMM1 + GEMM2 column tiles): tile_base unit
};

// a, b of the rows of m-tile e in minibatch mb: in the ring slot while the minibatch is
// still resident after a fused forward, else in the row buffer (replayed, or written by
// an unfused forward).
__device__ __forceinline__ const uint16_t* ab_rows(const BwdParams& p, const int4& e, int mb) {
  if (!p.ab_saved && mb >= int(p.P.hdr[kHdrNmb]) - p.S)
    return reinterpret_cast<const uint16_t*>(p.P.ring + (mb % p.S) * p.slot_bytes + p.slot_ab) +
           int64_t(e.x - p.P.mb_start[mb]) * 2 * p.I;
  return p.P.bab + int64_t(e.x) * 2 * p.I;
}

// ------------------------------------------------------------------------------------
// preparation
// ------------------------------------------------------------------------------------
// Panel column offsets: roff[e+1] = roff[e] + round_up(count[e], 64).
__global__ __launch_bounds__(64) void k_bwd_prep(BwdParams p) {
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    p.P.roff[0] = 0;
    for (int e = 0; e < p.nl; ++e) {
      acc += (p.P.counts[e] + 63) & ~63;
      p.P.roff[e + 1] = acc;
    }
  }
}


// Expert panels of X and of gate * dY: column roff[e] + q holds routed row offsets[e] + q
// of expert e (zero for q >= count[e]).  grid: (TKP / 64, D / 64).
__global__ __launch_bounds__(256) void k_bwd_panels(BwdParams p) {
  __shared__ uint16_t tx[64][72];
  __shared__ uint16_t tg[64][72];
  const int pc0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  if (pc0 >= p.P.roff[p.nl]) return;
  int e = 0;
  while (p.P.roff[e + 1] <= pc0) ++e;
  const int q0 = pc0 - p.P.roff[e];
  const int cnt = p.P.counts[e];
  const int rbase = p.P.offsets[e] + q0;
  const int t = threadIdx.x;
  // rows of the 64 x 64 block: panel column c <-> routed row rbase + c
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = it * 256 + t;
    const int c = idx >> 3, d8 = (idx & 7) * 8;
    v4u vx = v4u{0u, 0u, 0u, 0u}, vg = v4u{0u, 0u, 0u, 0u};
    if (q0 + c < cnt && d0 + d8 < p.D) {
      const int q = p.P.perm[rbase + c];
      const int64_t tok = q / p.k;
      vx = *reinterpret_cast<const v4u*>(p.a.x + tok * p.D + d0 + d8);
      const v4u vy = *reinterpret_cast<const v4u*>(p.a.dy + tok * p.D + d0 + d8);
      const float g = p.a.gates[q];
      const uint32_t w[4] = {vy.x, vy.y, vy.z, vy.w};
      uint32_t o[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        o[e2] = pack_bf16x2(g * bf16_to_f32(uint16_t(w[e2] & 0xFFFF)),
                            g * bf16_to_f32(uint16_t(w[e2] >> 16)));
      vg = v4u{o[0], o[1], o[2], o[3]};
    }
    *reinterpret_cast<v4u*>(&tx[c][d8]) = vx;
    *reinterpret_cast<v4u*>(&tg[c][d8]) = vg;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = it * 256 + t;
    const int d = idx >> 3, c8 = (idx & 7) * 8;
    if (d0 + d >= p.D) continue;
    uint32_t wx[4], wg[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      wx[e2] = uint32_t(tx[c8 + 2 * e2][d]) | (uint32_t(tx[c8 + 2 * e2 + 1][d]) << 16);
      wg[e2] = uint32_t(tg[c8 + 2 * e2][d]) | (uint32_t(tg[c8 + 2 * e2 + 1][d]) << 16);
    }
    const int64_t off = int64_t(d0 + d) * p.TKP + pc0 + c8;
    *reinterpret_cast<v4u*>(p.P.xt + off) = v4u{wx[0], wx[1], wx[2], wx[3]};
    *reinterpret_cast<v4u*>(p.P.gdyt + off) = v4u{wg[0], wg[1], wg[2], wg[3]};
  }
}

// ------------------------------------------------------------------------------------
// GEMM kernels (one m-tile of the schedule's table per workgroup row)
// ------------------------------------------------------------------------------------
// m-tile g (0 .. m-tiles - 1, in row order over all minibatches): its table entry and
// minibatch (binary search over the m-tile prefix, tile_base[mb] / per_mt).
__device__ __forceinline__ void mtile_at(const BwdParams& p, int g, int4& e, int& mb) {
  const int n_mb = int(p.P.hdr[kHdrNmb]);
  int lo = 0, hi = n_mb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.P.tile_base[mid] / p.per_mt <= g) lo = mid;
    else hi = mid - 1;
  }
  mb = lo;
  e = p.P.mt_tab[int64_t(lo) * p.mt_max + (g - p.P.tile_base[lo] / p.per_mt)];
}

// The row GEMMs of the backward run on a grid of one workgroup per CU that walks the
// (m-tile, column tile) pairs, row tiles slowest: the grid's size does not depend on
// the worst-case tile table, and no workgroup starts only to find its slot empty.  The
// K loop ends with a barrier and every epilogue that touches LDS ends with one, so the
// next tile's loads may start at once.

// Replay of GEMM1 for the m-tiles of minibatches whose a, b are no longer held.
__global__ __launch_bounds__(512) void k_bwd_gemm1(BwdParams p) {
  if (p.ab_saved) return;
  const int nN1 = (p.I + kBN1 - 1) / kBN1;
  const int n_mb = int(p.P.hdr[kHdrNmb]);
  // the m-tiles of minibatches [0, n_mb - S) come first in row order
  const int mb_end = n_mb - p.S;
  if (mb_end <= 0) return;
  const int nq = (p.P.tile_base[mb_end] / p.per_mt) * nN1;
  const int64_t wsz = int64_t(p.I) * p.D;
  for (int q = blockIdx.x; q < nq; q += gridDim.x) {
    int4 e;
    int mb;
    mtile_at(p, q / nN1, e, mb);
    const int nt = q % nN1;
    TileAcc acc;
    TileSrc src;
    tile_src_init_gather(src, geom::kPaired, p.a.x, p.D, p.P.perm + e.x, p.k, e.y,
                         p.a.wg + e.z * wsz, p.a.wu + e.z * wsz, p.D, nt * kBN1, nt * kBN1, p.I);
    tile_gemm<false>(src, p.D, acc);
    epi_swiglu<false>(acc, e.y, nt * kBN1, p.I, nullptr, p.I, p.P.bab + int64_t(e.x) * 2 * p.I);
  }
}

// dH GEMM: u = dY rows x W_down[e] (K = D over the rows of W_down, read K-major), fused
// SwiGLU backward and dG partials.
__global__ __launch_bounds__(512) void k_bwd_dh(BwdParams p) {
  const int nq = int(p.P.hdr[kHdrMtiles]) * p.nNdh;
  const int64_t wsz = int64_t(p.I) * p.D;
  for (int q = blockIdx.x; q < nq; q += gridDim.x) {
    int4 e;
    int mb;
    mtile_at(p, q / p.nNdh, e, mb);
    const int nt = q % p.nNdh;
    const int n0 = nt * kBN2;
    const uint16_t* wd = p.a.wd + e.z * wsz;
    KmOp a, b;
    km_init_kc_gather(a, p.a.dy, p.D, p.P.perm + e.x, p.k, e.y);
    km_init_weights(b, wd, wd, p.D, p.I, n0, p.I);
    TileAcc acc;
    tile_gemm_km<kKC, kKW>(a, b, p.D / kBK, acc);
    const int pc0 = p.P.roff[e.z] + (e.x - p.P.offsets[e.z]);
    epi_dh(acc, e.y, e.x, pc0, p.P.roff[e.z + 1], n0, p.I, p.TKP, ab_rows(p, e, mb), p.a.gates,
           p.P.perm, p.P.bdab, p.P.ht, p.P.dat, p.P.dbt, p.P.dgpart, nt, p.nNdh);
  }
}

// dX GEMM: dx rows = [da | db] x [W_gate; W_up][e] (K = 2I over the rows of W_gate, then
// W_up, read K-major), pushed to their pairs.
__global__ __launch_bounds__(512) void k_bwd_dx(BwdParams p) {
  const int nq = int(p.P.hdr[kHdrMtiles]) * p.nDt;
  const int64_t K = 2 * int64_t(p.I);
  const int64_t wsz = int64_t(p.I) * p.D;
  for (int q = blockIdx.x; q < nq; q += gridDim.x) {
    int4 e;
    int mb;
    mtile_at(p, q / p.nDt, e, mb);
    const int n0 = (q % p.nDt) * kBN2;
    KmOp a, b;
    km_init_kc(a, p.P.bdab + int64_t(e.x) * K, K, e.y);
    km_init_weights(b, p.a.wg + e.z * wsz, p.a.wu + e.z * wsz, p.I, p.D, n0, p.D);
    TileAcc acc;
    tile_gemm_km<kKC, kKW>(a, b, int(K / kBK), acc);
    epi_scatter<false>(acc, e.y, n0, p.D, p.P.perm + e.x, p.P.dxbuf);
  }
}

// dW GEMMs over the expert panels.  Per expert: dW_down tiles (D x I), then dW_gate and
// dW_up tiles (I x D); K = the expert's padded row count (zero rows give zero tiles).
__global__ __launch_bounds__(512) void k_bwd_dw(BwdParams p) {
  const int per = p.nDt * p.nIt;
  const int e = blockIdx.x / (3 * per);
  const int q = blockIdx.x % (3 * per);
  const int which = q / per, r = q % per;
  const int c0 = p.P.roff[e];
  const int K = p.P.roff[e + 1] - c0;
  const int64_t wsz = int64_t(p.I) * p.D;
  const uint16_t *A, *B;
  float* C;
  int M, N, mt, nt;
  if (which == 0) {  // dW_down[e] = gdY^T h : rows d, columns i
    M = p.D; N = p.I; mt = r / p.nIt; nt = r % p.nIt;
    A = p.P.gdyt; B = p.P.ht; C = p.a.dwd + e * wsz;
  } else {           // dW_gate / dW_up[e] = da^T x / db^T x : rows i, columns d
    M = p.I; N = p.D; mt = r / p.nDt; nt = r % p.nDt;
    A = which == 1 ? p.P.dat : p.P.dbt; B = p.P.xt; C = (which == 1 ? p.a.dwg : p.a.dwu) + e * wsz;
  }
  const int m0 = mt * kBM, n0 = nt * kBN2;
  const int rows = min(kBM, M - m0);
  TileSrc src;
  tile_src_init(src, geom::kSplit, A + int64_t(m0) * p.TKP + c0, p.TKP, rows, B + c0, B + c0,
                p.TKP, n0, n0 + 128, N);
  TileAcc acc;
  tile_gemm<false>(src, K, acc);
  epi_store_f32(acc, rows, n0, N, C + int64_t(m0) * N, N);
}

// ------------------------------------------------------------------------------------
// reductions back to token order
// ------------------------------------------------------------------------------------
// dG[t, j] = sum over dH n-tiles (ascending) of the partials of row pos[t, j]; 0 if none.
__global__ __launch_bounds__(256) void k_bwd_dg(BwdParams p) {
  const int64_t TK = int64_t(p.T) * p.k;
  for (int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x; q < TK; q += int64_t(gridDim.x) * 256) {
    const int r = p.P.pos[q];
    float s = 0.f;
    if (r >= 0)
      for (int nt = 0; nt < p.nNdh; ++nt) s += p.P.dgpart[int64_t(r) * p.nNdh + nt];
    p.a.dg[q] = s;
  }
}

// dX[t] = sum over local slots j (ascending) of dxbuf[t*k + j], fp32, rounded once.
__global__ __launch_bounds__(256) void k_bwd_dxsum(BwdParams p) {
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int lane = threadIdx.x & 63;
  for (int t = gw; t < p.T; t += nw) {
    const int64_t q0 = int64_t(t) * p.k;
    const uint64_t has = __ballot(lane < p.k && p.P.pos[q0 + (lane < p.k ? lane : 0)] >= 0);
    v4u* out = reinterpret_cast<v4u*>(p.a.dx + int64_t(t) * p.D);
    for (int c = lane; c < (p.D >> 3); c += 64) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
      uint64_t m = has;
      while (m) {
        const int j = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const v4u v = reinterpret_cast<const v4u*>(p.P.dxbuf + (q0 + j) * p.D)[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = __fadd_rn(acc[2 * e], bf16_to_f32(uint16_t(w[e] & 0xFFFF)));
          acc[2 * e + 1] = __fadd_rn(acc[2 * e + 1], bf16_to_f32(uint16_t(w[e] >> 16)));
        }
      }
      out[c] = v4u{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    }
  }
}

// ------------------------------------------------------------------------------------
// host
// ------------------------------------------------------------------------------------
mok_status_t launch_backward(const Layout& L, const Ptrs& P, const BwdArgs& a, hipStream_t st) {
  BwdParams p;
  p.P = P;
  p.a = a;
  p.T = int(L.T); p.D = int(L.D); p.I = int(L.I); p.k = int(L.k); p.nl = int(L.nl);
  p.mt_max = int(L.mt_max); p.n_mb_max = int(L.n_mb_max);
  p.nDt = int((L.D + kBN2 - 1) / kBN2);
  p.nIt = int((L.I + kBN2 - 1) / kBN2);
  p.nNdh = int(L.nNdh);
  p.TKP = int64_t(L.TKP);
  p.S = int(L.S);
  p.slot_bytes = int64_t(L.slot_bytes);
  p.slot_ab = int64_t(L.slot_ab);
  p.ab_saved = L.unfused ? 1 : 0;
  p.per_mt = int(L.nN1 + L.nN2);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return MOK_E_DEVICE;
  const dim3 tiles_grid = dim3(unsigned(cus));  // one 512-thread tile workgroup fits a CU
  hipLaunchKernelGGL(k_bwd_prep, dim3(1), dim3(64), 0, st, p);
  hipLaunchKernelGGL(k_bwd_panels, dim3(unsigned(L.TKP / 64), unsigned(L.D / 64)), dim3(256), 0, st,
                     p);
  hipLaunchKernelGGL(k_bwd_gemm1, tiles_grid, dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL(k_bwd_dh, tiles_grid, dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL(k_bwd_dx, tiles_grid, dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL(k_bwd_dw, dim3(unsigned(L.nl * 3 * p.nDt * p.nIt)), dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL(k_bwd_dg, dim3(unsigned(std::min<int64_t>((L.TK + 255) / 256, 65536))),
                     dim3(256), 0, st, p);
  hipLaunchKernelGGL(k_bwd_dxsum, dim3(unsigned(std::min<int64_t>((L.T + 3) / 4, 1 << 20))),
                     dim3(256), 0, st, p);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_E_LAUNCH;
}

}  // namespace mok
