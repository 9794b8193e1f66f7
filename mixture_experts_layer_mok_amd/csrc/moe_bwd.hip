// Backward of the MoE layer on one GPU's share (bf16 in, fp32 weight gradients).
//
// What is computed (Leiphone article on MoK, section 02: the backward reverses the two
// transfers, pulling dY by the schedule's table and pushing dX contributions back to
// their tokens; news brief, design decisions: the router-weight gradient is formed
// inside the SwiGLU backward), per routed row r of expert e (token t, slot j, gate g):
//   u = dY[t] W_down[e]                      dH GEMM (K over the rows of W_down)
//   dG[t,j] = <u, h>                          in the dH epilogue (no second pass over o)
//   da, db  = SwiGLU backward of g u          in the dH epilogue
//   dx_r = da W_gate[e] + db W_up[e]          dX GEMM (K over the rows of W_gate, W_up)
//   dX[t] = sum over local slots j (ascending) of dx_r          fixed order
//   dW_down[e] = sum_r dY[t]^T (g h),  dW_gate[e] = sum_r da^T x,  dW_up[e] = sum_r db^T x
// The GEMMs whose contraction runs over rows of a stored matrix (the weights for dH and
// dX, the expert's routed rows for dW) read that operand K-major as stored, through
// gfx950's transposing LDS reads: nothing is transposed in memory.  Each dW tile has one
// owner and one K order (the expert's rows ascending): no atomics, bitwise reproducible.
//
// dH, dX, dW and the row sums back to token order run in one persistent launch (tickets);
// the per-row offsets and the GEMM1 replay are launches before it.  The gate/up
// pre-activations a, b come from the forward where it still holds
// them and are recomputed otherwise (replay of GEMM1), following the reverse ring
// traversal: after a fused forward the ring slots hold the last S minibatches (the dH
// epilogue reads their a, b there), and only minibatches whose slot was recycled,
// mb < n_mb - S, are replayed into a row buffer.  An unfused forward that saves for the
// backward writes a, b of every row, and nothing is replayed.
//
// MXFP8 (Leiphone article on MoK, section 03: the MXFP8 mode covers the backward too):
// the two GEMMs that produce data gradients run on the scaled MFMA tile, each operand
// quantised along that GEMM's K in blocks of 32 — dH: dY rows along D (gathered and
// quantised by k_bwd_dyq) times W_down^T along D; dX: [da | db] rows along I (quantised
// per m-tile inside the persistent launch, once its dH tiles are done) times
// [W_gate; W_up]^T along I.  The transposed weight codes are made before the layer
// (mok_quantize_mx_t), as the forward's are.  The weight-gradient GEMMs stay bf16 with
// fp32 accumulation, on the same bf16 rows as the bf16 backward.  The MXFP8 forward that
// saves keeps a, b of every row, so nothing is replayed.
#include <algorithm>

#include "tile_ops.h"

namespace mok {

struct BwdParams {
  Ptrs P;
  BwdArgs a;
  int T, D, I, k, nl, mt_max, nDt, nIt, nNdh, n_mb_max, S;
  int64_t slot_bytes, slot_ab;
  int ab_saved;  // 1: the forward wrote a, b of every row (unfused); 0: ring only (fused)
  int ring_2g;   // 1: ring offsets stay below 2^31 bytes
  int64_t slot_x;
  int per_mt;    // forward tiles per m-tile (GEMM1 + GEMM2 column tiles): tile_base unit
  uint64_t wait_ticks;  // limit of a bounded wait (100 MHz ticks)
  int perturb;          // MOK_FLAG_PERTURB
  int64_t trace_tickets; // MOK_FLAG_TRACE: ticket records before the workgroup records
  // MXFP8: scale row strides of the dY rows (xs_ld), of the [da | db] rows and the
  // [W_gate; W_up]^T rows (abq_ld = 2I / 32), and the W_down^T scales the tiles read
  // (the caller's, or repacked in the workspace) with their stride
  int64_t xs_ld, abq_ld, wdts_ld;
  const uint8_t* wdts;
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

// After a fused forward with every minibatch still in its ring slot, the slots hold the
// X rows of all routed rows, in routed order per minibatch.
__device__ __forceinline__ bool x_in_ring(const BwdParams& p) {
  return !p.ab_saved && p.ring_2g && int(p.P.hdr[kHdrNmb]) <= p.S;
}

// Byte offsets of each routed row's dY and X data, for the dW tiles' gathered loads (no
// division or search in their load loop): dY row perm[r] / k of dy; X row from the ring
// slot that still holds it when every minibatch is resident after a fused forward
// (contiguous rows per minibatch), else row perm[r] / k of x.
__global__ __launch_bounds__(256) void k_bwd_rows(BwdParams p) {
  const int R = int(p.P.hdr[kHdrR]);
  const int n_mb = int(p.P.hdr[kHdrNmb]);
  const bool x_ring = x_in_ring(p);
  // counters of the backward launch that follows on the same stream
  const int nc = p.n_mb_max * p.mt_max;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < nc; i += gridDim.x * 256) p.P.bsync[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    p.P.hdr[kHdrBwdTicket] = 0;
    p.P.hdr[kHdrBwdDhDone] = 0;
    p.P.hdr[kHdrBwdDxDone] = 0;
    p.P.hdr[kHdrAbort] = 0;
  }
  for (int r = blockIdx.x * 256 + threadIdx.x; r < R; r += gridDim.x * 256) {
    const uint32_t tb = uint32_t(p.P.perm[r] / p.k) * uint32_t(p.D) * 2u;
    p.P.dyb[r] = tb;
    if (x_ring) {
      int lo = 0, hi = n_mb - 1;  // minibatch of row r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.P.mb_start[mid] <= r) lo = mid;
        else hi = mid - 1;
      }
      p.P.xb[r] = uint32_t((lo % p.S) * p.slot_bytes + p.slot_x) +
                  uint32_t(r - p.P.mb_start[lo]) * uint32_t(p.D) * 2u;
    } else {
      p.P.xb[r] = tb;
    }
  }
}

// MXFP8: dY row perm[r] / k of every routed row r, quantised along D into row r of the
// dY code buffer (one wave per row).
__global__ __launch_bounds__(256) void k_bwd_dyq(BwdParams p) {
  const int nw = gridDim.x * 4;
  for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < p.T; t += nw)
    wave_quant_row<false>(p.P.dyq + int64_t(t) * p.D, p.P.dyqs + int64_t(t) * p.xs_ld,
                          p.a.dy + int64_t(t) * p.D, p.D);
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
    tile_gemm<false, true>(src, p.D, acc);
    epi_swiglu<false>(acc, e.y, nt * kBN1, p.I, nullptr, p.I, p.P.bab + int64_t(e.x) * 2 * p.I);
  }
}

// dH tile (m-tile g, column tile nt): u = dY rows x W_down[e] (K = D over the rows of
// W_down, read K-major), fused SwiGLU backward and dG partials.  da, db are stored at
// device scope: dX tiles on other XCDs read them in the same launch.
template <bool MX>
__device__ __forceinline__ uint32_t dh_tile(const BwdParams& p, int g, int nt) {
  const int64_t wsz = int64_t(p.I) * p.D;
  int4 e;
  int mb;
  mtile_at(p, g, e, mb);
  const int n0 = nt * kBN2;
  TileAcc acc;
  if (MX) {
    // A = the quantised dY rows of the m-tile's tokens (quantised once per token by the
    // previous launch), gathered; B = W_down^T codes of the expert: rows n0 .. n0 + 255
    // of [I, D], K = D
    const uint8_t* B = p.a.wdt + int64_t(e.z) * wsz;
    const uint8_t* Bs = p.wdts + int64_t(e.z) * p.I * p.wdts_ld;
    MxSrc src;
    mx_src_init_gather(src, geom::kSplit, p.P.dyq, p.P.dyqs, p.D, p.xs_ld, p.P.perm + e.x, p.k,
                       e.y, B, Bs, B, Bs, p.D, p.wdts_ld, n0, n0 + 128, p.I, p.D);
    mx_gemm<false>(src, p.D, acc);
  } else {
    const uint16_t* wd = p.a.wd + e.z * wsz;
    KmOp a, b;
    km_init_kc_gather(a, p.a.dy, p.D, p.P.perm + e.x, p.k, e.y);
    km_init_weights(b, wd, wd, p.D, p.I, n0, p.I);
    tile_gemm_km<kKC, kKW>(a, b, p.D / kBK, acc);
  }
  const uint32_t t_k = uint32_t(wall_clock64());
  epi_dh<kCpolDev>(acc, e.y, e.x, n0, p.I, ab_rows(p, e, mb), p.a.gates, p.P.perm, p.P.bdab,
                   p.P.gh, p.P.dgpart, nt, p.nNdh);
  return t_k;
}

// dX tile (m-tile g, column tile nt): dx rows = [da | db] x [W_gate; W_up][e] (K = 2I over
// the rows of W_gate, then W_up, read K-major), pushed to their pairs.  The da, db rows
// come from dH tiles of the same launch, so they are read at device scope, and the dx
// rows are stored at device scope for the row sums of the same launch.
template <bool MX>
__device__ __forceinline__ uint32_t dx_tile(const BwdParams& p, int g, int nt) {
  const int64_t K = 2 * int64_t(p.I);
  const int64_t wsz = int64_t(p.I) * p.D;
  int4 e;
  int mb;
  mtile_at(p, g, e, mb);
  const int n0 = nt * kBN2;
  TileAcc acc;
  if (MX) {
    // A = the m-tile's quantised [da | db] rows (written by this launch on other XCDs:
    // device-scope loads), B = [W_gate; W_up]^T codes of the expert: rows n0 .. n0 + 255
    // of [D, 2I], K = 2I
    const uint8_t* B = p.a.wgut + int64_t(e.z) * 2 * wsz;
    const uint8_t* Bs = p.a.wguts + int64_t(e.z) * p.D * p.abq_ld;
    MxSrc src;
    mx_src_init(src, geom::kSplit, p.P.dabq + int64_t(e.x) * K, p.P.dabqs + int64_t(e.x) * p.abq_ld,
                K, p.abq_ld, e.y, B, Bs, B, Bs, K, p.abq_ld, n0, n0 + 128, p.D, int(K));
    mx_gemm<true, true>(src, int(K), acc);
  } else {
    KmOp a, b;
    km_init_kc(a, p.P.bdab + int64_t(e.x) * K, K, e.y);
    km_init_weights(b, p.a.wg + e.z * wsz, p.a.wu + e.z * wsz, p.I, p.D, n0, p.D);
    tile_gemm_km<kKCD, kKW, true>(a, b, int(K / kBK), acc);
  }
  const uint32_t t_k = uint32_t(wall_clock64());
  epi_scatter<true, false>(acc, e.y, n0, p.D, p.P.perm + e.x, p.P.dxbuf, int64_t(p.T) * p.k);
  return t_k;
}

// MXFP8: the [da | db] rows of m-tile g quantised along I (blocks of 32; I % 32 == 0, so
// a block never mixes da and db), one wave per row.  The rows come from this launch's dH
// tiles and go to its dX tiles, on other XCDs: device-scope loads and stores.
__device__ __forceinline__ void quant_dab_rows(const BwdParams& p, int g) {
  int4 e;
  int mb;
  mtile_at(p, g, e, mb);
  const int64_t K = 2 * int64_t(p.I);
  for (int r = threadIdx.x >> 6; r < e.y; r += kThreads / 64) {
    const int64_t row = int64_t(e.x) + r;
    wave_quant_row<true, kCpolDev>(p.P.dabq + row * K, p.P.dabqs + row * p.abq_ld,
                                   p.P.bdab + row * K, int(K));
  }
}

// dW GEMMs, K over the expert's routed rows in ascending order, both operands read
// K-major as stored: per expert, dW_down tiles (D x I: A = dY rows gathered by perm,
// B = g h rows), then dW_gate and dW_up tiles (I x D: A = da / db rows, B = X rows, from
// the ring when it holds them all).  g h, da and db come from dH tiles of the same
// launch and are read at device scope.  Rows past the expert's last read zero; an expert
// without rows gets zero tiles.  One workgroup owns each tile: no atomics.
// TR: the tile is computed transposed (measured on MI355X: the MXFP8 backward, 12.05 ->
// 11.75 ms at the config-4 shape, from the kernel's register allocation; the bf16
// backward is 2% faster untransposed, whose stores write whole row segments).
template <int AK, int BK, bool TR>
__device__ __forceinline__ uint32_t dw_tile(KmOp& a, KmOp& b, int nk, int rows, int n0, int N,
                                            float* C) {
  TileAcc acc;
  tile_gemm_km<AK, BK, TR>(a, b, nk, acc);
  const uint32_t t_k = uint32_t(wall_clock64());
  epi_store_f32<TR>(acc, rows, n0, N, C, N);
  return t_k;
}

// dW tile q of nl * 3 * nDt * nIt: expert, then dW_down / dW_gate / dW_up, then tiles.
template <bool TR>
__device__ __forceinline__ uint32_t dw_tile_at(const BwdParams& p, int q) {
  const int per = p.nDt * p.nIt;
  const int e = q / (3 * per);
  const int which = (q % (3 * per)) / per, r = q % per;
  const int rbeg = p.P.offsets[e], rend = rbeg + p.P.counts[e];
  const int nk = (rend - rbeg + kBK - 1) / kBK;
  const int64_t wsz = int64_t(p.I) * p.D;
  KmOp a, b;
  if (which == 0) {  // dW_down[e][d][i] = sum_r dY[t_r][d] (g h)[r][i]
    const int m0 = (r / p.nIt) * kBM, n0 = (r % p.nIt) * kBN2;
    km_init_rows<kKG>(a, p.a.dy, p.D, 0, m0, p.D, p.P.dyb, rbeg, rend);
    km_init_rows<kKRD>(b, p.P.gh, p.I, 0, n0, p.I, nullptr, rbeg, rend);
    return dw_tile<kKG, kKRD, TR>(a, b, nk, min(kBM, p.D - m0), n0, p.I,
                              p.a.dwd + e * wsz + int64_t(m0) * p.I);
  } else {           // dW_gate / dW_up[e][i][d] = sum_r da / db[r][i] X[t_r][d]
    const int m0 = (r / p.nDt) * kBM, n0 = (r % p.nDt) * kBN2;
    km_init_rows<kKRD>(a, p.P.bdab, 2 * int64_t(p.I), which == 1 ? 0 : p.I, m0, p.I, nullptr,
                       rbeg, rend);
    km_init_rows<kKG>(b, x_in_ring(p) ? static_cast<const void*>(p.P.ring) : p.a.x, p.D, 0, n0,
                      p.D, p.P.xb, rbeg, rend);
    return dw_tile<kKRD, kKG, TR>(a, b, nk, min(kBM, p.I - m0), n0, p.D,
                              (which == 1 ? p.a.dwg : p.a.dwu) + e * wsz + int64_t(m0) * p.D);
  }
}

// Tokens [c * kSumTokens, +kSumTokens): dX[t] = sum over local slots j (ascending) of the
// dx row of pair t*k + j, fp32, rounded once (zero for a token without local slots), one
// wave per token; dG[t, j] = sum over dH column tiles (ascending) of the partials of row
// pos[t, j], 0 if none.  The dx rows and the partials come from tiles of the same launch:
// device-scope reads.
constexpr int kSumTokens = 32;
__device__ __forceinline__ void sum_chunk(const BwdParams& p, int c) {
  const int t0 = c * kSumTokens, t1 = min(t0 + kSumTokens, p.T);
  for (int t = t0 + (threadIdx.x >> 6); t < t1; t += kThreads / 64)
    wave_pair_sum<kCpolDev, 2>(p.a.dx + int64_t(t) * p.D, p.P.dxbuf, int64_t(t) * p.k, p.D,
                               p.P.pos, nullptr, p.k);
  for (int64_t q = int64_t(t0) * p.k + threadIdx.x; q < int64_t(t1) * p.k; q += kThreads) {
    const int r = p.P.pos[q];
    float s = 0.f;
    if (r >= 0)
      for (int nt = 0; nt < p.nNdh; ++nt)
        s += __uint_as_float(ld_relaxed(reinterpret_cast<const uint32_t*>(
            p.P.dgpart + int64_t(r) * p.nNdh + nt)));
    p.a.dg[q] = s;
  }
}

// The backward GEMMs and row sums in one persistent launch (one workgroup per CU).
// Workgroups take tickets in this order:
//   1. every dH tile, m-tiles slowest and in reverse row order: the last minibatch first,
//      as the ring is walked backwards (its slots hold the most recent minibatches);
//   1b. MXFP8 only: one quantisation of [da | db] per m-tile, in the same order; one of
//      m-tile g waits until the dH tiles of g have signalled, then signals g once more;
//   2. every dX tile, m-tiles in the same order; one of m-tile g waits until the dH tiles
//      (and in MXFP8 the quantisation) of g have signalled;
//   3. the first two rounds of dW tiles; a workgroup's first dW tile waits until every
//      dH tile has signalled;
//   4. the row-sum chunks; a workgroup's first chunk waits until every dX tile has
//      signalled (they were all taken before, and are done by now in the normal case);
//   5. the remaining dW tiles.
// Every wait is on work with smaller tickets, so each ends.  One ticket stream removes the
// idle tails between the steps, and the dW epilogues (256 KB of fp32 stores a tile) no
// longer start on every CU at once: the CUs reach their dW tiles at different times.
// Waits are bounded and every loop exits once the abort word is set.
template <bool MX>
__global__ __launch_bounds__(512) void k_bwd_main(BwdParams p) {
  uint32_t* hdr = p.P.hdr;
  uint32_t* hd = p.P.bsync;
  const uint32_t mt = hdr[kHdrMtiles];
  const uint32_t nh = mt * uint32_t(p.nNdh);
  const uint32_t nq = MX ? mt : 0u;  // MXFP8: one [da | db] quantisation per m-tile
  const uint32_t nx = mt * uint32_t(p.nDt);
  const uint32_t nw = uint32_t(p.nl) * 3u * uint32_t(p.nDt) * uint32_t(p.nIt);
  const uint32_t ns = uint32_t((p.T + kSumTokens - 1) / kSumTokens);
  const uint32_t w1 = min(nw, 2u * gridDim.x);
  const uint32_t b_q = nh, b_x = b_q + nq, b_w1 = b_x + nx, b_s = b_w1 + w1, b_w2 = b_s + ns;
  // a dX tile of m-tile g waits for its dH tiles, and in MXFP8 for its quantisation too
  const uint32_t dx_need = uint32_t(p.nNdh) + (MX ? 1u : 0u);
  const uint32_t total = b_w2 + (nw - w1);
  bool dh_all = false, dx_all = false;
  const bool trace = p.P.trace != nullptr;
  const uint32_t t_start = trace ? uint32_t(wall_clock64()) : 0u;
  uint32_t n_taken = 0;
  __shared__ uint32_t s_tk;
  while (true) {
    if (threadIdx.x == 0) s_tk = fetch_add_relaxed(hdr + kHdrBwdTicket, 1u);
    __syncthreads();
    const uint32_t tk = __builtin_amdgcn_readfirstlane(s_tk);  // wave-uniform
    __syncthreads();
    if (tk >= total || aborted(hdr)) break;
    ++n_taken;
    const uint32_t t_tk = trace ? uint32_t(wall_clock64()) : 0u;
    uint32_t t_ready = t_tk, t_k = 0u, kind;
    if (tk < b_q) {
      kind = 0;
      const int g = int(mt) - 1 - int(tk) / p.nNdh;
      t_k = dh_tile<MX>(p, g, int(tk) % p.nNdh);
      perturb_pause(p.perturb, tk);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0) {
        fetch_add_relaxed(hd + g, 1u);
        fetch_add_relaxed(hdr + kHdrBwdDhDone, 1u);
      }
    } else if (tk < b_x) {
      kind = 4;
      const int g = int(mt) - 1 - int(tk - b_q);
      if (!wg_wait_geq(hd + g, uint32_t(p.nNdh), hdr, p.wait_ticks)) break;
      t_ready = trace ? uint32_t(wall_clock64()) : 0u;
      quant_dab_rows(p, g);
      t_k = trace ? uint32_t(wall_clock64()) : 0u;
      perturb_pause(p.perturb, tk);
      wg_signal_add(hd + g, 1u);
    } else if (tk < b_w1) {
      kind = 1;
      const int q = int(tk - b_x);
      const int g = int(mt) - 1 - q / p.nDt;
      if (!wg_wait_geq(hd + g, dx_need, hdr, p.wait_ticks)) break;
      t_ready = trace ? uint32_t(wall_clock64()) : 0u;
      t_k = dx_tile<MX>(p, g, q % p.nDt);
      perturb_pause(p.perturb, tk);
      wg_signal_add(hdr + kHdrBwdDxDone, 1u);
    } else if (tk >= b_s && tk < b_w2) {
      kind = 3;
      if (!dx_all) {
        if (!wg_wait_geq(hdr + kHdrBwdDxDone, nx, hdr, p.wait_ticks)) break;
        dx_all = true;
      }
      t_ready = trace ? uint32_t(wall_clock64()) : 0u;
      perturb_pause(p.perturb, tk);
      sum_chunk(p, int(tk - b_s));
      t_k = trace ? uint32_t(wall_clock64()) : 0u;
    } else {
      kind = 2;
      if (!dh_all) {
        if (!wg_wait_geq(hdr + kHdrBwdDhDone, nh, hdr, p.wait_ticks)) break;
        dh_all = true;
      }
      t_ready = trace ? uint32_t(wall_clock64()) : 0u;
      t_k = dw_tile_at<MX>(p, int(tk < b_s ? tk - b_w1 : w1 + (tk - b_w2)));
    }
    if (trace && threadIdx.x == 0) {
      uint32_t* rec = p.P.trace + int64_t(tk) * 8;
      rec[0] = blockIdx.x; rec[1] = kind; rec[2] = t_tk; rec[3] = t_ready; rec[4] = t_k;
      rec[5] = uint32_t(wall_clock64()); rec[6] = 0; rec[7] = 0;
    }
  }
  if (trace && threadIdx.x == 0 && blockIdx.x < MOK_TRACE_MAX_WORKGROUPS) {
    uint32_t* rec = p.P.trace + p.trace_tickets * 8 + int64_t(blockIdx.x) * 8;
    rec[0] = t_start; rec[1] = t_start; rec[2] = uint32_t(wall_clock64()); rec[3] = rec[2];
    rec[4] = 0; rec[5] = n_taken; rec[6] = 0; rec[7] = 0;
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
  p.S = int(L.S);
  p.slot_bytes = int64_t(L.slot_bytes);
  p.slot_ab = int64_t(L.slot_ab);
  // an unfused forward and a MXFP8 forward that save write a, b of every row
  p.ab_saved = (L.unfused || L.mx) ? 1 : 0;
  p.slot_x = int64_t(L.slot_x);
  p.ring_2g = int64_t(L.S) * int64_t(L.slot_bytes) < (int64_t(1) << 31) ? 1 : 0;
  p.per_mt = int(L.nN1 + L.nN2);
  p.wait_ticks = L.short_waits ? kShortWaitTicks : kWaitTicks;
  p.perturb = L.perturb ? 1 : 0;
  p.trace_tickets = int64_t(L.trace_tickets);
  p.xs_ld = L.xs_ld;
  p.abq_ld = L.abq_ld;
  p.wdts_ld = L.repack_wdt ? L.xs_ld : L.D / 32;
  p.wdts = L.repack_wdt ? P.wdts : a.wdts;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return MOK_E_DEVICE;
  const dim3 tiles_grid = dim3(unsigned(cus));  // one 512-thread tile workgroup fits a CU
  hipLaunchKernelGGL(k_bwd_rows, dim3(unsigned(std::min<int64_t>((L.TK + 255) / 256, 4096))),
                     dim3(256), 0, st, p);
  if (L.mx) {
    if (L.repack_wdt) launch_mx_repack(a.wdts, L.nl * L.I, int(L.D / 32), P.wdts, int(L.xs_ld), st);
    hipLaunchKernelGGL(k_bwd_dyq, dim3(unsigned(std::min<int64_t>((L.T + 3) / 4, 65536))),
                       dim3(256), 0, st, p);
    hipLaunchKernelGGL(k_bwd_main<true>, tiles_grid, dim3(kThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL(k_bwd_gemm1, tiles_grid, dim3(kThreads), 0, st, p);
    hipLaunchKernelGGL(k_bwd_main<false>, tiles_grid, dim3(kThreads), 0, st, p);
  }
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_E_LAUNCH;
}

}  // namespace mok
