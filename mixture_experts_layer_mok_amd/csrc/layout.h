// Workspace layout of one layer call, computed identically on the host (sizes,
// pointer arithmetic) and described to the kernels through MokParams.
//
// Everything the layer keeps between its kernels lives in one caller-owned workspace:
//   header words, schedule tables, device counters, the per-pair result buffer,
//   the ring of S minibatch slots and (optional) full-size buffers for the unfused
//   path and the backward pass.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/mok.h"

namespace mok {

// GEMM tiling shared by every grouped-GEMM kernel.
constexpr int kBM = 256;       // rows per m-tile (m-tiles start at expert offsets)
constexpr int kBN1 = 128;      // intermediate columns per GEMM1 tile (gate and up each)
constexpr int kBN2 = 256;      // hidden columns per GEMM2 tile
constexpr int kBK = 64;        // K step (bf16 elements, 128 bytes per row)
constexpr int kThreads = 512;  // threads per GEMM workgroup (8 waves of 64)

// Schedule kernels.
constexpr int kSchedChunk = 4096;  // pairs per counting block (4 waves x 1024)
constexpr int kSchedSub = 1024;    // pairs per wave sub-chunk
constexpr int kMaxLocalExperts = 1024;

// Header words (int32) at the start of the workspace.
enum HdrWord : int {
  kHdrStatus = 0,      // sticky MOK_DEV_* bits
  kHdrR = 1,           // routed local rows
  kHdrNmb = 2,         // minibatches
  kHdrMtiles = 3,      // m-tiles over all minibatches
  kHdrFwdTicket = 4,   // fused forward: next tile ticket
  kHdrAbort = 5,       // set when a bounded wait expires; every loop exits
  kHdrFwdTiles = 6,    // fused forward: total tiles
  kHdrDrainTicket = 7, // fused forward: next drain work chunk
  kHdrBwdTicket = 8,   // backward kernel: next ticket
  kHdrBwdDhDone = 9,   // backward kernel: dH tiles done
  kHdrBwdDxDone = 10,  // backward kernel: dX tiles done
  kHdrArrive = 11,     // fused forward: workgroups started (each takes the next number)
  kHdrFillTicket = 12, // fused forward: next chunk of minibatch 0's rows (the fill)
  kHdrWords = 64
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
  // shape
  int64_t T, D, I, E, k, e0, nl, M, S, TK;
  int64_t NB;        // counting blocks of the schedule
  int64_t NS;        // wave sub-chunks (4 per block)
  int64_t n_mb_max;  // ceil(T*k / M)
  int64_t mt_max;    // m-tiles per minibatch, upper bound
  int64_t nN1, nN2;  // n-tiles of GEMM1 (over I) and GEMM2 (over D)
  bool mx, save, unfused, short_waits, perturb, trace, overlap_next;
  // MXFP8: bytes per scale row of the layer's own X and H buffers (one dword per 128-wide
  // K step), and of the weight scales the tiles read (the caller's K / 32 when K % 128
  // == 0, else a repacked copy in the workspace with the padded stride)
  int64_t xs_ld, hs_ld, wgs_ld, wds_ld;
  bool repack_wg, repack_wd;
  // byte offsets into the workspace
  size_t off_hdr, off_counts, off_offsets, off_blk, off_perm, off_pos, off_mt_tab, off_mt_cnt,
      off_tile_base, off_mb_start, off_sync, sync_bytes, sync_bwd, off_obuf, off_ring, slot_bytes;
  int64_t slot_rows;  // rows one slot holds: a minibatch's tiles may run past its window
  size_t slot_x, slot_xs, slot_h, slot_hs, slot_ab;  // offsets inside one slot
  size_t off_full_x, off_full_xs, off_full_h, off_full_hs;
  size_t off_wsg, off_wsu, off_wsd;  // repacked weight scales (MXFP8, when needed)
  // backward (present with MOK_FLAG_SAVE_FOR_BWD)
  int64_t nNdh;     // n-tiles of the dH GEMM (over I)
  size_t off_bab, off_bdab, off_dxbuf, off_dgpart, off_gh, off_dyb, off_xb;
  // MXFP8 backward (MXFP8 forward that saves): dY quantised along D once per token
  // (codes [T, D], scales [T, xs_ld]; the dH tiles gather them by token), [da | db] rows
  // quantised along I per half
  // (codes [T*k, 2I], scales [T*k, 2I / 32]), and W_down^T's scales repacked to the
  // tile's stride when D % 128 != 0
  size_t off_dyq, off_dyqs, off_dabq, off_dabqs, off_wdts;
  int64_t abq_ld;
  bool repack_wdt;
  size_t off_trace, trace_words, trace_tickets;  // MOK_FLAG_TRACE: ticket records, then
                                                // workgroup records
  // workgroups of the unfused gather, GEMM1, GEMM2 and combine launches
  int64_t unf_grid[4];
  size_t total;
};

// Fills `L` from the descriptor; returns MOK_OK or the first violated check.
inline mok_status_t make_layout(const mok_desc_t* d, Layout* L) {
  if (!d || !L) return MOK_E_NULL;
  const int64_t T = d->num_tokens, D = d->hidden, I = d->intermediate, E = d->num_experts;
  const int64_t k = d->top_k, e0 = d->expert_begin, nl = d->num_local_experts;
  const int64_t M = d->minibatch_rows, S = d->ring_slots;
  if (T < 1 || T > (1 << 24)) return MOK_E_SHAPE;
  if (D < 64 || D % 64 != 0 || D > 65536) return MOK_E_SHAPE;
  if (I < 64 || I % 64 != 0 || I > 65536) return MOK_E_SHAPE;
  if (E < 1 || k < 1 || k > 64 || k > E) return MOK_E_SHAPE;
  if (nl < 1 || nl > kMaxLocalExperts || e0 < 0 || e0 + nl > E) return MOK_E_SHAPE;
  if (M < 1 || M > (1 << 20) || S < 1 || S > 64) return MOK_E_SHAPE;
  if (T * k > (int64_t(1) << 24)) return MOK_E_SHAPE;
  if (D * I >= (int64_t(1) << 31)) return MOK_E_SHAPE;  // a weight matrix in 32-bit offsets
  if (d->comm_cus < 1) return MOK_E_SHAPE;
  if (d->precision != MOK_PREC_BF16 && d->precision != MOK_PREC_MXFP8) return MOK_E_UNSUPPORTED;
  if (d->flags & ~(MOK_FLAG_SAVE_FOR_BWD | MOK_FLAG_UNFUSED | MOK_FLAG_SHORT_WAITS |
                   MOK_FLAG_PERTURB | MOK_FLAG_TRACE | MOK_FLAG_OVERLAP_NEXT))
    return MOK_E_UNSUPPORTED;
  L->T = T; L->D = D; L->I = I; L->E = E; L->k = k; L->e0 = e0; L->nl = nl; L->M = M; L->S = S;
  L->TK = T * k;
  L->mx = d->precision == MOK_PREC_MXFP8;
  L->save = (d->flags & MOK_FLAG_SAVE_FOR_BWD) != 0;
  L->unfused = (d->flags & MOK_FLAG_UNFUSED) != 0;
  L->short_waits = (d->flags & MOK_FLAG_SHORT_WAITS) != 0;
  L->perturb = (d->flags & MOK_FLAG_PERTURB) != 0;
  L->trace = (d->flags & MOK_FLAG_TRACE) != 0;
  L->overlap_next = (d->flags & MOK_FLAG_OVERLAP_NEXT) != 0;
  L->NB = (L->TK + kSchedChunk - 1) / kSchedChunk;
  L->NS = L->NB * (kSchedChunk / kSchedSub);
  L->n_mb_max = (L->TK + M - 1) / M;
  // m-tiles start at expert offsets and every kBM rows after; a minibatch holds the
  // m-tiles whose first row lies in its window [i*M, (i+1)*M): at most M/kBM + 1 per
  // expert segment it touches.
  L->mt_max = (M + kBM - 1) / kBM + nl + 1;
  if (L->mt_max > L->TK / kBM + 1 + nl) L->mt_max = L->TK / kBM + 1 + nl;
  L->slot_rows = M + kBM;
  L->xs_ld = (D + 127) / 128 * 4;
  L->hs_ld = (I + 127) / 128 * 4;
  L->repack_wg = L->mx && D % 128 != 0;
  L->repack_wd = L->mx && I % 128 != 0;
  L->wgs_ld = L->repack_wg ? L->xs_ld : D / 32;
  L->wds_ld = L->repack_wd ? L->hs_ld : I / 32;
  L->nN1 = (I + kBN1 - 1) / kBN1;
  L->nN2 = (D + kBN2 - 1) / kBN2;

  const size_t A = 256;
  size_t o = 0;
  L->off_hdr = o; o = align_up(o + kHdrWords * 4, A);
  L->off_counts = o; o = align_up(o + nl * 4, A);
  L->off_offsets = o; o = align_up(o + (nl + 1) * 4, A);
  L->off_blk = o; o = align_up(o + L->NS * (nl + 1) * 4, A);  // per sub-chunk counts + bad
  L->off_perm = o; o = align_up(o + L->TK * 4, A);
  L->off_pos = o; o = align_up(o + L->TK * 4, A);
  L->off_mt_tab = o; o = align_up(o + L->n_mb_max * L->mt_max * 16, A);
  L->off_mt_cnt = o; o = align_up(o + L->n_mb_max * 4, A);
  L->off_tile_base = o; o = align_up(o + (L->n_mb_max + 1) * 4, A);
  L->off_mb_start = o; o = align_up(o + (L->n_mb_max + 1) * 4, A);
  // forward counters: ready[n_mb], done[n_mb], hdone[n_mb * mt_max];
  // backward counters (from sync_bwd): dH tiles done per m-tile [n_mb * mt_max]
  L->sync_bwd = align_up((2 * L->n_mb_max + L->n_mb_max * L->mt_max) * 4, A);
  L->sync_bytes = L->sync_bwd + align_up(L->n_mb_max * L->mt_max * 4, A);
  L->off_sync = o; o = align_up(o + L->sync_bytes, A);
  L->off_obuf = o; o = align_up(o + size_t(L->TK) * D * 2, A);
  // one ring slot
  size_t so = 0;
  const size_t SR = size_t(L->slot_rows);
  L->slot_x = so; so = align_up(so + SR * D * (L->mx ? 1 : 2), A);
  L->slot_xs = so; so = align_up(so + (L->mx ? SR * L->xs_ld : 0), A);
  L->slot_h = so; so = align_up(so + SR * I * (L->mx ? 1 : 2), A);
  L->slot_hs = so; so = align_up(so + (L->mx ? SR * L->hs_ld : 0), A);
  L->slot_ab = so; so = align_up(so + (L->save && !L->mx ? SR * 2 * I * 2 : 0), A);
  L->slot_bytes = so;
  L->off_ring = o; o = align_up(o + L->slot_bytes * S, A);
  // full-size buffers for the unfused path
  L->off_full_x = L->off_full_xs = L->off_full_h = L->off_full_hs = 0;
  if (L->unfused) {
    L->off_full_x = o; o = align_up(o + size_t(L->TK) * D * (L->mx ? 1 : 2), A);
    L->off_full_xs = o; o = align_up(o + (L->mx ? size_t(L->TK) * L->xs_ld : 0), A);
    L->off_full_h = o; o = align_up(o + size_t(L->TK) * I * (L->mx ? 1 : 2), A);
    L->off_full_hs = o; o = align_up(o + (L->mx ? size_t(L->TK) * L->hs_ld : 0), A);
  }
  L->off_wsg = L->off_wsu = L->off_wsd = 0;
  if (L->repack_wg) {
    L->off_wsg = o; o = align_up(o + size_t(nl) * I * L->wgs_ld, A);
    L->off_wsu = o; o = align_up(o + size_t(nl) * I * L->wgs_ld, A);
  }
  if (L->repack_wd) {
    L->off_wsd = o; o = align_up(o + size_t(nl) * D * L->wds_ld, A);
  }
  // backward regions (present when the forward saves for backward): row buffers indexed
  // by routed row (at most T*k rows).
  L->nNdh = (I + kBN2 - 1) / kBN2;
  L->off_bab = L->off_bdab = L->off_dxbuf = L->off_dgpart = L->off_gh = L->off_dyb = L->off_xb = 0;
  if (L->save) {
    // the backward GEMMs read weights with 32-bit offsets, and X, dY, [da | db] and g h
    // rows as K-major routed rows, whose offsets stay below 2^31 bytes (bit 31 marks a
    // row past the expert's end)
    if (2 * I * D >= (int64_t(1) << 31) || 2 * T * D >= (int64_t(1) << 31) ||
        L->TK * 4 * I >= (int64_t(1) << 31))
      return MOK_E_SHAPE;
    const size_t TK = size_t(L->TK);
    L->off_bab = o; o = align_up(o + TK * 2 * I * 2, A);
    L->off_bdab = o; o = align_up(o + TK * 2 * I * 2, A);
    L->off_dxbuf = o; o = align_up(o + TK * D * 2, A);
    L->off_dgpart = o; o = align_up(o + TK * L->nNdh * 4, A);
    L->off_gh = o; o = align_up(o + TK * I * 2, A);
    L->off_dyb = o; o = align_up(o + TK * 4, A);
    L->off_xb = o; o = align_up(o + TK * 4, A);
  }
  L->off_dyq = L->off_dyqs = L->off_dabq = L->off_dabqs = L->off_wdts = 0;
  L->abq_ld = 2 * I / 32;  // I % 64 == 0: 2I is a whole number of 128-wide steps
  L->repack_wdt = L->mx && L->save && D % 128 != 0;
  if (L->mx && L->save) {
    const size_t TK = size_t(L->TK);
    L->off_dyq = o; o = align_up(o + size_t(L->T) * D, A);
    L->off_dyqs = o; o = align_up(o + size_t(L->T) * L->xs_ld, A);
    L->off_dabq = o; o = align_up(o + TK * 2 * I, A);
    L->off_dabqs = o; o = align_up(o + TK * L->abq_ld, A);
    if (L->repack_wdt) { L->off_wdts = o; o = align_up(o + size_t(nl) * I * L->xs_ld, A); }
  }
  L->unf_grid[0] = std::min<int64_t>((L->TK + 3) / 4, 1 << 20);
  L->unf_grid[1] = L->n_mb_max * L->mt_max * L->nN1;
  L->unf_grid[2] = L->n_mb_max * L->mt_max * L->nN2;
  L->unf_grid[3] = std::min<int64_t>((T + 3) / 4, 1 << 20);
  L->off_trace = L->trace_words = L->trace_tickets = 0;
  if (L->trace) {
    // records for every forward tile ticket, or every backward ticket (dH, dX, dW tiles
    // and row-sum chunks of 32 tokens), whichever is more
    const size_t nDt = size_t((D + kBN2 - 1) / kBN2), nIt = size_t((I + kBN2 - 1) / kBN2);
    const size_t fwd = size_t(L->n_mb_max) * L->mt_max * (L->nN1 + L->nN2);
    const size_t bwd = size_t(L->n_mb_max) * L->mt_max * (nIt + nDt + (L->mx ? 1 : 0)) +
                       size_t(nl) * 3 * nDt * nIt + size_t((T + 31) / 32);
    L->trace_tickets = fwd > bwd ? fwd : bwd;
    L->trace_words = L->trace_tickets * 8 + size_t(MOK_TRACE_MAX_WORKGROUPS) * 8;
    if (L->unfused) {
      // the unfused forward's launches: 8 header words (their workgroup counts), then per
      // launch and workgroup two 64-bit timestamps
      size_t w = 8;
      for (int ph = 0; ph < 4; ++ph) w += size_t(L->unf_grid[ph]) * 4;
      if (w > L->trace_words) L->trace_words = w;
    }
    L->off_trace = o; o = align_up(o + L->trace_words * 4, A);
  }
  L->total = o;
  return MOK_OK;
}

}  // namespace mok
