// Forward of the MoE layer on one GPU's share, bf16 or MXFP8.
//
// Steps (Leiphone article on MoK, sections 02-03; news brief, design decisions):
//   dispatch  — pull: row r of minibatch mb is copied from the token pool,
//               X[perm[r] / k], into ring slot mb % S (the owner lays rows out itself,
//               already grouped by expert); in MXFP8 mode the row is quantised on the
//               way (e4m3 codes, one e8m0 scale per 32 values along D);
//   GEMM1     — per expert segment: a = X W_gate^T, b = X W_up^T sharing the A tile,
//               SwiGLU h = silu(a) * b in the epilogue, H written to the slot (MXFP8:
//               quantised along I in the same epilogue);
//   GEMM2     — o = H W_down^T, pushed straight to its pair's row of the result buffer
//               (the destination of every result is known from the schedule);
//   combine   — the final weighted sum: y[t] = sum_j gate[t,j] * o[t*k+j] over local
//               slots in ascending j, fp32 (multiply, then add), rounded once to bf16.
//
// Fused form (one persistent kernel, one workgroup per CU): workgroups number
// themselves in the order they start (an atomic counter); the first comm_cus move data
// (dispatch + combine), the rest run MFMA tiles.  Handoff data (slot rows, H, the
// result rows) is written and read at device scope (each MI355X XCD has its own L2),
// and the counters are relaxed device-scope atomics bumped after a workgroup's stores
// have completed:
//   ready[mb]  comm workgroups that finished gathering their share of mb;
//   hdone[mb][i]  GEMM1 tiles finished for m-tile i of mb (GEMM2 of that m-tile waits);
//   done[mb]   GEMM2 tiles finished for mb — frees slot mb % S and allows combining
//              the tokens whose last local row lies in mb.
// Compute workgroups take tiles from an atomic ticket.  Tickets run in blocks
// j = 0, 1, ...: block j holds the GEMM1 tiles of minibatch j followed by the GEMM2
// tiles of minibatch j - L, with a lookahead L = 1 when the ring has two slots or more
// (L = 0 otherwise), so a GEMM2 tile's H was normally finished a whole block earlier.
// Every wait is on work with a smaller ticket (GEMM2 of mb on GEMM1 of mb) or on a
// comm step that only depends on such work (the gather of mb on GEMM2 of mb - S, in
// block mb - S + L < mb): no cycle.  Every role, ticket and chunk goes to a workgroup
// that is already running, so no wait depends on a workgroup that has not started: the
// kernel needs no co-residency guarantee (no cooperative launch), only that more than
// comm_cus of its workgroups can run at once.  A token is combined by the comm workgroup that
// owns its highest local row, right after that row's minibatch is done, so most of the
// combine overlaps later minibatches' GEMMs.
#include <algorithm>

#include "tile_ops.h"

namespace mok {

struct FwdParams {
  Ptrs P;
  FwdArgs a;
  int T, D, I, k, M, S, mt_max, nN1, nN2, n_mb_max, save;
  uint64_t wait_ticks;  // limit of a bounded wait (100 MHz ticks)
  int perturb;          // MOK_FLAG_PERTURB
  int overlap_next;     // MOK_FLAG_OVERLAP_NEXT: compute workgroups skip the drain
  int64_t trace_tiles;  // MOK_FLAG_TRACE: tile records before the workgroup records
  int64_t ph_rec[4];    // MOK_FLAG_TRACE, unfused: first 64-bit word of each launch's records
  int64_t slot_bytes, slot_x, slot_xs, slot_h, slot_hs, slot_ab;
  // MXFP8: scale row strides of X / H rows and of the weight scales the tiles read, and
  // those weight scales (the caller's, or repacked copies in the workspace)
  int64_t xs_ld, hs_ld, wgs_ld, wds_ld;
  const uint8_t* wsg;
  const uint8_t* wsu;
  const uint8_t* wsd;
};

// MX operands of GEMM1 for m-tile row block A (codes) / As (scales) of local expert e.
__device__ __forceinline__ MxOperands mx_ops_gemm1(const FwdParams& p, const uint8_t* A,
                                                   const uint8_t* As, int e) {
  const int64_t wsz = int64_t(p.I) * p.D;
  MxOperands o;
  o.A = A; o.As = As; o.as_ld = p.xs_ld;
  o.w0 = static_cast<const uint8_t*>(p.a.wg) + e * wsz;
  o.w0s = p.wsg + int64_t(e) * p.I * p.wgs_ld;
  o.w1 = static_cast<const uint8_t*>(p.a.wu) + e * wsz;
  o.w1s = p.wsu + int64_t(e) * p.I * p.wgs_ld;
  o.ws_ld = p.wgs_ld;
  return o;
}
__device__ __forceinline__ MxOperands mx_ops_gemm2(const FwdParams& p, const uint8_t* A,
                                                   const uint8_t* As, int e) {
  const int64_t wsz = int64_t(p.I) * p.D;
  MxOperands o;
  o.A = A; o.As = As; o.as_ld = p.hs_ld;
  o.w0 = static_cast<const uint8_t*>(p.a.wd) + e * wsz;
  o.w0s = p.wsd + int64_t(e) * p.D * p.wds_ld;
  o.w1 = o.w0; o.w1s = o.w0s;
  o.ws_ld = p.wds_ld;
  return o;
}

// ------------------------------------------------------------------------------------
// combine
// ------------------------------------------------------------------------------------
// y[t] = sum_j gate_j * o[t*k+j] over the slots j with a local row, in ascending j
// (wave_pair_sum_loaded).
// Routed row r: combine its token if r is the token's last local row.  The token's slot
// rows and gates are loaded together, once, for both the test and the sum.
__device__ __forceinline__ void combine_if_last(const FwdParams& p, int r) {
  const int lane = threadIdx.x & 63;
  const int t = p.P.perm[r] / p.k;
  const int64_t q0 = int64_t(t) * p.k;
  const int32_t ps = lane < p.k ? p.P.pos[q0 + lane] : -1;
  const float g = lane < p.k ? p.a.gates[q0 + lane] : 0.f;
  if (wave_max(ps) == r)
    wave_pair_sum_loaded<kCpolDev | kCpolStream, 4>(p.a.y + q0 / p.k * p.D, p.P.obuf, q0, p.D, ps, g);
}

// ------------------------------------------------------------------------------------
// Unfused kernels: the same steps over full-size buffers, one launch per step.
// ------------------------------------------------------------------------------------
// With MOK_FLAG_TRACE, every workgroup of launch ph (0 gather, 1 GEMM1, 2 GEMM2,
// 3 combine) writes its start and end, 64-bit values of the 100 MHz constant clock, to
// its own record: 64-bit words ph_rec[ph] + 2 blockIdx.x and + 1 of the trace region (no
// atomics, so the records do not slow the launch down).  The end is taken once the
// workgroup's memory operations have completed.  k_phase_init writes the four launches'
// workgroup counts into the region's first words.
__global__ __launch_bounds__(64) void k_phase_init(uint32_t* trace, uint32_t g0, uint32_t g1,
                                                   uint32_t g2, uint32_t g3) {
  if (threadIdx.x < 8) trace[threadIdx.x] = threadIdx.x == 0 ? g0 : threadIdx.x == 1 ? g1 :
                                            threadIdx.x == 2 ? g2 : threadIdx.x == 3 ? g3 : 0u;
}
__device__ __forceinline__ uint64_t phase_start(const FwdParams& p) {
  return p.P.trace ? wall_clock64() : 0ull;
}
__device__ __forceinline__ void phase_end(const FwdParams& p, int ph, uint64_t t0) {
  if (!p.P.trace) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t* rec = reinterpret_cast<uint64_t*>(p.P.trace) + p.ph_rec[ph] + 2 * int64_t(blockIdx.x);
    rec[0] = t0;
    rec[1] = wall_clock64();
  }
}

template <bool MX>
__global__ __launch_bounds__(256) void k_gather_all(FwdParams p) {
  const uint64_t t0 = phase_start(p);
  const int R = int(p.P.hdr[kHdrR]);
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  for (int r = gw; r < R; r += nw) {
    const uint16_t* src = p.a.x + int64_t(p.P.perm[r] / p.k) * p.D;
    if (MX)
      wave_quant_row<false>(p.P.full_x + int64_t(r) * p.D, p.P.full_xs + int64_t(r) * p.xs_ld,
                            src, p.D);
    else
      wave_copy_row<false>(reinterpret_cast<uint16_t*>(p.P.full_x) + int64_t(r) * p.D, src, p.D);
  }
  phase_end(p, 0, t0);
}

template <bool MX>
__device__ __forceinline__ void gemm1_tile_unfused(const FwdParams& p) {
  const int nt = blockIdx.x % p.nN1;
  const int f = blockIdx.x / p.nN1;
  const int mb = f / p.mt_max, i = f % p.mt_max;
  if (mb >= int(p.P.hdr[kHdrNmb]) || i >= p.P.mt_cnt[mb]) return;
  const int4 e = p.P.mt_tab[int64_t(mb) * p.mt_max + i];
  if (MX) {
    TileAcc acc;
    const MxOperands o = mx_ops_gemm1(p, p.P.full_x + int64_t(e.x) * p.D,
                                      p.P.full_xs + int64_t(e.x) * p.xs_ld, e.z);
    run_tile_mx<false>(true, o, e.y, nt * kBN1, p.D, p.I, acc);
    epi_swiglu_mx<false>(acc, e.y, nt * kBN1, p.I, p.P.full_h + int64_t(e.x) * p.I, p.I,
                         p.P.full_hs + int64_t(e.x) * p.hs_ld, p.hs_ld,
                         p.save ? p.P.bab + int64_t(e.x) * 2 * p.I : nullptr);
    return;
  }
  const uint16_t* X = reinterpret_cast<const uint16_t*>(p.P.full_x);
  uint16_t* H = reinterpret_cast<uint16_t*>(p.P.full_h);
  const int64_t wsz = int64_t(p.I) * p.D;
  TileAcc acc;
  run_tile<false>(true, X + int64_t(e.x) * p.D, e.y,
                  reinterpret_cast<const uint16_t*>(p.a.wg) + e.z * wsz,
                  reinterpret_cast<const uint16_t*>(p.a.wu) + e.z * wsz, nt * kBN1, p.D, p.I, acc);
  // saving for the backward: a, b of every row go straight to its row buffer
  epi_swiglu<false>(acc, e.y, nt * kBN1, p.I, H + int64_t(e.x) * p.I, p.I,
                    p.save ? p.P.bab + int64_t(e.x) * 2 * p.I : nullptr);
}

template <bool MX>
__global__ __launch_bounds__(512) void k_gemm1_all(FwdParams p) {
  const uint64_t t0 = phase_start(p);
  gemm1_tile_unfused<MX>(p);
  phase_end(p, 1, t0);
}

template <bool MX>
__device__ __forceinline__ void gemm2_tile_unfused(const FwdParams& p) {
  const int nt = blockIdx.x % p.nN2;
  const int f = blockIdx.x / p.nN2;
  const int mb = f / p.mt_max, i = f % p.mt_max;
  if (mb >= int(p.P.hdr[kHdrNmb]) || i >= p.P.mt_cnt[mb]) return;
  const int4 e = p.P.mt_tab[int64_t(mb) * p.mt_max + i];
  if (MX) {
    TileAcc acc;
    const MxOperands o = mx_ops_gemm2(p, p.P.full_h + int64_t(e.x) * p.I,
                                      p.P.full_hs + int64_t(e.x) * p.hs_ld, e.z);
    run_tile_mx<false>(false, o, e.y, nt * kBN2, p.D, p.I, acc);
    epi_scatter<false, true>(acc, e.y, nt * kBN2, p.D, p.P.perm + e.x, p.P.obuf, int64_t(p.T) * p.k);
    return;
  }
  const uint16_t* H = reinterpret_cast<const uint16_t*>(p.P.full_h);
  const int64_t wsz = int64_t(p.I) * p.D;
  TileAcc acc;
  run_tile<false>(false, H + int64_t(e.x) * p.I, e.y,
                  reinterpret_cast<const uint16_t*>(p.a.wd) + e.z * wsz, nullptr, nt * kBN2, p.D,
                  p.I, acc);
  epi_scatter<false, true>(acc, e.y, nt * kBN2, p.D, p.P.perm + e.x, p.P.obuf, int64_t(p.T) * p.k);
}

template <bool MX>
__global__ __launch_bounds__(512) void k_gemm2_all(FwdParams p) {
  const uint64_t t0 = phase_start(p);
  gemm2_tile_unfused<MX>(p);
  phase_end(p, 2, t0);
}

// One wave per token; the next token's slot rows and gates are loaded while this one is
// summed, so that the per-token lookups do not add a memory round trip each.  Two slots of
// 16 chunks per lane at a time: a whole row of D <= 8192 per pass (measured on MI355X:
// config-3 combine 81 -> 76 us against four slots of 8 chunks; config 4 unchanged).
__global__ __launch_bounds__(256) void k_combine_all(FwdParams p) {
  const uint64_t t0 = phase_start(p);
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int lane = threadIdx.x & 63;
  auto load = [&](int t, int32_t& ps, float& g) {
    const bool on = t < p.T && lane < p.k;
    ps = on ? p.P.pos[int64_t(t) * p.k + lane] : -1;
    g = on ? p.a.gates[int64_t(t) * p.k + lane] : 0.f;
  };
  int32_t ps_n;
  float g_n;
  load(gw, ps_n, g_n);
  for (int t = gw; t < p.T; t += nw) {
    const int32_t ps = ps_n;
    const float g = g_n;
    load(t + nw, ps_n, g_n);
    if (wave_max(ps) >= 0)
      wave_pair_sum_loaded<kCpolStream, 2, 16>(p.a.y + int64_t(t) * p.D, p.P.obuf, int64_t(t) * p.k,
                                          p.D, ps, g);
    else
      wave_zero_row(p.a.y + int64_t(t) * p.D, p.D);
  }
  phase_end(p, 3, t0);
}

// ------------------------------------------------------------------------------------
// Fused persistent kernel
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fwd_prep(FwdParams p) {
  const int64_t words = 2 * int64_t(p.n_mb_max) + int64_t(p.n_mb_max) * p.mt_max;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < words; i += gridDim.x * 256) p.P.sync[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    p.P.hdr[kHdrFwdTicket] = 0;
    p.P.hdr[kHdrDrainTicket] = 0;
    p.P.hdr[kHdrAbort] = 0;
    p.P.hdr[kHdrArrive] = 0;
    p.P.hdr[kHdrFillTicket] = 0;
  }
}

// Rows of minibatch mb into its ring slot (slot mb mod S), row r by wave (r - lo) mod nw
// == gw; MXFP8 rows are quantised on the way.  When a row fits in one pass (D <= 8192),
// the loads of the wave's next row are issued before the current row is stored: vector
// memory operations retire in issue order, so waiting for a load issued after a store
// would also wait for that store to reach memory.  Two row buffers alternate, so no
// register copy forces an early wait.
template <bool MX>
__device__ __forceinline__ void gather_mb(const FwdParams& p, int mb, int gw, int nw) {
  gw = __builtin_amdgcn_readfirstlane(gw);
  uint8_t* slot = p.P.ring + (mb % p.S) * p.slot_bytes;
  const int lo = p.P.mb_start[mb], hi = p.P.mb_start[mb + 1];
  const uint32_t bytes = uint32_t(p.D) * 2;
  auto src_row = [&](int r) { return p.a.x + int64_t(p.P.perm[r] / p.k) * p.D; };
  if (bytes > 64u * 16u * kRowBatch) {
    for (int r = lo + gw; r < hi; r += nw) {
      if (MX)
        wave_quant_row<true>(slot + p.slot_x + int64_t(r - lo) * p.D,
                             slot + p.slot_xs + int64_t(r - lo) * p.xs_ld, src_row(r), p.D);
      else
        wave_copy_row<true>(reinterpret_cast<uint16_t*>(slot + p.slot_x) + int64_t(r - lo) * p.D,
                            src_row(r), p.D);
    }
    return;
  }
  static_assert(kRowBatch == kQuantBatch, "one pass holds the same chunks in both paths");
  const int r0 = lo + gw;
  if (r0 >= hi) return;
  const int nrows = (hi - r0 + nw - 1) / nw;  // the wave's rows: r0 + i * nw, i < nrows
  const uint32_t lane = threadIdx.x & 63;
  // perm of the wave's rows, 64 at a time (lane j holds row i0 + j): one vector load
  // per 64 rows, whose wait also covers the stores issued before it
  int32_t pv = 0;
  auto token_of = [&](int i) {
    if ((i & 63) == 0) {
      const int j = i + int(lane);
      pv = j < nrows ? p.P.perm[r0 + j * nw] : 0;
    }
    return __builtin_amdgcn_readlane(pv, i & 63) / p.k;
  };
  // loads of the wave's row i into buf (an empty range when i >= nrows: nothing is read)
  auto issue = [&](v4u (&buf)[kRowBatch], int i) {
    const bool live = i < nrows;
    const rsrc_t rs = row_rsrc(live ? p.a.x + int64_t(token_of(i)) * p.D : p.a.x,
                               live ? bytes : 0u);
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) buf[u] = buf_ld16<kCpolPlain>(rs, (lane + 64 * u) * 16);
  };
  auto put = [&](const v4u (&buf)[kRowBatch], int i) {
    const int64_t q = int64_t(r0 - lo) + int64_t(i) * nw;  // row within the slot
    if (MX) {
      const rsrc_t rc = row_rsrc(slot + p.slot_x + q * p.D, uint32_t(p.D));
      const rsrc_t rsc = row_rsrc(slot + p.slot_xs + q * p.xs_ld, uint32_t(p.D) >> 5);
      quant_store_pass<kCpolDev>(buf, rc, rsc, 0);
    } else {
      const rsrc_t rd = row_rsrc(slot + p.slot_x + q * bytes, bytes);
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) buf_st16<kCpolDev>(rd, (lane + 64 * u) * 16, buf[u]);
    }
  };
  // two row buffers in turn, so that two rows' loads are in flight
  v4u a[kRowBatch], b[kRowBatch];
  issue(a, 0);
  for (int i = 0;;) {
    issue(b, i + 1);
    put(a, i);
    if (++i >= nrows) break;
    issue(a, i + 1);
    put(b, i);
    if (++i >= nrows) break;
  }
}

// The fill: minibatch 0's rows go into slot 0 in chunks of one row per wave, taken from
// a ticket by every workgroup as it starts, before the roles split; ready[0] counts the
// rows done (the GEMM1 tiles of minibatch 0 wait for all of them).  Only running
// workgroups take chunks, so the fill never waits for one that has not started.
constexpr int kFillRows = kThreads / 64;

template <bool MX>
__device__ __forceinline__ void fill_mb0(const FwdParams& p, uint32_t* ready) {
  uint32_t* hdr = p.P.hdr;
  const int lo = p.P.mb_start[0], hi = p.P.mb_start[1];
  const uint32_t chunks = uint32_t((hi - lo + kFillRows - 1) / kFillRows);
  const int w = threadIdx.x >> 6;
  uint8_t* slot = p.P.ring;
  __shared__ uint32_t s_fk;
  uint32_t rows = 0;
  while (true) {
    if (threadIdx.x == 0) s_fk = fetch_add_relaxed(hdr + kHdrFillTicket, 1u);
    __syncthreads();
    const uint32_t fk = s_fk;
    __syncthreads();
    if (fk >= chunks) break;
    const int r0 = lo + int(fk) * kFillRows;
    rows += uint32_t(min(kFillRows, hi - r0));
    const int r = r0 + w;
    if (r < hi) {
      const uint16_t* src = p.a.x + int64_t(p.P.perm[r] / p.k) * p.D;
      if (MX)
        wave_quant_row<true>(slot + p.slot_x + int64_t(r - lo) * p.D,
                             slot + p.slot_xs + int64_t(r - lo) * p.xs_ld, src, p.D);
      else
        wave_copy_row<true>(reinterpret_cast<uint16_t*>(slot + p.slot_x) + int64_t(r - lo) * p.D,
                            src, p.D);
    }
  }
  if (rows) {
    perturb_pause(p.perturb, blockIdx.x);
    wg_signal_add(ready, rows);
  }
}

// Comm workgroups: gather minibatches 1.. into the ring (minibatch 0 is the fill, done by
// every workgroup before the roles split), reusing a slot once the GEMM2 tiles of the minibatch
// it held are done, and combine the tokens of that older minibatch.  The last S
// minibatches are combined in the drain.
template <bool MX>
__device__ __forceinline__ void comm_role(const FwdParams& p, int c, int C, uint32_t* ready, uint32_t* done) {
  uint32_t* hdr = p.P.hdr;
  const int n_mb = int(hdr[kHdrNmb]);
  const int w = threadIdx.x >> 6;
  const int gw = c * (kThreads / 64) + w, nw = C * (kThreads / 64);
  auto mb_tiles2 = [&](int mb) { return uint32_t(p.P.mt_cnt[mb] * p.nN2); };
  for (int mb = 1; mb < n_mb; ++mb) {
    if (mb >= p.S) {
      if (!wg_wait_geq(done + (mb - p.S), mb_tiles2(mb - p.S), hdr, p.wait_ticks)) return;
    }
    gather_mb<MX>(p, mb, gw, nw);
    perturb_pause(p.perturb, blockIdx.x * 7919u + uint32_t(mb));
    wg_signal_add(ready + mb, 1);
    if (mb >= p.S) {
      const int cm = mb - p.S;
      const int lo = p.P.mb_start[cm], hi = p.P.mb_start[cm + 1];
      for (int r = lo + gw; r < hi; r += nw) combine_if_last(p, r);
    }
  }
}

// Waits until the GEMM2 tiles of minibatches [from, to] are all done.  Wave 0 checks 64
// counters per load; only the unfinished ones are waited for.
__device__ __forceinline__ bool wait_done_range(const FwdParams& p, const uint32_t* done,
                                                int from, int to) {
  __shared__ uint64_t s_pending;
  for (int c0 = from; c0 <= to; c0 += 64) {
    if (threadIdx.x < 64) {
      const int c = c0 + int(threadIdx.x);
      const bool pend = c <= to && ld_relaxed(done + c) < uint32_t(p.P.mt_cnt[c] * p.nN2);
      const uint64_t b = __ballot(pend);
      if (threadIdx.x == 0) s_pending = b;
    }
    __syncthreads();
    uint64_t m = s_pending;
    __syncthreads();
    while (m) {
      const int c = c0 + __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      if (!wg_wait_geq(done + c, uint32_t(p.P.mt_cnt[c] * p.nN2), p.P.hdr, p.wait_ticks))
        return false;
    }
  }
  return true;
}

// MOK_FLAG_TRACE: low 32 bits of the 100 MHz constant clock, and one record of 8 words
// written by thread 0 (the layout is documented with mok_trace_layout).
__device__ __forceinline__ uint32_t trace_now() { return uint32_t(wall_clock64()); }
__device__ __forceinline__ void trace_put(uint32_t* rec, uint32_t a, uint32_t b, uint32_t c,
                                          uint32_t d, uint32_t e, uint32_t f, uint32_t g = 0) {
  if (threadIdx.x != 0) return;
  rec[0] = a; rec[1] = b; rec[2] = c; rec[3] = d; rec[4] = e; rec[5] = f; rec[6] = g; rec[7] = 0;
}

// Drain, run by every workgroup once its role is done, so that the compute CUs help with
// the data movement left at the end (with MOK_FLAG_OVERLAP_NEXT only the data movers run
// it, and the compute CUs go to the next macrobatch's forward).  Work comes in chunks from a ticket: first the
// token chunks (y = 0 for tokens without a local row), then, minibatch by minibatch, the
// row chunks of the last S minibatches.  A row chunk of minibatch cm combines the tokens
// whose last row it holds; their other rows lie in minibatches before cm, whose GEMM2
// tiles may finish after cm's, so it waits for the tiles of every minibatch up to cm.
constexpr int kDrainTokens = 64;
constexpr int kDrainRows = 8;  // one row per wave: the final combine spreads over every CU

__device__ __forceinline__ uint32_t drain(const FwdParams& p, const uint32_t* done) {
  uint32_t* hdr = p.P.hdr;
  const int n_mb = int(hdr[kHdrNmb]);
  const int w = threadIdx.x >> 6;
  constexpr int W = kThreads / 64;
  const uint32_t nz = uint32_t((p.T + kDrainTokens - 1) / kDrainTokens);
  auto chunks = [&](int mb) {
    return uint32_t((p.P.mb_start[mb + 1] - p.P.mb_start[mb] + kDrainRows - 1) / kDrainRows);
  };
  __shared__ uint32_t s_tk;
  int cm = max(0, n_mb - p.S);
  uint32_t cbase = nz;  // first ticket of minibatch cm's row chunks (tickets only grow)
  int waited = 0;       // minibatches [0, waited) are known to be done
  uint32_t taken = 0;   // chunks this workgroup took (trace)
  while (true) {
    if (threadIdx.x == 0) s_tk = fetch_add_relaxed(hdr + kHdrDrainTicket, 1u);
    __syncthreads();
    const uint32_t tk = s_tk;
    __syncthreads();
    if (aborted(hdr)) return taken;
    perturb_pause(p.perturb, tk * 31u + blockIdx.x);
    ++taken;
    if (tk < nz) {
      const int t1 = min(p.T, int(tk + 1) * kDrainTokens);
      for (int t = int(tk) * kDrainTokens + w; t < t1; t += W)
        if (token_last_row(p.P.pos, t, p.k) < 0) wave_zero_row(p.a.y + int64_t(t) * p.D, p.D);
      continue;
    }
    while (cm < n_mb && tk >= cbase + chunks(cm)) cbase += chunks(cm++);
    if (cm >= n_mb) return taken - 1;  // this ticket was past the last chunk
    if (waited <= cm) {
      if (!wait_done_range(p, done, waited, cm)) return taken;
      waited = cm + 1;
    }
    const int lo = p.P.mb_start[cm] + int(tk - cbase) * kDrainRows;
    const int hi = min(p.P.mb_start[cm + 1], lo + kDrainRows);
    for (int r = lo + w; r < hi; r += W) combine_if_last(p, r);
  }
}

template <bool MX>
__device__ __forceinline__ void compute_role(const FwdParams& p, int vid, int C,
                                             uint32_t* ready, uint32_t* done, uint32_t* hdone) {
  uint32_t* hdr = p.P.hdr;
  const uint32_t total = hdr[kHdrFwdTiles];
  const int n_mb = int(hdr[kHdrNmb]);
  const int64_t wsz = int64_t(p.I) * p.D;
  __shared__ uint32_t s_ticket;
  const int L = p.S >= 2 ? 1 : 0;
  const uint32_t per_mt = uint32_t(p.nN1 + p.nN2);
  const bool trace = p.P.trace != nullptr;
  // m-tiles in minibatches [0, i), and the first ticket of block j
  auto mt_before = [&](int i) {
    i = i < 0 ? 0 : (i > n_mb ? n_mb : i);
    return uint32_t(p.P.tile_base[i]) / per_mt;
  };
  auto block_start = [&](int j) {
    return uint32_t(p.nN1) * mt_before(j) + uint32_t(p.nN2) * mt_before(j - L);
  };
  int j = 0;
  while (true) {
    if (threadIdx.x == 0) s_ticket = fetch_add_relaxed(hdr + kHdrFwdTicket, 1u);
    __syncthreads();
    const uint32_t tk = s_ticket;
    __syncthreads();
    if (tk >= total || aborted(hdr)) break;
    const uint32_t t_tk = trace ? trace_now() : 0u;
    while (j + 1 < n_mb + L && block_start(j + 1) <= tk) ++j;
    const uint32_t q0 = tk - block_start(j);
    const uint32_t g1n = j < n_mb ? uint32_t(p.P.mt_cnt[j] * p.nN1) : 0u;
    const bool g1 = q0 < g1n;
    const int mb = g1 ? j : j - L;
    const int q = int(g1 ? q0 : q0 - g1n + uint32_t(p.P.mt_cnt[mb] * p.nN1));
    const int nmt = p.P.mt_cnt[mb];
    const int s = mb % p.S;
    uint8_t* slot = p.P.ring + s * p.slot_bytes;
    uint16_t* slot_x = reinterpret_cast<uint16_t*>(slot + p.slot_x);
    uint16_t* slot_h = reinterpret_cast<uint16_t*>(slot + p.slot_h);
    const int lo = p.P.mb_start[mb];
    const int qq = g1 ? q : q - nmt * p.nN1;
    const int nn = g1 ? p.nN1 : p.nN2;
    const int i = qq / nn, nt = qq % nn;
    uint32_t* hd = hdone + int64_t(mb) * p.mt_max + i;
    if (g1) {
      const uint32_t need = mb == 0 ? uint32_t(p.P.mb_start[1] - p.P.mb_start[0]) : uint32_t(C);
      if (!wg_wait_geq(ready + mb, need, hdr, p.wait_ticks)) break;
    } else {
      if (!wg_wait_geq(hd, uint32_t(p.nN1), hdr, p.wait_ticks)) break;
    }
    const uint32_t t_ready = trace ? trace_now() : 0u;
    uint32_t* rec = trace ? p.P.trace + int64_t(tk) * 8 : nullptr;
    const uint32_t kind = (uint32_t(mb) << 1) | (g1 ? 0u : 1u);
    const int4 e = p.P.mt_tab[int64_t(mb) * p.mt_max + i];
    const int r0 = e.x - lo;
    if (MX) {
      const int n0 = nt * (g1 ? kBN1 : kBN2);
      TileAcc acc;
      if (g1) {
        const MxOperands o = mx_ops_gemm1(p, slot + p.slot_x + int64_t(r0) * p.D,
                                          slot + p.slot_xs + int64_t(r0) * p.xs_ld, e.z);
        run_tile_mx<true>(true, o, e.y, n0, p.D, p.I, acc);
        const uint32_t t_k = trace ? trace_now() : 0u;
        // saving for the backward: a, b of every row go to the row buffer (the MXFP8
        // backward reads them there, so no minibatch is replayed)
        epi_swiglu_mx<true>(acc, e.y, n0, p.I, slot + p.slot_h + int64_t(r0) * p.I, p.I,
                            slot + p.slot_hs + int64_t(r0) * p.hs_ld, p.hs_ld,
                            p.save ? p.P.bab + int64_t(e.x) * 2 * p.I : nullptr);
        const uint32_t t_e = trace ? trace_now() : 0u;
        perturb_pause(p.perturb, tk);
        wg_signal_add(hd, 1);
        if (trace) trace_put(rec, uint32_t(vid), kind, t_tk, t_ready, t_k, trace_now(), t_e);
      } else {
        const MxOperands o = mx_ops_gemm2(p, slot + p.slot_h + int64_t(r0) * p.I,
                                          slot + p.slot_hs + int64_t(r0) * p.hs_ld, e.z);
        run_tile_mx<true>(false, o, e.y, n0, p.D, p.I, acc);
        const uint32_t t_k = trace ? trace_now() : 0u;
        epi_scatter<true, true>(acc, e.y, n0, p.D, p.P.perm + e.x, p.P.obuf, int64_t(p.T) * p.k);
        const uint32_t t_e = trace ? trace_now() : 0u;
        perturb_pause(p.perturb, tk);
        wg_signal_add(done + mb, 1);
        if (trace) trace_put(rec, uint32_t(vid), kind, t_tk, t_ready, t_k, trace_now(), t_e);
      }
      continue;
    }
    const uint16_t* A = g1 ? slot_x + int64_t(r0) * p.D : slot_h + int64_t(r0) * p.I;
    const uint16_t* w0 = reinterpret_cast<const uint16_t*>(g1 ? p.a.wg : p.a.wd) + e.z * wsz;
    const uint16_t* w1 = reinterpret_cast<const uint16_t*>(p.a.wu) + e.z * wsz;
    const int n0 = nt * (g1 ? kBN1 : kBN2);
    TileAcc acc;
    run_tile<true>(g1, A, e.y, w0, w1, n0, p.D, p.I, acc);
    const uint32_t t_k = trace ? trace_now() : 0u;
    uint32_t t_e = 0u;
    if (g1) {
      uint16_t* ab = p.save ? reinterpret_cast<uint16_t*>(slot + p.slot_ab) + int64_t(r0) * 2 * p.I
                            : nullptr;
      epi_swiglu<true>(acc, e.y, n0, p.I, slot_h + int64_t(r0) * p.I, p.I, ab);
      t_e = trace ? trace_now() : 0u;
      perturb_pause(p.perturb, tk);
      wg_signal_add(hd, 1);
    } else {
      epi_scatter<true, true>(acc, e.y, n0, p.D, p.P.perm + e.x, p.P.obuf, int64_t(p.T) * p.k);
      t_e = trace ? trace_now() : 0u;
      perturb_pause(p.perturb, tk);
      wg_signal_add(done + mb, 1);
    }
    if (trace) trace_put(rec, uint32_t(vid), kind, t_tk, t_ready, t_k, trace_now(), t_e);
  }
}

template <bool MX>
__global__ __launch_bounds__(512) void k_fwd_fused(FwdParams p) {
  uint32_t* ready = p.P.sync;
  uint32_t* done = ready + p.n_mb_max;
  uint32_t* hdone = done + p.n_mb_max;
  const int C = p.a.comm_cus;
  // the workgroup's number in order of arrival: roles go to running workgroups
  __shared__ uint32_t s_vid;
  if (threadIdx.x == 0) s_vid = fetch_add_relaxed(p.P.hdr + kHdrArrive, 1u);
  __syncthreads();
  const int vid = int(s_vid);
  const bool trace = p.P.trace != nullptr && vid < MOK_TRACE_MAX_WORKGROUPS;
  const uint32_t t0 = trace ? trace_now() : 0u;
  if (p.P.hdr[kHdrNmb] > 0) fill_mb0<MX>(p, ready);
  const uint32_t t1 = trace ? trace_now() : 0u;
  if (vid < C) comm_role<MX>(p, vid, C, ready, done);
  else compute_role<MX>(p, vid, C, ready, done, hdone);
  const uint32_t t2 = trace ? trace_now() : 0u;
  // macrobatch interleave: a compute workgroup leaves once no tile is left, so that the
  // next macrobatch's forward can start on its CU while the data movers drain this one
  const uint32_t nd = (p.overlap_next && vid >= C) ? 0u : drain(p, done);
  if (trace)
    trace_put(p.P.trace + p.trace_tiles * 8 + int64_t(vid) * 8, t0, t1, t2, trace_now(),
              vid < C ? 1u : 0u, nd);
}

// ------------------------------------------------------------------------------------
// host
// ------------------------------------------------------------------------------------
static FwdParams make_params(const Layout& L, const Ptrs& P, const FwdArgs& a) {
  FwdParams p;
  p.P = P;
  p.a = a;
  p.T = int(L.T); p.D = int(L.D); p.I = int(L.I); p.k = int(L.k); p.M = int(L.M);
  p.S = int(L.S); p.mt_max = int(L.mt_max); p.nN1 = int(L.nN1); p.nN2 = int(L.nN2);
  p.n_mb_max = int(L.n_mb_max); p.save = L.save ? 1 : 0;
  p.wait_ticks = L.short_waits ? kShortWaitTicks : kWaitTicks;
  p.perturb = L.perturb ? 1 : 0;
  p.overlap_next = L.overlap_next ? 1 : 0;
  p.trace_tiles = int64_t(L.trace_tickets);
  for (int ph = 0, w = 4; ph < 4; w += 2 * int(L.unf_grid[ph]), ++ph) p.ph_rec[ph] = w;
  p.slot_bytes = int64_t(L.slot_bytes); p.slot_x = int64_t(L.slot_x);
  p.slot_xs = int64_t(L.slot_xs); p.slot_h = int64_t(L.slot_h); p.slot_hs = int64_t(L.slot_hs);
  p.slot_ab = int64_t(L.slot_ab);
  p.xs_ld = L.xs_ld; p.hs_ld = L.hs_ld; p.wgs_ld = L.wgs_ld; p.wds_ld = L.wds_ld;
  p.wsg = L.repack_wg ? P.wsg : a.sg;
  p.wsu = L.repack_wg ? P.wsu : a.su;
  p.wsd = L.repack_wd ? P.wsd : a.sd;
  return p;
}

static int fused_grid_size(const void* kernel) {
  int dev = 0, cus = 0, occ = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, 0) != hipSuccess)
    return 0;
  return cus * occ;
}

mok_status_t launch_forward(const Layout& L, const Ptrs& P, const FwdArgs& a, hipStream_t st) {
  FwdParams p = make_params(L, P, a);
  // the fused kernel's grid (device queries only), checked before anything is enqueued
  const void* kern = L.mx ? reinterpret_cast<const void*>(k_fwd_fused<true>)
                          : reinterpret_cast<const void*>(k_fwd_fused<false>);
  const int grid = L.unfused ? 0 : fused_grid_size(kern);
  if (!L.unfused && grid <= 0) return MOK_E_DEVICE;
  if (!L.unfused && a.comm_cus >= grid) return MOK_E_SHAPE;
  if (L.repack_wg) {
    launch_mx_repack(a.sg, L.nl * L.I, int(L.D / 32), P.wsg, int(L.wgs_ld), st);
    launch_mx_repack(a.su, L.nl * L.I, int(L.D / 32), P.wsu, int(L.wgs_ld), st);
  }
  if (L.repack_wd) launch_mx_repack(a.sd, L.nl * L.D, int(L.I / 32), P.wsd, int(L.wds_ld), st);
  if (L.unfused) {
    const unsigned gw = unsigned(L.unf_grid[0]), gc = unsigned(L.unf_grid[3]);
    const dim3 g1(unsigned(L.unf_grid[1])), g2(unsigned(L.unf_grid[2]));
    if (P.trace)
      hipLaunchKernelGGL(k_phase_init, dim3(1), dim3(64), 0, st, P.trace, gw, g1.x, g2.x, gc);
    if (L.mx) {
      hipLaunchKernelGGL(k_gather_all<true>, dim3(gw), dim3(256), 0, st, p);
      hipLaunchKernelGGL(k_gemm1_all<true>, g1, dim3(kThreads), 0, st, p);
      hipLaunchKernelGGL(k_gemm2_all<true>, g2, dim3(kThreads), 0, st, p);
    } else {
      hipLaunchKernelGGL(k_gather_all<false>, dim3(gw), dim3(256), 0, st, p);
      hipLaunchKernelGGL(k_gemm1_all<false>, g1, dim3(kThreads), 0, st, p);
      hipLaunchKernelGGL(k_gemm2_all<false>, g2, dim3(kThreads), 0, st, p);
    }
    hipLaunchKernelGGL(k_combine_all, dim3(gc), dim3(256), 0, st, p);
    return hipGetLastError() == hipSuccess ? MOK_OK : MOK_E_LAUNCH;
  }
  hipLaunchKernelGGL(k_fwd_prep, dim3(64), dim3(256), 0, st, p);
  if (L.mx)
    hipLaunchKernelGGL(k_fwd_fused<true>, dim3(grid), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(k_fwd_fused<false>, dim3(grid), dim3(kThreads), 0, st, p);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_E_LAUNCH;
}

}  // namespace mok
