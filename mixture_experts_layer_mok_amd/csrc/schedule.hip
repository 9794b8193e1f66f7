// Schedule: per-expert counts, offsets and the dispatch table (perm/pos) for one GPU's
// share of the routed pairs, plus the minibatch m-tile table the grouped GEMMs walk.
//
// What is computed follows the Leiphone article on MoK, section 01 (count each
// expert's rows, decide where each lands, keep one expert's rows together so the
// grouped GEMM gets regular input) and the news brief's design-decision section (a
// single schedule table drives all four transfers and costs a few percent of the
// layer).  The single-GPU form: a row's "source location" is its pair index t*k + j.
//
// The absolute first row of expert e's pairs in sub-chunk s is an exclusive prefix sum
// in expert-major order, q = e * NS + s, of the per-sub-chunk counts: it adds the rows of
// every earlier expert (the expert's offset) and of the expert's earlier sub-chunks.
//
// Two launches, no host synchronisation:
//   count  — each wave builds an LDS histogram of its 1024-pair sub-chunk;
//   place  — every workgroup scans the whole count table itself (it has nl * NS entries,
//            a few thousand at most on this path), workgroup 0 also writes the offsets,
//            R, the minibatch count and the m-tile table; then each wave walks its
//            sub-chunk 64 pairs at a time, grouping the lanes routed to one expert with a
//            ballot and ranking them with a prefix popcount, which keeps ascending (token,
//            slot) order inside every expert.
// A count table too large to scan in every workgroup (more than kFusedScanMax entries)
// takes a third launch between the two: one workgroup scans it and writes the tables.
// Each wave issues all loads of its sub-chunk before using any: these kernels are bound
// by memory latency, not bandwidth.
#include "device.h"
#include "launch.h"

namespace mok {

constexpr int kFusedScanMax = 8192;  // count-table entries every place workgroup scans

__global__ __launch_bounds__(256) void sched_count(const int32_t* __restrict__ ids, int64_t TK,
                                                   int E, int e0, int nl,
                                                   int32_t* __restrict__ blk) {
  __shared__ int32_t hist[4][kMaxLocalExperts + 1];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int e = lane; e <= nl; e += 64) hist[w][e] = 0;
  __syncthreads();
  const int64_t sub = int64_t(blockIdx.x) * 4 + w;
  const int64_t p0 = sub * kSchedSub;
  // all of the wave's loads first (one memory latency, not one per group of 64)
  constexpr int kG = kSchedSub / 64;
  int idv[kG];
#pragma unroll
  for (int u = 0; u < kG; ++u) {
    const int64_t p = p0 + 64 * u + lane;
    idv[u] = p < TK ? ids[p] : -1;
  }
  int bad = 0;
#pragma unroll
  for (int u = 0; u < kG; ++u) {
    const int id = idv[u];
    if (id < -1 || id >= E) {
      ++bad;
    } else if (id >= e0 && id < e0 + nl) {
      atomicAdd(&hist[w][id - e0], 1);
    }
  }
  if (bad) atomicAdd(&hist[w][nl], bad);
  __syncthreads();
  for (int e = lane; e <= nl; e += 64) blk[sub * (nl + 1) + e] = hist[w][e];
}

// Inclusive sum over the NW waves of the workgroup (wave prefix sums by shuffles, then
// the wave totals); *total receives the sum of all values.
template <int NW>
__device__ __forceinline__ int32_t block_incl_scan(int32_t v, int32_t* s_wave, int32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  if (lane == 63) s_wave[w] = v;
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int32_t t = s_wave[i];
    before += i < w ? t : 0;
    all += t;
  }
  __syncthreads();  // s_wave may be rewritten by the next call
  *total = all;
  return v + before;
}

// Tables written by one workgroup of NW waves once the offsets are known (s_off[0..nl],
// s_off[nl] = R, in LDS): counts, offsets, the header words, the m-tile table and the
// per-minibatch tile bases.  bad = ids outside [-1, E) (sets MOK_DEV_BAD_ID).
//
// m-tile table: expert e's rows are cut into m-tiles [off_e + kBM*q, +kBM) (the last one
// may be short); minibatch mb holds the m-tiles whose first row lies in its window
// [mb*M, (mb+1)*M), so it covers rows [mb_start[mb], mb_start[mb+1]) and may run up to
// kBM-1 rows past its window.  mb_start[n_mb] = R.  tile_base: prefix over minibatches
// of m-tiles * (nN1 + nN2).
template <int NW>
__device__ void write_tables(const Ptrs& P, const int32_t* s_off, int32_t* s_wave, int nl,
                             int M, int mt_max, int nN1, int nN2, int32_t bad) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x;
  for (int e = tid; e < nl; e += NT) {
    P.counts[e] = s_off[e + 1] - s_off[e];
    P.offsets[e] = s_off[e];
  }
  const int32_t R = s_off[nl];
  const int32_t n_mb = (R + M - 1) / M;
  if (tid == 0) {
    P.offsets[nl] = R;
    P.hdr[kHdrStatus] = bad ? MOK_DEV_BAD_ID : 0u;
    P.hdr[kHdrR] = uint32_t(R);
    P.hdr[kHdrNmb] = uint32_t(n_mb);
  }
  int32_t carry_mt = 0;
  for (int base = 0; base < n_mb; base += NT) {
    const int mb = base + tid;
    int cnt = 0;
    if (mb < n_mb) {
      const int32_t lo = mb * M;
      const int32_t hi = min(lo + M, R);
      int e_lo = 0, e_hi = nl - 1;  // expert whose rows contain lo
      while (e_lo < e_hi) {
        const int mid = (e_lo + e_hi) >> 1;
        if (s_off[mid + 1] <= lo) e_lo = mid + 1; else e_hi = mid;
      }
      int e = e_lo;
      int32_t t = s_off[e] + ((lo - s_off[e] + kBM - 1) / kBM) * kBM;  // first tile start >= lo
      if (t >= s_off[e + 1]) {
        t = s_off[e + 1];
        ++e;
      }
      P.mb_start[mb] = t;
      while (t < hi) {
        while (e < nl && s_off[e + 1] <= t) ++e;  // skip finished and empty experts
        const int32_t rows = min(kBM, s_off[e + 1] - t);
        P.mt_tab[int64_t(mb) * mt_max + cnt] = make_int4(t, rows, e, 0);
        ++cnt;
        t += rows;
      }
      P.mt_cnt[mb] = cnt;
    }
    int32_t tot = 0;
    const int32_t incl = block_incl_scan<NW>(cnt, s_wave, &tot);
    if (mb < n_mb) P.tile_base[mb] = (carry_mt + incl - cnt) * (nN1 + nN2);
    carry_mt += tot;
  }
  if (tid == 0) {
    P.mb_start[n_mb] = R;
    P.tile_base[n_mb] = carry_mt * (nN1 + nN2);
    P.hdr[kHdrMtiles] = uint32_t(carry_mt);
    P.hdr[kHdrFwdTiles] = uint32_t(carry_mt * (nN1 + nN2));
  }
}

// ids outside [-1, E), summed over the sub-chunks (column nl of the count table).
template <int NW>
__device__ __forceinline__ int32_t count_bad(const int32_t* blk, int64_t NS, int nl,
                                             int32_t* s_wave) {
  int32_t bad = 0;
  for (int64_t sc = threadIdx.x; sc < NS; sc += NW * 64) bad += blk[sc * (nl + 1) + nl];
  int32_t total = 0;
  block_incl_scan<NW>(bad, s_wave, &total);
  return total;
}

// Large count tables: one workgroup of 1024 threads turns the counts into absolute bases
// in place (one parallel scan over the nl * NS counts, in passes of 1024) and writes the
// tables.
__global__ __launch_bounds__(1024) void sched_scan(Ptrs P, int64_t NS, int nl, int M, int mt_max,
                                                   int nN1, int nN2) {
  __shared__ int32_t s_off[kMaxLocalExperts + 1];
  __shared__ int32_t s_wave[16];
  const int tid = threadIdx.x;
  const int64_t n = int64_t(nl) * NS;
  int32_t carry = 0, total = 0;
  for (int64_t q0 = 0; q0 < n; q0 += 1024) {
    const int64_t q = q0 + tid;
    const int64_t e = q / NS, sc = q - e * NS;
    int32_t* cell = P.blk + sc * (nl + 1) + e;
    const int32_t v = q < n ? *cell : 0;
    const int32_t excl = carry + block_incl_scan<16>(v, s_wave, &total) - v;
    if (q < n) {
      *cell = excl;
      if (sc == 0) s_off[e] = excl;
    }
    carry += total;
  }
  const int32_t bad = count_bad<16>(P.blk, NS, nl, s_wave);
  if (tid == 0) s_off[nl] = carry;
  __syncthreads();
  write_tables<16>(P, s_off, s_wave, nl, M, mt_max, nN1, nN2, bad);
}

// One wave places its sub-chunk (idv: its ids, lane l holding pair p0 + 64 u + l) from
// the bases of its sub-chunk (the first row of each expert's pairs in it).
//   kMode 0 (nl <= 16): one ballot per local expert and step; lane e keeps expert e's
//           next row;
//   kMode 1 (nl <= 64): one ballot round per distinct expert among the step's 64 pairs;
//           lane e keeps expert e's next row;
//   kMode 2 (larger): the same rounds, the next rows in LDS (base_lds).
template <int kMode>
__device__ __forceinline__ void place_subchunk(const int (&idv)[kSchedSub / 64], int64_t p0,
                                               int64_t TK, int e0, int nl, int32_t base_v,
                                               int32_t* base_lds, int32_t* __restrict__ perm,
                                               int32_t* __restrict__ pos) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int step = 0; step < kSchedSub / 64; ++step) {
    if (p0 + step * 64 >= TK) break;  // wave-uniform
    const int64_t p = p0 + step * 64 + lane;
    const bool valid = p < TK;
    const int id = idv[step];
    const bool local = valid && id >= e0 && id < e0 + nl;
    const int e = id - e0;
    int32_t row = -1;
    if (kMode == 0) {
      uint64_t mine = 0;
      int32_t add = 0;
      for (int x = 0; x < nl; ++x) {
        const uint64_t m = __ballot(local && e == x);
        if (local && e == x) mine = m;
        if (lane == x) add = __popcll(m);
      }
      const int32_t b = __shfl(base_v, local ? e : 0);
      if (local)
        row = b + int32_t(__builtin_amdgcn_mbcnt_hi(uint32_t(mine >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(uint32_t(mine), 0u)));
      base_v += add;
    } else {
      uint64_t todo = __ballot(local);
      while (todo) {
        const int leader = __ffsll((unsigned long long)todo) - 1;
        const int el = __builtin_amdgcn_readfirstlane(__shfl(e, leader));
        const uint64_t m = __ballot(local && e == el);
        const int32_t b = kMode == 1 ? __builtin_amdgcn_readlane(base_v, el) : base_lds[el];
        if (local && e == el) {
          const uint32_t below = __builtin_amdgcn_mbcnt_hi(
              uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
          row = b + int32_t(below);
        }
        if (kMode == 1) {
          if (lane == el) base_v = b + __popcll(m);
        } else if (lane == leader) {
          base_lds[el] = b + __popcll(m);
        }
        todo &= ~m;
      }
    }
    if (valid) {
      pos[p] = row;
      if (row >= 0) perm[row] = int32_t(p);
    }
  }
}

// One wave: its sub-chunk's ids (load_subchunk), its bases (bases[e * base_stride],
// e < nl): place.
__device__ __forceinline__ void load_subchunk(const int32_t* __restrict__ ids, int64_t TK,
                                              int64_t sub, int (&idv)[kSchedSub / 64]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kSchedSub / 64; ++u) {
    const int64_t p = sub * kSchedSub + 64 * u + lane;
    idv[u] = p < TK ? ids[p] : -1;
  }
}

template <int kMode>
__device__ __forceinline__ void place_wave(const int (&idv)[kSchedSub / 64], int64_t TK, int e0,
                                           int nl, int64_t sub, const int32_t* bases,
                                           int64_t base_stride, int32_t* base_lds,
                                           int32_t* __restrict__ perm, int32_t* __restrict__ pos) {
  const int lane = threadIdx.x & 63;
  const int64_t p0 = sub * kSchedSub;
  int32_t base_v = 0;
  if (kMode < 2) {
    base_v = lane < nl ? bases[int64_t(lane) * base_stride] : 0;
  } else {
    for (int e = lane; e < nl; e += 64) base_lds[e] = bases[int64_t(e) * base_stride];
  }
  place_subchunk<kMode>(idv, p0, TK, e0, nl, base_v, base_lds, perm, pos);
}

// Place after a separate scan: the bases of sub-chunk sub are blk[sub][0..nl).
template <int kMode>
__global__ __launch_bounds__(256) void sched_place(const int32_t* __restrict__ ids, int64_t TK,
                                                   int e0, int nl,
                                                   const int32_t* __restrict__ blk,
                                                   int32_t* __restrict__ perm,
                                                   int32_t* __restrict__ pos) {
  __shared__ int32_t base[4][kMode == 2 ? kMaxLocalExperts : 1];
  const int w = threadIdx.x >> 6;
  const int64_t sub = int64_t(blockIdx.x) * 4 + w;
  int idv[kSchedSub / 64];
  load_subchunk(ids, TK, sub, idv);
  place_wave<kMode>(idv, TK, e0, nl, sub, blk + sub * (nl + 1), 1, base[w], perm, pos);
}

// Place with the scan folded in: the workgroup loads the whole count table (nl * NS <=
// kFusedScanMax entries) in expert-major order into LDS, scans it (each thread a
// contiguous run), takes its waves' bases from it, and workgroup 0 writes the tables.
template <int kMode>
__global__ __launch_bounds__(256) void sched_place_scan(const int32_t* __restrict__ ids,
                                                        int64_t TK, int e0, Ptrs P, int64_t NS,
                                                        int nl, int M, int mt_max, int nN1,
                                                        int nN2) {
  __shared__ int32_t s_q[kFusedScanMax];
  __shared__ int32_t s_off[kMaxLocalExperts + 1];
  __shared__ int32_t s_wave[4];
  __shared__ int32_t base[4][kMode == 2 ? kMaxLocalExperts : 1];
  const int tid = threadIdx.x, w = tid >> 6;
  const int64_t sub = int64_t(blockIdx.x) * 4 + w;
  int idv[kSchedSub / 64];
  load_subchunk(ids, TK, sub, idv);  // in flight during the scan
  const int n = int(int64_t(nl) * NS);
  for (int q = tid; q < n; q += 256) s_q[q] = P.blk[int64_t(q % NS) * (nl + 1) + q / NS];
  __syncthreads();
  const int c = (n + 255) / 256, q0 = tid * c;
  int32_t sum = 0;
  for (int i = 0; i < c; ++i)
    if (q0 + i < n) sum += s_q[q0 + i];
  int32_t total = 0;
  int32_t run = block_incl_scan<4>(sum, s_wave, &total) - sum;
  for (int i = 0; i < c; ++i)
    if (q0 + i < n) {
      const int32_t v = s_q[q0 + i];
      s_q[q0 + i] = run;
      run += v;
    }
  __syncthreads();
  for (int e = tid; e < nl; e += 256) s_off[e] = s_q[int64_t(e) * NS];
  if (tid == 0) s_off[nl] = total;
  __syncthreads();
  // every wave has a sub-chunk (NS = 4 * workgroups); those past the pairs place nothing
  place_wave<kMode>(idv, TK, e0, nl, sub, s_q + sub, NS, base[w], P.perm, P.pos);
  if (blockIdx.x == 0) {
    const int32_t bad = count_bad<4>(P.blk, NS, nl, s_wave);
    write_tables<4>(P, s_off, s_wave, nl, M, mt_max, nN1, nN2, bad);
  }
}

mok_status_t launch_schedule(const Layout& L, const Ptrs& P, const int32_t* ids, hipStream_t st) {
  hipLaunchKernelGGL(sched_count, dim3(unsigned(L.NB)), dim3(256), 0, st, ids, L.TK, int(L.E),
                     int(L.e0), int(L.nl), P.blk);
  if (hipGetLastError() != hipSuccess) return MOK_E_LAUNCH;
  const int mode = L.nl <= 16 ? 0 : (L.nl <= 64 ? 1 : 2);
  const dim3 g(unsigned(L.NB)), b(256);
  if (L.nl * L.NS <= kFusedScanMax) {
    const int64_t TK = L.TK, NS = L.NS;
    const int e0 = int(L.e0), nl = int(L.nl), M = int(L.M), mt = int(L.mt_max),
              n1 = int(L.nN1), n2 = int(L.nN2);
    if (mode == 0)
      hipLaunchKernelGGL(sched_place_scan<0>, g, b, 0, st, ids, TK, e0, P, NS, nl, M, mt, n1, n2);
    else if (mode == 1)
      hipLaunchKernelGGL(sched_place_scan<1>, g, b, 0, st, ids, TK, e0, P, NS, nl, M, mt, n1, n2);
    else
      hipLaunchKernelGGL(sched_place_scan<2>, g, b, 0, st, ids, TK, e0, P, NS, nl, M, mt, n1, n2);
    return hipGetLastError() == hipSuccess ? MOK_OK : MOK_E_LAUNCH;
  }
  hipLaunchKernelGGL(sched_scan, dim3(1), dim3(1024), 0, st, P, L.NS, int(L.nl), int(L.M),
                     int(L.mt_max), int(L.nN1), int(L.nN2));
  if (hipGetLastError() != hipSuccess) return MOK_E_LAUNCH;
  if (mode == 0)
    hipLaunchKernelGGL(sched_place<0>, g, b, 0, st, ids, L.TK, int(L.e0), int(L.nl), P.blk,
                       P.perm, P.pos);
  else if (mode == 1)
    hipLaunchKernelGGL(sched_place<1>, g, b, 0, st, ids, L.TK, int(L.e0), int(L.nl), P.blk,
                       P.perm, P.pos);
  else
    hipLaunchKernelGGL(sched_place<2>, g, b, 0, st, ids, L.TK, int(L.e0), int(L.nl), P.blk,
                       P.perm, P.pos);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_E_LAUNCH;
}

}  // namespace mok
