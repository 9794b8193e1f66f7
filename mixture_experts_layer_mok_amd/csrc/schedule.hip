// Schedule: per-expert counts, offsets and the dispatch table (perm/pos) for one GPU's
// share of the routed pairs, plus the minibatch m-tile table the grouped GEMMs walk.
//
// What is computed follows the Leiphone article on MoK, section 01 (count each
// expert's rows, decide where each lands, keep one expert's rows together so the
// grouped GEMM gets regular input) and the news brief's design-decision section (a
// single schedule table drives all four transfers and costs a few percent of the
// layer).  The single-GPU form: a row's "source location" is its pair index t*k + j.
//
// Three launches, no host synchronisation:
//   count  — each wave builds an LDS histogram of its 1024-pair sub-chunk;
//   scan   — one workgroup turns the per-sub-chunk counts into absolute bases with one
//            parallel prefix sum in expert-major order, and writes the offsets, R, the
//            minibatch count and the m-tile table;
//   place  — each wave walks its sub-chunk 64 pairs at a time; lanes routed to the
//            same expert are grouped with a ballot and ranked with a prefix popcount,
//            which keeps ascending (token, slot) order inside every expert.
// Each wave issues all loads of its sub-chunk before using any: these kernels are
// bound by memory latency, not bandwidth.
#include "device.h"
#include "launch.h"

namespace mok {

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

// Inclusive sum over the 1024 threads of the workgroup (wave prefix sums by shuffles,
// then the 16 wave totals); *total receives the sum of all 1024 values.
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
  for (int i = 0; i < 16; ++i) {
    const int32_t t = s_wave[i];
    before += i < w ? t : 0;
    all += t;
  }
  __syncthreads();  // s_wave may be rewritten by the next call
  *total = all;
  return v + before;
}

// One workgroup of 1024 threads.  The absolute first row of expert e's pairs in
// sub-chunk s is an exclusive prefix sum in expert-major order, q = e * NS + s, of the
// per-sub-chunk counts: it adds the rows of every earlier expert (the expert's offset)
// and of the expert's earlier sub-chunks.  One parallel scan over those nl * NS counts,
// in passes of 1024, gives every base, the offsets (the bases at s = 0) and R.
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
    const int32_t excl = carry + block_incl_scan(v, s_wave, &total) - v;
    if (q < n) {
      *cell = excl;
      if (sc == 0) s_off[e] = excl;
    }
    carry += total;
  }
  // ids outside [-1, E): one counter per sub-chunk in column nl
  int32_t bad = 0;
  for (int64_t sc = tid; sc < NS; sc += 1024) bad += P.blk[sc * (nl + 1) + nl];
  block_incl_scan(bad, s_wave, &bad);
  if (tid == 0) s_off[nl] = carry;
  __syncthreads();
  for (int e = tid; e < nl; e += 1024) {
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
  // m-tile table.  Expert e's rows are cut into m-tiles [off_e + kBM*q, +kBM) (the last
  // one may be short); minibatch mb holds the m-tiles whose first row lies in its
  // window [mb*M, (mb+1)*M), so it covers rows [mb_start[mb], mb_start[mb+1]) and may
  // run up to kBM-1 rows past its window.  mb_start[n_mb] = R.
  for (int mb = tid; mb < n_mb; mb += 1024) {
    const int32_t lo = mb * M;
    const int32_t hi = min(lo + M, R);
    // expert whose rows contain lo
    int e_lo = 0, e_hi = nl - 1;
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
    int cnt = 0;
    while (t < hi) {
      while (e < nl && s_off[e + 1] <= t) ++e;  // skip finished and empty experts
      const int32_t rows = min(kBM, s_off[e + 1] - t);
      P.mt_tab[int64_t(mb) * mt_max + cnt] = make_int4(t, rows, e, 0);
      ++cnt;
      t += rows;
    }
    P.mt_cnt[mb] = cnt;
  }
  if (tid == 0) P.mb_start[n_mb] = R;
  __threadfence();
  __syncthreads();
  // tile_base: prefix over minibatches of m-tiles * (nN1 + nN2); total m-tiles.  The
  // counts were written by other threads of this workgroup: device-scope loads.
  int32_t carry_mt = 0;
  for (int base = 0; base < n_mb; base += 1024) {
    const int mb = base + tid;
    const int32_t c = mb < n_mb ? int32_t(__hip_atomic_load(P.mt_cnt + mb, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)) : 0;
    int32_t tot = 0;
    const int32_t incl = block_incl_scan(c, s_wave, &tot);
    if (mb < n_mb) P.tile_base[mb] = (carry_mt + incl - c) * (nN1 + nN2);
    carry_mt += tot;
  }
  if (tid == 0) {
    P.tile_base[n_mb] = carry_mt * (nN1 + nN2);
    P.hdr[kHdrMtiles] = uint32_t(carry_mt);
    P.hdr[kHdrFwdTiles] = uint32_t(carry_mt * (nN1 + nN2));
  }
}

// Each wave places its 1024-pair sub-chunk 64 pairs at a time, in ascending pair order:
// the lanes routed to one expert are found with a ballot (one round per distinct expert
// among the 64) and ranked with a prefix popcount.  The wave's next free row of every
// expert starts at the scanned base; with at most 64 local experts lane e keeps expert
// e's in a register (no LDS round trip per round), otherwise it lives in LDS.
__global__ __launch_bounds__(256) void sched_place(const int32_t* __restrict__ ids, int64_t TK,
                                                   int e0, int nl,
                                                   const int32_t* __restrict__ blk,
                                                   int32_t* __restrict__ perm,
                                                   int32_t* __restrict__ pos) {
  __shared__ int32_t base[4][kMaxLocalExperts];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t sub = int64_t(blockIdx.x) * 4 + w;
  const int64_t p0 = sub * kSchedSub;
  const bool in_regs = nl <= 64;
  int32_t base_v = 0;
  if (in_regs) {
    base_v = lane < nl ? blk[sub * (nl + 1) + lane] : 0;
  } else {
    for (int e = lane; e < nl; e += 64) base[w][e] = blk[sub * (nl + 1) + e];
  }
  constexpr int kG = kSchedSub / 64;
  int idv[kG];
#pragma unroll
  for (int u = 0; u < kG; ++u) {
    const int64_t p = p0 + 64 * u + lane;
    idv[u] = p < TK ? ids[p] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int step = 0; step < kG; ++step) {
    if (p0 + step * 64 >= TK) break;  // wave-uniform
    const int64_t p = p0 + step * 64 + lane;
    const bool valid = p < TK;
    const int id = idv[step];
    const bool local = valid && id >= e0 && id < e0 + nl;
    const int e = id - e0;
    int32_t row = -1;
    uint64_t todo = __ballot(local);
    while (todo) {
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int el = __builtin_amdgcn_readfirstlane(__shfl(e, leader));
      const uint64_t m = __ballot(local && e == el);
      const int32_t b = in_regs ? __builtin_amdgcn_readlane(base_v, el) : base[w][el];
      if (local && e == el) {
        const uint32_t below = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                         __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
        row = b + int32_t(below);
      }
      if (in_regs) {
        if (lane == el) base_v = b + __popcll(m);
      } else if (lane == leader) {
        base[w][el] = b + __popcll(m);
      }
      todo &= ~m;
    }
    if (valid) {
      pos[p] = row;
      if (row >= 0) perm[row] = int32_t(p);
    }
  }
}

mok_status_t launch_schedule(const Layout& L, const Ptrs& P, const int32_t* ids, hipStream_t st) {
  hipLaunchKernelGGL(sched_count, dim3(unsigned(L.NB)), dim3(256), 0, st, ids, L.TK, int(L.E),
                     int(L.e0), int(L.nl), P.blk);
  if (hipGetLastError() != hipSuccess) return MOK_E_LAUNCH;
  hipLaunchKernelGGL(sched_scan, dim3(1), dim3(1024), 0, st, P, L.NS, int(L.nl), int(L.M),
                     int(L.mt_max), int(L.nN1), int(L.nN2));
  if (hipGetLastError() != hipSuccess) return MOK_E_LAUNCH;
  hipLaunchKernelGGL(sched_place, dim3(unsigned(L.NB)), dim3(256), 0, st, ids, L.TK, int(L.e0),
                     int(L.nl), P.blk, P.perm, P.pos);
  if (hipGetLastError() != hipSuccess) return MOK_E_LAUNCH;
  return MOK_OK;
}

}  // namespace mok
