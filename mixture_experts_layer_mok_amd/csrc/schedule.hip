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
//   scan   — one workgroup turns the per-sub-chunk counts into absolute bases
//            (expert-major, sub-chunk-minor), the offsets, R, the minibatch count and
//            the m-tile table;
//   place  — each wave walks its sub-chunk 64 pairs at a time; lanes routed to the
//            same expert are grouped with a ballot and ranked with a prefix popcount,
//            which keeps ascending (token, slot) order inside every expert.
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
  int bad = 0;
  for (int i = lane; i < kSchedSub; i += 64) {
    const int64_t p = p0 + i;
    if (p >= TK) break;
    const int id = ids[p];
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

// One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void sched_scan(Ptrs P, int64_t NS, int nl, int M, int mt_max,
                                                   int nN1, int nN2) {
  __shared__ int32_t s_cnt[kMaxLocalExperts + 1];
  __shared__ int32_t s_off[kMaxLocalExperts + 1];
  __shared__ int32_t s_bad;
  __shared__ int32_t s_part[1024];
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  // per expert: running sum over sub-chunks (relative bases), total count
  for (int e = tid; e < nl; e += 1024) {
    int32_t run = 0;
    for (int64_t s = 0; s < NS; ++s) {
      const int32_t c = P.blk[s * (nl + 1) + e];
      P.blk[s * (nl + 1) + e] = run;
      run += c;
    }
    s_cnt[e] = run;
  }
  {
    int32_t b = 0;
    for (int64_t s = tid; s < NS; s += 1024) b += P.blk[s * (nl + 1) + nl];
    if (b) atomicAdd(&s_bad, b);
  }
  __syncthreads();
  // exclusive scan of counts -> offsets (nl <= 1024: one element per thread)
  {
    int32_t v = tid < nl ? s_cnt[tid] : 0;
    s_part[tid] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      int32_t add = tid >= d ? s_part[tid - d] : 0;
      __syncthreads();
      s_part[tid] += add;
      __syncthreads();
    }
    if (tid < nl) s_off[tid] = s_part[tid] - v;
    if (tid == 0) s_off[nl] = s_part[1023];
  }
  __syncthreads();
  const int32_t R = s_off[nl];
  const int32_t n_mb = (R + M - 1) / M;
  for (int e = tid; e < nl; e += 1024) {
    P.counts[e] = s_cnt[e];
    P.offsets[e] = s_off[e];
  }
  if (tid == 0) {
    P.offsets[nl] = R;
    P.hdr[kHdrStatus] = s_bad ? MOK_DEV_BAD_ID : 0u;
    P.hdr[kHdrR] = uint32_t(R);
    P.hdr[kHdrNmb] = uint32_t(n_mb);
  }
  // absolute bases per (sub-chunk, expert)
  for (int64_t idx = tid; idx < NS * nl; idx += 1024) {
    const int64_t s = idx / nl;
    const int e = int(idx % nl);
    P.blk[s * (nl + 1) + e] += s_off[e];
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
  __syncthreads();
  __threadfence_block();
  // tile_base: prefix over minibatches of m-tiles * (nN1 + nN2); total m-tiles
  {
    int32_t carry = 0, carry_mt = 0;
    for (int base = 0; base < n_mb; base += 1024) {
      const int mb = base + tid;
      const int32_t c = mb < n_mb ? P.mt_cnt[mb] : 0;
      s_part[tid] = c;
      __syncthreads();
      for (int d = 1; d < 1024; d <<= 1) {
        int32_t add = tid >= d ? s_part[tid - d] : 0;
        __syncthreads();
        s_part[tid] += add;
        __syncthreads();
      }
      if (mb < n_mb) P.tile_base[mb] = (carry_mt + s_part[tid] - c) * (nN1 + nN2);
      const int32_t tot = s_part[1023];
      __syncthreads();
      carry_mt += tot;
      (void)carry;
    }
    if (tid == 0) {
      P.tile_base[n_mb] = carry_mt * (nN1 + nN2);
      P.hdr[kHdrMtiles] = uint32_t(carry_mt);
      P.hdr[kHdrFwdTiles] = uint32_t(carry_mt * (nN1 + nN2));
    }
  }
}

__global__ __launch_bounds__(256) void sched_place(const int32_t* __restrict__ ids, int64_t TK,
                                                   int e0, int nl,
                                                   const int32_t* __restrict__ blk,
                                                   int32_t* __restrict__ perm,
                                                   int32_t* __restrict__ pos) {
  __shared__ int32_t base[4][kMaxLocalExperts];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t sub = int64_t(blockIdx.x) * 4 + w;
  for (int e = lane; e < nl; e += 64) base[w][e] = blk[sub * (nl + 1) + e];
  __syncthreads();
  const int64_t p0 = sub * kSchedSub;
  for (int step = 0; step < kSchedSub / 64; ++step) {
    const int64_t p = p0 + step * 64 + lane;
    if (p0 + step * 64 >= TK) break;  // wave-uniform
    const bool valid = p < TK;
    const int id = valid ? ids[p] : -1;
    const bool local = valid && id >= e0 && id < e0 + nl;
    const int e = id - e0;
    int32_t row = -1;
    uint64_t todo = __ballot(local);
    while (todo) {
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int el = __shfl(e, leader);
      const uint64_t m = __ballot(local && e == el);
      const int32_t b = base[w][el];
      if (local && e == el) {
        const uint32_t below = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                         __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
        row = b + int32_t(below);
      }
      if (lane == leader) base[w][el] = b + __popcll(m);
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
