// Device building blocks shared by the forward and backward kernels: wave-level row
// copies and reductions, the grouped-GEMM tile runner and its epilogues.
#pragma once
#include "gemm_bf16.h"
#include "gemm_mx.h"
#include "launch.h"
#include "mx.h"

namespace mok {

// One of the two tile stages as an LDS (address space 3) pointer: selecting between the
// stage arrays as integers avoids generic-pointer selects, for which the compiler can
// emit an invalid null check of the shared aperture.
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
typedef __attribute__((address_space(3))) const uint64_t lds_cu64_t;
__device__ __forceinline__ lds_u16_t* stage16(bool second) {
  return reinterpret_cast<lds_u16_t*>(uintptr_t(second ? lds_addr(g_lds_b) : lds_addr(g_lds_a)));
}

// ------------------------------------------------------------------------------------
// wave-level data movement
// ------------------------------------------------------------------------------------
// Rows are moved by one wave each, 16 bytes per lane, with kRowBatch loads per lane in
// flight before the first store (a row of D = 7168 bf16 is 14 chunks per lane, so one
// pass): the data movers run on a few CUs, so their bandwidth is set by the bytes each
// wave keeps in flight.  Accesses go through row-length buffer resources, so the chunks
// of a pass that lie past the row's end cost an issue slot but no memory traffic.
constexpr int kRowBatch = 16;

template <bool kCoherent>
__device__ __forceinline__ void wave_copy_row(uint16_t* __restrict__ dst,
                                              const uint16_t* __restrict__ src, int D) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t bytes = uint32_t(D) * 2;
  const rsrc_t rs = row_rsrc(src, bytes), rd = row_rsrc(dst, bytes);
  for (uint32_t b0 = 0; b0 < bytes; b0 += 64 * 16 * kRowBatch) {
    v4u v[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) v[u] = buf_ld16<kCpolPlain>(rs, b0 + (lane + 64 * u) * 16);
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u)
      buf_st16<kCoherent ? kCpolDev : kCpolPlain>(rd, b0 + (lane + 64 * u) * 16, v[u]);
  }
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Highest local row of token t (-1 when it has none).  Lanes j < k read pos[t*k+j].
__device__ __forceinline__ int token_last_row(const int32_t* pos, int t, int k) {
  const int lane = threadIdx.x & 63;
  const int v = lane < k ? pos[int64_t(t) * k + lane] : -1;
  return wave_max(v);
}

__device__ __forceinline__ void wave_zero_row(uint16_t* dst, int D) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t bytes = uint32_t(D) * 2;
  const rsrc_t rd = row_rsrc(dst, bytes);
  for (uint32_t b = lane * 16; b < bytes; b += 64 * 16)
    buf_st16<kCpolPlain>(rd, b, v4u{0u, 0u, 0u, 0u});
}

// dst = sum_j g_j * rows[q0 + j] over the slots j < k with pos[q0 + j] >= 0, per element
// in ascending j (acc = 0, then acc += g_j * row_j, each step rounded to fp32), rounded
// once to bf16; g_j = gates[q0 + j], or 1 without gates.  rows holds pair-indexed rows of
// D bf16.  One wave per destination row; lane l owns the 16-byte chunks l, l + 64, ....
// With a single slot (the usual case of an even expert share) the row is processed in
// passes of kRowBatch chunks per lane; otherwise the wave loads kChunks chunks of kSlots
// slots at a time (kChunks kSlots loads per lane in flight; the forward's data movers
// take 4 slots of kCombChunks, which their registers allow beside the tile code of the
// same kernel).  Source
// loads use the cache policy kPol (device scope for rows written by other workgroups of
// a running kernel); the destination row is stored non-temporally (nothing in the layer
// reads it again); every access goes through a row-length buffer resource.
constexpr int kCombChunks = 8;

__device__ __forceinline__ void acc_gated(float (&acc)[8], v4u v, float g) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] = __fadd_rn(acc[2 * e], __fmul_rn(g, bf16_to_f32(uint16_t(w[e] & 0xFFFF))));
    acc[2 * e + 1] = __fadd_rn(acc[2 * e + 1], __fmul_rn(g, bf16_to_f32(uint16_t(w[e] >> 16))));
  }
}
__device__ __forceinline__ v4u pack_acc(const float (&acc)[8]) {
  return v4u{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
             pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
}

// The same with the slots' rows and gates already loaded: lane j < k holds my_pos =
// pos[q0 + j] and my_g = gates[q0 + j] (1 without gates); other lanes -1 and 0.  A caller
// that walks tokens loads the next token's values while this one is summed.
template <int kPol, int kSlots, int kChunks = kCombChunks>
__device__ __forceinline__ void wave_pair_sum_loaded(uint16_t* dst, const uint16_t* rows,
                                                     int64_t q0, int D, int32_t my_pos,
                                                     float my_g) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t bytes = uint32_t(D) * 2;
  const uint64_t has = __ballot(my_pos >= 0);
  const rsrc_t ry = row_rsrc(dst, bytes);
  if (__popcll(has) == 1) {
    const int j = __ffsll((unsigned long long)has) - 1;
    const float g = __shfl(my_g, j);
    const rsrc_t ro = row_rsrc(rows + (q0 + j) * D, bytes);
    for (uint32_t b0 = 0; b0 < bytes; b0 += 64 * 16 * kRowBatch) {
      v4u v[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) v[u] = buf_ld16<kPol>(ro, b0 + (lane + 64 * u) * 16);
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        acc_gated(acc, v[u], g);
        buf_st16<kCpolStream>(ry, b0 + (lane + 64 * u) * 16, pack_acc(acc));
      }
    }
    return;
  }
  for (uint32_t b0 = 0; b0 < bytes; b0 += 64 * 16 * kChunks) {
    float acc[kChunks][8];
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
    uint64_t m = has;
    while (m) {
      // the next kSlots local slots in ascending order; missing ones get a zero-length
      // range, whose loads read nothing
      int js[kSlots];
      rsrc_t rs[kSlots];
#pragma unroll
      for (int u = 0; u < kSlots; ++u) {
        js[u] = m ? __ffsll((unsigned long long)m) - 1 : -1;
        if (m) m &= m - 1;
        rs[u] = row_rsrc(rows + (q0 + (js[u] >= 0 ? js[u] : 0)) * D, js[u] >= 0 ? bytes : 0u);
      }
      v4u v[kSlots][kChunks];
#pragma unroll
      for (int c = 0; c < kChunks; ++c)
#pragma unroll
        for (int u = 0; u < kSlots; ++u) v[u][c] = buf_ld16<kPol>(rs[u], b0 + (lane + 64 * c) * 16);
#pragma unroll
      for (int u = 0; u < kSlots; ++u) {
        if (js[u] >= 0) {  // wave-uniform
          const float g = __shfl(my_g, js[u]);
#pragma unroll
          for (int c = 0; c < kChunks; ++c) acc_gated(acc[c], v[u][c], g);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      buf_st16<kCpolStream>(ry, b0 + (lane + 64 * c) * 16, pack_acc(acc[c]));
  }
}

template <int kPol, int kSlots>
__device__ __forceinline__ void wave_pair_sum(uint16_t* dst, const uint16_t* rows, int64_t q0,
                                              int D, const int32_t* pos, const float* gates,
                                              int k) {
  const int lane = threadIdx.x & 63;
  const int32_t my_pos = lane < k ? pos[q0 + lane] : -1;
  const float my_g = lane < k ? (gates ? gates[q0 + lane] : 1.0f) : 0.f;
  wave_pair_sum_loaded<kPol, kSlots>(dst, rows, q0, D, my_pos, my_g);
}

// ------------------------------------------------------------------------------------
// GEMM tiles
// ------------------------------------------------------------------------------------
// The gate/up pre-activations of a transposed GEMM1 tile (tile_gemm with TR, paired
// layout; see epi_swiglu) stored as bf16 rows [rows, 2I] at AB: gate in [0, I), up in
// [I, 2I).  Staged in LDS as rows of 256 columns (tile rows 0..127 in the A stages,
// 128..255 in the B stages; 16-byte chunk c of row r at c ^ (r % 32)), one 8-byte write
// per group of four columns, then written as whole row segments, 16 bytes a lane,
// non-temporally (the rows are read by the backward's launch).  Ends with a barrier.
template <bool kCoherent>
__device__ __forceinline__ void epi_store_ab(const TileAcc& acc, int rows, int n0, int I,
                                               uint16_t* AB) {
  constexpr int kPol = (kCoherent ? kCpolDev : kCpolPlain) | kCpolStream;
  constexpr int W = kThreads / 64;
  typedef __attribute__((address_space(3))) uint64_t lds_u64_t;
  const int tid = opaque(threadIdx.x);
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int hs = lane >> 5, l32 = lane & 31;
  const int wr = __builtin_amdgcn_readfirstlane(w);
  lds_u64_t* st = reinterpret_cast<lds_u64_t*>(stage16(wm));
  auto stage_row = [](int r) { return stage16(r >> 7); };
  auto pack4 = [](float a, float b, float c, float d) {
    return uint64_t(pack_bf16x2(a, b)) | (uint64_t(pack_bf16x2(c, d)) << 32);
  };
  {
    // rows of 256 columns: gate chunks 0..15, up chunks 16..31
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 32 * i + l32;  // row within the wave's half; rr % 32 = l32
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (n0 + 16 * (2 * wn + j) >= I) continue;  // wave-uniform: never stored
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const f32x16_t& c = acc.c[i][j];
          const int ch = 2 * (2 * wn + j) + g;
          st[rr * 64 + (ch ^ l32) * 2 + hs] = pack4(c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]);
          st[rr * 64 + ((ch + 16) ^ l32) * 2 + hs] =
              pack4(c[8 + 4 * g], c[9 + 4 * g], c[10 + 4 * g], c[11 + 4 * g]);
        }
      }
    }
    __syncthreads();
    // wave w: row pairs 2w, 2w + 1, 2w + 16, ..: lanes 0..31 write one row, 32..63 the
    // next; in each half-wave 16 lanes write the gate segment and 16 the up segment
    constexpr int kPairs = 128 / W;
    const int rs = lane >> 5, seg = (lane >> 4) & 1, l16 = lane & 15;
    const bool col16_ok = n0 + 8 * l16 < I;  // I % 16 == 0: an 8-column group is all in or out
    v4u val[kPairs];
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int r = 2 * (wr + W * k) + rs;
      const int ch = (l16 + 16 * seg) ^ (r & 31);
      val[k] = *reinterpret_cast<lds_cv4u*>(stage_row(r) + (r & 127) * 256 + 8 * ch);
    }
    const rsrc_t rab = row_rsrc(AB, uint32_t(rows) * uint32_t(2 * I) * 2u);
    const uint32_t coff = uint32_t((seg ? I : 0) + n0 + 8 * l16) * 2u;
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int r = 2 * (wr + W * k) + rs;
      if (2 * (wr + W * k) >= rows) break;  // wave-uniform; the odd row is checked below
      if (col16_ok && r < rows) buf_st16<kPol>(rab, uint32_t(r) * uint32_t(2 * I) * 2u + coff, val[k]);
    }
    __syncthreads();
  }
}

// Epilogue of GEMM1 (SwiGLU) on a transposed tile (tile_gemm with TR, paired layout).
// Lane l of MFMA block (i, j) of wave (wm, wn) holds tile row 128 wm + 32 i + l % 32;
// its values v < 8 are the gate pre-activations of intermediate columns
// n0 + 16 (2 wn + j) + 8 (v / 4) + 4 (l / 32) + v % 4 and v + 8 the up ones of the same
// columns.  So each lane forms h for two groups of four consecutive columns of its row
// with no data exchange, and stages each group as one 8-byte LDS write (lanes l and
// l + 32 fill one 16-byte chunk).  Writes H [rows, ldh] at column n0.. (when H != null)
// and, when AB != null, the gate/up pre-activations as [rows, 2I]: gate in [0, I), up in
// [I, 2I); h is formed from the fp32 accumulators.  Each output is staged as bf16 rows
// (tile rows 0..127 in the A stages, 128..255 in the B stages; 16-byte chunk c of row r
// at c ^ (r % 32) for rows of 256 columns, c ^ (r % 16) for rows of 128, so that the 32
// rows of a write and the chunks of a row read hit different banks) and then written as
// whole row segments, 16 bytes a lane.  With kCoherent the stores are device scope: in
// the fused kernel a ring slot is rewritten by workgroups on other XCDs within one
// launch.  Ends with a barrier.
template <bool kCoherent>
__device__ __forceinline__ void epi_swiglu(const TileAcc& acc, int rows, int n0, int I,
                                             uint16_t* H, int64_t ldh, uint16_t* AB) {
  constexpr int kPol = kCoherent ? kCpolDev : kCpolPlain;
  constexpr int W = kThreads / 64;
  typedef __attribute__((address_space(3))) uint64_t lds_u64_t;
  const int tid = opaque(threadIdx.x);
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int hs = lane >> 5, l32 = lane & 31;
  const int wr = __builtin_amdgcn_readfirstlane(w);
  lds_u64_t* st = reinterpret_cast<lds_u64_t*>(stage16(wm));
  auto stage_row = [](int r) { return stage16(r >> 7); };
  auto pack4 = [](float a, float b, float c, float d) {
    return uint64_t(pack_bf16x2(a, b)) | (uint64_t(pack_bf16x2(c, d)) << 32);
  };
  if (AB) epi_store_ab<kCoherent>(acc, rows, n0, I, AB);
  if (H) {
    // rows of 128 columns
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 32 * i + l32;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (n0 + 16 * (2 * wn + j) >= I) continue;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const f32x16_t& c = acc.c[i][j];
          const int ch = 2 * (2 * wn + j) + g;
          st[rr * 32 + (ch ^ (l32 & 15)) * 2 + hs] =
              pack4(silu_f(c[4 * g]) * c[8 + 4 * g], silu_f(c[4 * g + 1]) * c[9 + 4 * g],
                    silu_f(c[4 * g + 2]) * c[10 + 4 * g], silu_f(c[4 * g + 3]) * c[11 + 4 * g]);
        }
      }
    }
    __syncthreads();
    // wave w: row quads w, w + 8, ..; a 256-byte segment is 16 lanes: four rows a store
    constexpr int kQuads = 64 / W;
    const int rq = lane >> 4, l16 = lane & 15;
    const bool col16_ok = n0 + 8 * l16 < I;
    v4u val[kQuads];
#pragma unroll
    for (int k = 0; k < kQuads; ++k) {
      const int r = 4 * (wr + W * k) + rq;
      val[k] = *reinterpret_cast<lds_cv4u*>(stage_row(r) + (r & 127) * 128 + 8 * (l16 ^ (r & 15)));
    }
    const rsrc_t rh = row_rsrc(H, uint32_t(rows) * uint32_t(ldh) * 2u);
    const uint32_t coff = uint32_t(n0 + 8 * l16) * 2u;
#pragma unroll
    for (int k = 0; k < kQuads; ++k) {
      const int r = 4 * (wr + W * k) + rq;
      if (4 * (wr + W * k) >= rows) break;  // wave-uniform; later rows are checked below
      if (col16_ok && r < rows) buf_st16<kPol>(rh, uint32_t(r) * uint32_t(ldh) * 2u + coff, val[k]);
    }
    __syncthreads();
  }
}

// Epilogue of GEMM2 and of dX on a transposed tile (tile_gemm, tile_gemm_km or mx_gemm
// with TR): rows [0, rows), columns [n0, n0 + 256) of D (B tile row b is column n0 + b in
// the split layout); row r's result goes to obuf row perm_rows[r] (its pair index t*k + j;
// obuf holds obuf_rows rows of D).  Lane l of block (i, j) holds row 128 wm + 32 i + l % 32
// at columns brow_of(j, wn) + 8 (v / 4) + 4 (l / 32) + v % 4, so each group of four
// columns is staged in LDS with one 8-byte write, lanes l and l + 32 filling one 16-byte
// chunk (tile rows 0..127 in the A stages, 128..255 in the B stages, free once the K loop
// has ended; chunk c of row r at c ^ (r % 32), so the 32 rows of a write and the chunks
// of a row read hit different banks).  Each wave then writes whole 512-byte row segments,
// 16 bytes a lane when every byte offset of obuf fits in 32 bits (two rows a store
// through one resource), else 8 bytes a lane through a resource per row.  With kCoherent
// the row stores are device scope; with kStream non-temporal (GEMM2 results, read once by
// the combine).  Ends with a barrier.
template <bool kCoherent, bool kStream>
__device__ __forceinline__ void epi_scatter(const TileAcc& acc, int rows, int n0, int D,
                                            const int32_t* perm_rows, uint16_t* obuf,
                                            int64_t obuf_rows) {
  const int tid = opaque(threadIdx.x);
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wn = w & 3;
  {
    typedef __attribute__((address_space(3))) uint64_t lds_u64_t;
    lds_u64_t* st = reinterpret_cast<lds_u64_t*>(stage16(w >> 2));
    const int l32 = lane & 31, hs = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 32 * i + l32;  // row within the wave's half; rr % 32 = l32
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& c = acc.c[i][j];
          const int ch = 8 * wn + 4 * j + g;
          st[rr * 64 + (ch ^ l32) * 2 + hs] =
              uint64_t(pack_bf16x2(c[4 * g], c[4 * g + 1])) |
              (uint64_t(pack_bf16x2(c[4 * g + 2], c[4 * g + 3])) << 32);
        }
    }
  }
  __syncthreads();
  // wave w writes tile rows w, w + 8, ..: their destinations are loaded one per lane
  // and all 32 staged rows are read before the first store, so that no load waits
  // behind a store (vector memory operations complete in order)
  constexpr int kPol = (kCoherent ? kCpolDev : kCpolPlain) | (kStream ? kCpolStream : 0);
  constexpr int kRowsPerWave = 256 / (kThreads / 64);
  const int wr = __builtin_amdgcn_readfirstlane(w);
  const int my_r = wr + (kThreads / 64) * (lane % kRowsPerWave);
  const int my_dst = my_r < rows ? perm_rows[my_r] : 0;
  if (obuf_rows * int64_t(D) * 2 < (int64_t(1) << 32)) {
    // two rows a store, 16 bytes a lane (each half-wave one 512-byte row segment), with
    // one resource for the whole buffer: every offset fits in 32 bits
    const int h = lane >> 5, l32 = lane & 31;
    v4u val[kRowsPerWave / 2];
#pragma unroll
    for (int k = 0; k < kRowsPerWave / 2; ++k) {
      const int r = wr + (kThreads / 64) * (2 * k + h);
      val[k] = *reinterpret_cast<__attribute__((address_space(3))) const v4u*>(
          stage16(r >> 7) + (r & 127) * 256 + 8 * (l32 ^ (r & 31)));
    }
    const rsrc_t rb = row_rsrc(obuf, uint32_t(obuf_rows * int64_t(D) * 2));
#pragma unroll
    for (int k = 0; k < kRowsPerWave / 2; ++k) {
      const int r = wr + (kThreads / 64) * (2 * k + h);
      if (wr + (kThreads / 64) * 2 * k >= rows) break;  // wave-uniform; row r checked below
      const int d0 = __builtin_amdgcn_readlane(my_dst, 2 * k);
      const int d1 = __builtin_amdgcn_readlane(my_dst, 2 * k + 1);
      const int dst = h ? d1 : d0;
      if (r < rows && n0 + 8 * l32 < D)
        buf_st16<kPol>(rb, (uint32_t(dst) * uint32_t(D) + uint32_t(n0 + 8 * l32)) * 2u, val[k]);
    }
    __syncthreads();
    return;
  }
  uint64_t val[kRowsPerWave];
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int r = wr + (kThreads / 64) * k;
    val[k] = *reinterpret_cast<lds_cu64_t*>(stage16(r >> 7) + (r & 127) * 256 +
                                            8 * ((lane >> 1) ^ (r & 31)) + 4 * (lane & 1));
  }
  const uint32_t row_bytes = uint32_t(D) * 2u;
  const uint32_t off = uint32_t(n0 + 4 * lane) * 2u;  // columns past D are dropped
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int r = wr + (kThreads / 64) * k;
    if (r >= rows) break;  // wave-uniform
    const int dst = __builtin_amdgcn_readlane(my_dst, k);
    buf_st8<kPol>(row_rsrc(obuf + int64_t(dst) * D, row_bytes), off, val[k]);
  }
  __syncthreads();
}

// Epilogue of the MXFP8 GEMM1 on a transposed tile (mx_gemm with TR, paired layout; the
// lanes' values as in epi_swiglu): SwiGLU, then H MX-quantised along I.  A 32-column MX
// block [n0 + 32 wn, +32) of tile row r is MFMA blocks j = 0, 1 of wave column wn: lane l
// holds 16 of its h values (columns 16 j + 8 g + 4 (l / 32) + 0..3 of the block) and lane
// l ^ 32 the other 16, so the block maximum is the lane's own maximum and one exchange.
// The codes are staged in LDS (row r at byte r * 128; its 4-byte chunk c at
// c ^ 2 ((r / 2) % 16), so the 32 rows of a write hit different banks; scales after
// them), then written as 128-byte row segments, 4 bytes a lane, and one byte per row and
// block.  Writes codes Hc[row * ldh + col] and scales Hs[row * hs_ld + col / 32]; I is a
// multiple of 32, so a block is wholly inside or outside [0, I).  With AB, the gate/up
// pre-activations are stored first, as bf16 rows (epi_store_ab).  Ends with a barrier.
template <bool kCoherent>
__device__ __forceinline__ void epi_swiglu_mx(const TileAcc& acc, int rows, int n0, int I,
                                                uint8_t* Hc, int64_t ldh, uint8_t* Hs,
                                                int64_t hs_ld, uint16_t* AB = nullptr) {
  if (AB) epi_store_ab<kCoherent>(acc, rows, n0, I, AB);  // bf16 a, b for the backward
  constexpr int kPol = kCoherent ? kCpolDev : kCpolPlain;
  constexpr int W = kThreads / 64;
  typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
  typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
  const int tid = opaque(threadIdx.x);
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int hs = lane >> 5, l32 = lane & 31;
  lds_u32_t* sc = reinterpret_cast<lds_u32_t*>(uintptr_t(lds_addr(g_lds_a)));  // [256][32]
  lds_u8_t* ss = reinterpret_cast<lds_u8_t*>(uintptr_t(lds_addr(g_lds_a))) + 256 * 128;  // [256][4]
  auto swz = [](int r) { return 2 * ((r >> 1) & 15); };
  if (n0 + 32 * wn < I) {  // wave-uniform
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 128 * wm + 32 * i + l32;
      float h[2][8];
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          h[j][v] = silu_f(acc.c[i][j][v]) * acc.c[i][j][v + 8];
          m = fmaxf(m, fabsf(h[j][v]));
        }
      m = fmaxf(m, __shfl_xor(m, 32));
      const int n = mx_shared_exp(m);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const uint32_t code =
              e4m3x2(ldexpf(h[j][4 * g], -n), ldexpf(h[j][4 * g + 1], -n)) |
              (e4m3x2(ldexpf(h[j][4 * g + 2], -n), ldexpf(h[j][4 * g + 3], -n)) << 16);
          sc[r * 32 + ((8 * wn + 4 * j + 2 * g + hs) ^ swz(r))] = code;
        }
      if (hs == 0) ss[r * 4 + wn] = uint8_t(n + 127);
      __builtin_amdgcn_sched_barrier(0);  // one block row at a time: few live registers
    }
  }
  __syncthreads();
  // wave w: row pairs w, w + 8, ..; lanes 0..31 write row 2p, lanes 32..63 row 2p + 1
  // (one resource for the tile's rows: a buffer resource's base is wave-uniform, and the
  // two half-waves write different rows)
  const bool col_ok = n0 + 4 * l32 < I;  // I % 32 == 0: a 4-column group is all in or out
  const rsrc_t rh = row_rsrc(Hc, uint32_t(rows) * uint32_t(ldh));
  const int wr = __builtin_amdgcn_readfirstlane(w);
#pragma unroll 4
  for (int k = 0; k < 128 / W; ++k) {
    const int r = 2 * (wr + W * k) + hs;
    if (2 * (wr + W * k) >= rows) break;  // wave-uniform; the odd row is checked below
    if (r < rows && col_ok)
      buf_st4<kPol>(rh, uint32_t(r) * uint32_t(ldh) + uint32_t(n0 + 4 * l32),
                    sc[r * 32 + (l32 ^ swz(r))]);
  }
  if (tid < rows) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (n0 + 32 * b >= I) break;
      uint8_t* sp = Hs + int64_t(tid) * hs_ld + ((n0 + 32 * b) >> 5);
      if (kCoherent) st_dev_u8(sp, ss[tid * 4 + b]);
      else *sp = ss[tid * 4 + b];
    }
  }
  __syncthreads();
}

// MXFP8 operands of one tile of either GEMM:
//   GEMM1: A = dispatched X codes [rows, D] (scales xs_ld bytes per row), B = W_gate /
//          W_up codes, rows n0.., K = D;
//   GEMM2: A = H codes [rows, I] (scales hs_ld per row), B = W_down codes rows
//          n0..n0+255, K = I.
struct MxOperands {
  const uint8_t* A;
  const uint8_t* As;
  int64_t as_ld;
  const uint8_t* w0;
  const uint8_t* w0s;
  const uint8_t* w1;
  const uint8_t* w1s;
  int64_t ws_ld;
};

// Both GEMMs' tiles come out transposed (epi_swiglu_mx, epi_scatter).
template <bool kCoherent>
__device__ __forceinline__ void run_tile_mx(bool gemm1, const MxOperands& o, int rows, int n0,
                                            int D, int I, TileAcc& acc) {
  MxSrc src;
  if (gemm1)
    mx_src_init(src, geom::kPaired, o.A, o.As, D, o.as_ld, rows, o.w0, o.w0s, o.w1, o.w1s, D,
                o.ws_ld, n0, n0, I, D);
  else
    mx_src_init(src, geom::kSplit, o.A, o.As, I, o.as_ld, rows, o.w0, o.w0s, o.w0, o.w0s, I,
                o.ws_ld, n0, n0 + 128, D, I);
  mx_gemm<kCoherent, true>(src, gemm1 ? D : I, acc);
}

// Operands of one tile of either GEMM (one K loop serves both).
//   GEMM1: A = dispatched rows [rows, D], B = W_gate/W_up rows n0.., K = D.
//   GEMM2: A = hidden rows [rows, I], B = W_down rows n0..n0+255, K = I.
// Both GEMMs' tiles come out transposed (epi_swiglu, epi_scatter).
template <bool kCoherent>
__device__ __forceinline__ void run_tile(bool gemm1, const uint16_t* A, int rows,
                                         const uint16_t* w0, const uint16_t* w1, int n0, int D,
                                         int I, TileAcc& acc) {
  TileSrc src;
  if (gemm1) {
    tile_src_init(src, geom::kPaired, A, D, rows, w0, w1, D, n0, n0, I);
    tile_gemm<kCoherent, true>(src, D, acc);
  } else {
    tile_src_init(src, geom::kSplit, A, I, rows, w0, w0, I, n0, n0 + 128, D);
    tile_gemm<kCoherent, true>(src, I, acc);
  }
}

// Epilogue of the dH GEMM of the backward (SwiGLU backward and router-weight gradient
// fused).  The tile covered routed rows row0 + [0, rows) and intermediate columns
// n0 + [0, 256) of u = dY W_down.  Per element, with a, b the saved gate/up
// pre-activations, g the row's gate weight, s = sigmoid(a):
//   h = a s b;  dh = g u;  da = dh b s (1 + a (1 - s));  db = dh a s.
// a, b of tile row r are ab_tile[r * 2I + col] and ab_tile[r * 2I + I + col] (the tile's
// rows in the ring slot or in the row buffer).  Writes da, db row-major into bdab
// [R, 2I], g h row-major into gh [R, I] (the dW_down operand: the gate weight is folded
// into h there), and the partial sum of u h over this tile's columns for each row into
// dgpart[row][nt] (lanes first, then the four column waves in order: a fixed summation
// order).  Loads and stores go through buffer resources sized to the tile's rows, so
// rows past the tile read zero and their stores are dropped.  kStPol is the cache policy
// of the da, db, g h and dG-partial stores (kCpolDev when the same launch reads them on
// other XCDs).
template <int kStPol>
__device__ __forceinline__ void epi_dh(const TileAcc& acc, int rows, int row0, int n0, int I,
                                       const uint16_t* ab_tile, const float* gates,
                                       const int32_t* perm, uint16_t* bdab, uint16_t* gh,
                                       float* dgpart, int nt, int nNdh) {
  const int tid = opaque(threadIdx.x);
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wn = w & 3;
  float* red = reinterpret_cast<float*>(g_lds_a);  // [4][256] row partials per column wave
  float* gate_of = red + 4 * 256;                  // [256] gate weight of each tile row
  const int64_t twoI = 2 * int64_t(I);
  if (tid < 256) gate_of[tid] = tid < rows ? gates[perm[row0 + tid]] : 0.f;
  const rsrc_t ab_res = row_rsrc(ab_tile, uint32_t(rows) * uint32_t(twoI) * 2u);
  const rsrc_t dab_res = row_rsrc(bdab + int64_t(row0) * twoI, uint32_t(rows) * uint32_t(twoI) * 2u);
  const rsrc_t gh_res = row_rsrc(gh + int64_t(row0) * I, uint32_t(rows) * uint32_t(I) * 2u);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float s[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t) s[q][t] = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int cb = n0 + wn * 64 + j * 32;  // I % 64 == 0: the block is all in or all out
      if (cb >= I) continue;
      const int col = cb + (lane & 31);
      // a and b of the lane's 16 rows (acc_row(i, 4q + t) = acc_row(i, 0) + 8q + t), all
      // loads issued before the first use
      const uint32_t row_i = uint32_t(acc_row(tid, i, 0));
      const uint32_t voff = (row_i * uint32_t(twoI) + col) * 2u;
      const uint32_t goff = (row_i * uint32_t(I) + col) * 2u;
      uint16_t av[16], bv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t so = uint32_t(8 * (v >> 2) + (v & 3)) * uint32_t(twoI) * 2u;
        av[v] = __builtin_amdgcn_raw_buffer_load_b16(ab_res, voff, so, 0);
        bv[v] = __builtin_amdgcn_raw_buffer_load_b16(ab_res, voff, so + uint32_t(I) * 2u, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int rr = acc_row(tid, i, 4 * q + t);  // four consecutive rows
          const bool ok = rr < rows;
          const float g = gate_of[rr];
          const float u = acc.c[i][j][4 * q + t];
          const float a = bf16_to_f32(av[4 * q + t]);
          const float b = bf16_to_f32(bv[4 * q + t]);
          const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
          const float sl = a * sg;
          const float h = sl * b;
          s[q][t] += ok ? u * h : 0.f;
          const float dh = g * u;
          const float da = dh * b * sg * (1.0f + a * (1.0f - sg));
          const float db = dh * sl;
          const uint32_t r8 = uint32_t(8 * q + t);
          const uint32_t so = r8 * uint32_t(twoI) * 2u;
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(da), dab_res, voff, so, kStPol);
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(db), dab_res, voff,
                                                so + uint32_t(I) * 2u, kStPol);
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(g * h), gh_res, goff,
                                                r8 * uint32_t(I) * 2u, kStPol);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // sum over the 32 lanes of the half-wave: a DPP butterfly inside each 16-lane row
        // (every lane ends with the same bits: each step adds a lane's value to its
        // partner's, and addition commutes), then the two rows through one permlane swap
        float v = row16_sum(s[q][t]);
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                         false, false);
        v += __uint_as_float((lane & 16) ? sw[0] : sw[1]);
        const int rr = acc_row(tid, i, 4 * q + t);
        if ((lane & 31) == 0 && rr < rows) red[wn * 256 + rr] = v;
      }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  for (int r = tid; r < rows; r += kThreads) {
    const float v = ((red[r] + red[256 + r]) + red[512 + r]) + red[768 + r];
    float* d = dgpart + int64_t(row0 + r) * nNdh + nt;
    if (kStPol == kCpolDev)
      __hip_atomic_store(reinterpret_cast<uint32_t*>(d), __float_as_uint(v), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else
      *d = v;
  }
  __syncthreads();
}

// Epilogue storing the fp32 tile: rows [0, rows) at C + row * ldc, columns n0 + b for
// B tile row b (split layout) below N.  Untransposed (lane l of block (i, j) holds column
// brow_of(j, wn) + l % 32 at rows acc_row), each store writes 128-byte row segments;
// transposed (TR: lane l holds row 128 wm + 32 i + l % 32 at columns brow_of(j, wn) +
// 8 (v / 4) + 4 (l / 32) + v % 4), four consecutive columns (16 bytes) a store, N and ldc
// multiples of 4.
template <bool TR>
__device__ __forceinline__ void epi_store_f32(const TileAcc& acc, int rows, int n0, int N,
                                              float* C, int64_t ldc) {
  const int tid = opaque(threadIdx.x);
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x16_t& c = acc.c[i][j];
      if (TR) {
        const int row = 128 * wm + 32 * i + (lane & 31);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + brow_of(j, wn) + 8 * g + 4 * (lane >> 5);
          if (row < rows && col < N)
            *reinterpret_cast<float4*>(C + int64_t(row) * ldc + col) =
                make_float4(c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]);
        }
      } else {
        const int col = n0 + brow_of(j, wn) + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = acc_row(tid, i, v);
          if (row < rows && col < N) C[int64_t(row) * ldc + col] = c[v];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace mok
