// MXFP8 grouped-GEMM tile for gfx950: the bf16 tile's structure (256 x 256 per
// workgroup, 8 waves of 128 x 64 each, two-stage direct-to-LDS ring of whole 128-byte
// row segments) over e4m3 codes.  One K step is 128 elements = 128 code bytes per row
// plus one dword of four e8m0 scales per row (one per 32-element block); a step is two
// 64-deep slices of v_mfma_scale_f32_32x32x64_f8f6f4, which applies the A-row and B-row
// block scales inside the MFMA.
//
// Scaled MFMA operands (32 x 32 x 64, 8-bit elements), as measured on gfx950: lane l
// holds row (column) l % 32; its bytes 0..15 are K 16 (l / 32) .. +16 of the slice and
// its bytes 16..31 are K 32 + 16 (l / 32) .. +16, so K block 0 of the slice (32 values)
// is the first half of both lane groups and block 1 the second half.  The scale of
// block b of row r comes from lane r + 32 b, as the byte of a 32-bit register selected
// by op_sel.  A lane reads the step's scale dword of each of its rows once (blocks
// 0..3 of the 128-wide step), shifts it right by 8 (l / 32), and slice s then uses
// byte 2 s: block 2 s + l / 32.
//
// The scale dwords of a step are staged in LDS beside the data stages: each lane of
// waves 0-3 loads the dword of one A row and each lane of waves 4-7 that of one B row
// (global_load_lds_dword: per-lane addresses, since in the paired layout a B row's
// matrix depends on the lane).  Scale rows are padded to a multiple of 4 bytes by the
// producers of the A scales; weight scales are used as given when K % 128 == 0 and
// repacked otherwise.
//
// K need only be a multiple of 64: when K % 128 == 64 the last step is a half step
// that loads chunks 0..3 of each row and runs slice 0 only (slice 1 reads whatever the
// stage held and is not multiplied).
#pragma once
#include "gemm_bf16.h"

namespace mok {

static __shared__ uint32_t g_lds_sa[2 * 256];  // A scale dwords, two stages
static __shared__ uint32_t g_lds_sb[2 * 256];  // B scale dwords, two stages

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Direct-to-LDS load of one dword per lane from a per-lane address: lane l's dword
// lands at lds_wave_base + 4 l.  COH adds sc1 (device scope).
template <bool COH>
__device__ __forceinline__ void dma4(const void* src, const uint32_t* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  if (COH)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off sc1" ::"v"(src), "s"(m0)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0)
                 : "memory", "m0");
}

// Buffer resource whose range ends 2^31 bytes after base: every offset the MX tile forms
// stays below that (a tile spans at most 256 rows of at most 65536 bytes; a weight matrix
// holds fewer than 2^31 codes, checked on the host), so setting bit 31 of a lane's
// offset turns its load into an out-of-range load, which reads no memory.
__device__ __forceinline__ i32x4_t make_rsrc_2g(const void* base) {
  i32x4_t r = make_rsrc(base);
  r.z = int(0x80000000u);
  return r;
}
constexpr uint32_t kOffOutOfRange = 0x80000000u;

struct MxSrc {
  TileSrc data;          // code rows, as rows of ld / 2 two-byte units
  const uint8_t* scale;  // this lane's scale row (A for waves 0-3, B for waves 4-7)
  int half_last;         // K % 128 == 64: the last step is a half step
};

// A = codes [rows, K] (lda bytes per row) with scales As (as_ld bytes per row);
// B0 / B1 = weight codes [N, K] (ldb bytes per row) with scales B0s / B1s (bs_ld bytes
// per row); B layout as for the bf16 tile.
__device__ __forceinline__ void mx_src_init(MxSrc& s, int layout, const uint8_t* A,
                                            const uint8_t* As, int64_t lda, int64_t as_ld,
                                            int rows_valid, const uint8_t* B0,
                                            const uint8_t* B0s, const uint8_t* B1,
                                            const uint8_t* B1s, int64_t ldb, int64_t bs_ld,
                                            int nb0, int nb1, int N, int K) {
  tile_src_init(s.data, layout, reinterpret_cast<const uint16_t*>(A), lda / 2, rows_valid,
                reinterpret_cast<const uint16_t*>(B0), reinterpret_cast<const uint16_t*>(B1),
                ldb / 2, nb0, nb1, N);
  s.data.ra = make_rsrc_2g(A);
  s.data.rb0 = make_rsrc_2g(B0);
  s.data.rb1 = make_rsrc_2g(B1);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (w < 4) {
    s.scale = As + geom::mx_a_scale_offset(w, l, rows_valid, as_ld);
  } else {
    const int m = geom::b_matrix_of_row(layout, geom::mx_scale_row(w, l));
    s.scale = (m ? B1s : B0s) + geom::mx_b_scale_offset(layout, w, l, nb0, nb1, N, bs_ld);
  }
  s.half_last = (K & 127) != 0;
}

// As mx_src_init with the A rows gathered: tile row r (clamped to rows_valid - 1) is row
// rowmap[r] / k of the code matrix A [*, lda] and of its scales As [*, as_ld] (A holds
// fewer than 2^31 bytes, checked on the host).
__device__ __forceinline__ void mx_src_init_gather(MxSrc& s, int layout, const uint8_t* A,
                                                   const uint8_t* As, int64_t lda, int64_t as_ld,
                                                   const int32_t* rowmap, int k, int rows_valid,
                                                   const uint8_t* B0, const uint8_t* B0s,
                                                   const uint8_t* B1, const uint8_t* B1s,
                                                   int64_t ldb, int64_t bs_ld, int nb0, int nb1,
                                                   int N, int K) {
  mx_src_init(s, layout, A, As, lda, as_ld, rows_valid, B0, B0s, B1, B1s, ldb, bs_ld, nb0, nb1,
              N, K);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int p = 0; p < geom::kLoads; ++p) {
    int r = geom::dma_row(p, w, l);
    if (r > rows_valid - 1) r = rows_valid - 1;
    s.data.oa[p] = uint32_t(int64_t(rowmap[r] / k) * lda + geom::dma_chunk(w, l) * 16);
  }
  if (w < 4) {
    int r = geom::mx_scale_row(w, l);
    if (r > rows_valid - 1) r = rows_valid - 1;
    s.scale = As + int64_t(rowmap[r] / k) * as_ld;
  }
}

// Loads of step ks into stage STAGE: 4 A + 4 B data loads and one scale load per lane,
// with no branches (a branch here lets the compiler move the MFMAs around it).
//   valid = false: the step does not exist; the data loads are made out of range (no
//     memory is read) and the scale load repeats the last step's dword (always in
//     bounds).  The stage is not read afterwards.
//   half: the lanes whose chunk lies in the upper half of the 128-byte segment load the
//     chunk 64 bytes lower instead (same row, in bounds); their LDS slots belong to
//     slice 1, which a half step multiplies with zero scales.
template <bool COH, int STAGE>
__device__ __forceinline__ void mx_issue_part(const MxSrc& s, int ks, int nk, bool valid, bool half,
                                              int q) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const uint32_t kb = uint32_t(ks) * 128;
  const TileSrc& d = s.data;
  const uint32_t adj = valid ? ((half && !geom::mx_chunk_in_half(w, l)) ? 0u - 64u : 0u)
                             : kOffOutOfRange;
  if (q < geom::kLoads) {
    dma16<COH>(d.ra, d.oa[q] + adj, kb, stage_a<STAGE>() + (q * 8 + w) * 64);
  } else if (q < 2 * geom::kLoads) {
    const int p = q - geom::kLoads;
    const bool paired_up = d.layout == geom::kPaired && ((w >> 1) & 1);
    const bool use_b1 = d.layout == geom::kPaired ? paired_up : (p >= 2);
    dma16<false>(use_b1 ? d.rb1 : d.rb0, d.ob[p] + adj, kb, stage_b<STAGE>() + (p * 8 + w) * 64);
  } else {
    // one instruction for every wave: the LDS destination is a wave-uniform select
    const uint32_t* sdst = (w < 4 ? g_lds_sa : g_lds_sb) + STAGE * 256 + (w & 3) * 64;
    dma4<COH>(s.scale + (valid ? ks : nk - 1) * 4, sdst);
  }
}

template <bool COH, int STAGE>
__device__ __forceinline__ void mx_issue(const MxSrc& s, int ks, int nk, bool valid, bool half) {
#pragma unroll
  for (int q = 0; q <= 2 * geom::kLoads; ++q) mx_issue_part<COH, STAGE>(s, ks, nk, valid, half, q);
}

struct MxScales {
  uint32_t a[4], b[2];
};

// Per-lane LDS byte addresses of the A fragment reads: for slice sl and half h (first /
// second 16 bytes of the lane's 32), logical chunk 4 sl + 2 h + l / 32 (block 2 sl + h,
// the lane group's 16 values of it), swizzled by the row; index 2 sl + h.  A lane's B rows have the same row-in-block r32, hence the same
// swizzle, so its B addresses are the A addresses plus a wave-uniform distance.
struct MxFragAddr {
  uint32_t a[4];
  uint32_t b_minus_a;  // wave-uniform
};

__device__ __forceinline__ void mx_frag_addr_init(MxFragAddr& fa) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int r32 = lane & 31;
  const int sw = lds_swz(r32);
  const uint32_t a0 = lds_addr(g_lds_a) + uint32_t(wm * 128 + r32) * 128;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = 4 * (q >> 1) + 2 * (q & 1) + (lane >> 5);
    fa.a[q] = a0 + uint32_t((c ^ sw) * 16);
  }
  fa.b_minus_a = __builtin_amdgcn_readfirstlane(
      lds_addr(g_lds_b) + uint32_t(wn * 64) * 128 - lds_addr(g_lds_a) - uint32_t(wm * 128) * 128);
}

__device__ __forceinline__ i32x8_t lds_read32(uint32_t lo_addr, uint32_t hi_addr) {
  const v4u lo = *reinterpret_cast<lds_cv4u*>(uintptr_t(lo_addr));
  const v4u hi = *reinterpret_cast<lds_cv4u*>(uintptr_t(hi_addr));
  return i32x8_t{int(lo.x), int(lo.y), int(lo.z), int(lo.w),
                 int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
}

// A fragment of MFMA row block i, slice sl, stage S.
template <int S>
__device__ __forceinline__ i32x8_t mx_read_a(const MxFragAddr& fa, int sl, int i) {
  const uint32_t o = S * kStageBytes + i * 32 * 128;
  return lds_read32(fa.a[2 * sl] + o, fa.a[2 * sl + 1] + o);
}
template <int S>
__device__ __forceinline__ i32x8_t mx_read_b(const MxFragAddr& fa, int sl, int j) {
  const uint32_t o = S * kStageBytes + j * 32 * 128;
  return lds_read32(fa.a[2 * sl] + fa.b_minus_a + o, fa.a[2 * sl + 1] + fa.b_minus_a + o);
}

// Scale dwords of the lane's rows for the step in stage S, shifted to the lane group.
template <int S>
__device__ __forceinline__ void mx_scales_read(MxScales& sc) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int r32 = lane & 31;
  const int sh = 8 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) sc.a[i] = g_lds_sa[S * 256 + wm * 128 + i * 32 + r32] >> sh;
#pragma unroll
  for (int j = 0; j < 2; ++j) sc.b[j] = g_lds_sb[S * 256 + wn * 64 + j * 32 + r32] >> sh;
}

// With TR the B fragment (and its scales) takes the MFMA's A slot: the block holds C^T,
// as for the bf16 tile (mma_blk).
template <int SL, bool TR>
__device__ __forceinline__ void mx_mma_row(const i32x8_t& a, const i32x8_t (&b)[2], uint32_t sa,
                                           const MxScales& sc, f32x16_t (&c)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
    c[j] = TR ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a, c[j], 0, 0, 2 * SL,
                                                                 int(sc.b[j]), 2 * SL, int(sa))
              : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[j], c[j], 0, 0, 2 * SL,
                                                                 int(sa), 2 * SL, int(sc.b[j]));
}

// s_waitcnt vmcnt(0) lgkmcnt(0): every load of this wave, global and LDS, has landed.
__device__ __forceinline__ void wait_all_loads() {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0 << 8) | (0 << 14));
}

// One K step ks held in stage S (S = ks % 2).  On entry a[] and b[] hold slice 0 of the
// step and sc its scales; on exit they hold slice 0 of step ks + 1 and its scales (stale
// when ks is the last step; never used then).  A fragments rotate: as soon as the two
// MFMAs of row block i have issued, a[i] is refilled with the next slice's block i, so
// only the B fragments are double-buffered; the scales are replaced after the last MFMA
// that reads them.  The body has no branches, so the compiler keeps its order.
template <bool COH, int S, bool TR>
__device__ __forceinline__ void mx_step(const MxSrc& src, const MxFragAddr& fa, int ks, int nk,
                                        i32x8_t (&a)[4], i32x8_t (&b)[2], MxScales& sc,
                                        TileAcc& acc) {
  constexpr int SN = S ^ 1;
  i32x8_t bn[2];
  // slice 0, refilling with slice 1 of this stage
  bn[0] = mx_read_b<S>(fa, 1, 0);
  bn[1] = mx_read_b<S>(fa, 1, 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    mx_mma_row<0, TR>(a[i], b, sc.a[i], sc, acc.c[i]);
    __builtin_amdgcn_sched_barrier(0);
    a[i] = mx_read_a<S>(fa, 1, i);
  }
  b[0] = bn[0];
  b[1] = bn[1];
  __builtin_amdgcn_sched_barrier(0);
  // step ks+1 (the only loads in flight) must have landed: mine by the wait, everyone's
  // by the barrier, which also tells that every wave has finished reading stage S.
  wait_all_loads();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // the loads of step ks + 2: the scales now, the data two per MFMA row of slice 1 (a
  // burst of them fills the vector-memory queue and holds up the MFMAs behind it)
  const bool nvalid = ks + 2 < nk, nhalf = src.half_last && ks + 2 == nk - 1;
  mx_issue_part<COH, S>(src, ks + 2, nk, nvalid, nhalf, 2 * geom::kLoads);
  bn[0] = mx_read_b<SN>(fa, 0, 0);
  bn[1] = mx_read_b<SN>(fa, 0, 1);
  // slice 1 (zero scales on a half step: its products fall below the smallest float),
  // refilling with slice 0 of the next step
  const bool half = src.half_last && ks == nk - 1;
  MxScales s1;
#pragma unroll
  for (int i = 0; i < 4; ++i) s1.a[i] = half ? 0u : sc.a[i];
#pragma unroll
  for (int j = 0; j < 2; ++j) s1.b[j] = half ? 0u : sc.b[j];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    mx_mma_row<1, TR>(a[i], b, s1.a[i], s1, acc.c[i]);
    mx_issue_part<COH, S>(src, ks + 2, nk, nvalid, nhalf, 2 * i);
    mx_issue_part<COH, S>(src, ks + 2, nk, nvalid, nhalf, 2 * i + 1);
    __builtin_amdgcn_sched_barrier(0);
    a[i] = mx_read_a<SN>(fa, 0, i);
  }
  mx_scales_read<SN>(sc);
  b[0] = bn[0];
  b[1] = bn[1];
  __builtin_amdgcn_sched_barrier(0);
}

// Full K loop; K (elements = bytes) a multiple of 64; with TR the accumulators hold C^T.
// Ends with a barrier after all of its loads have landed, so the stages may be reused as
// soon as it returns.
template <bool COH, bool TR = false>
__device__ __forceinline__ void mx_gemm(const MxSrc& src, int K, TileAcc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.f;
  const int nk = (K + 127) / 128;
  if (nk == 0) return;  // empty contraction: the tile is zero
  asm volatile("" ::: "memory");
  mx_issue<COH, 0>(src, 0, nk, true, src.half_last && nk == 1);
  mx_issue<COH, 1>(src, 1, nk, nk > 1, src.half_last && nk == 2);
  wait_vmcnt<2 * geom::kLoads + 1>();  // step 0 landed: at most step 1's 9 loads remain
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  MxFragAddr fa;
  mx_frag_addr_init(fa);
  i32x8_t a[4], b[2];
  MxScales sc;
  mx_scales_read<0>(sc);
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = mx_read_a<0>(fa, 0, i);
  b[0] = mx_read_b<0>(fa, 0, 0);
  b[1] = mx_read_b<0>(fa, 0, 1);
  for (int ks = 0; ks < nk; ks += 2) {
    mx_step<COH, 0, TR>(src, fa, ks, nk, a, b, sc, acc);
    if (ks + 1 < nk) mx_step<COH, 1, TR>(src, fa, ks + 1, nk, a, b, sc, acc);
  }
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace mok
