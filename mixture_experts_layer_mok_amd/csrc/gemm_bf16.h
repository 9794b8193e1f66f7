// bf16 grouped-GEMM tile for gfx950: one workgroup (8 waves, two per SIMD) computes a
// 256 x 256 fp32 tile C = A * B^T with A [rows, K] and B [256 rows, K] both K-contiguous,
// using v_mfma_f32_32x32x16_bf16.  Wave w owns rows 128 * (w / 4) .. +128 and B rows
// 64 * (w % 4) .. +64 (4 x 2 MFMA blocks, 128 accumulator registers), which leaves room
// for double-buffered fragments without spills, and the second wave per SIMD covers the
// other's waits.
//
// The 256 B rows come from two matrices (B0, B1) so the same tile serves
//   GEMM1: W_gate and W_up rows of the same 128 intermediate columns, paired per MFMA
//          block (16 gate rows then the same 16 up rows), so that in a transposed tile
//          (TR: the MFMA computes C^T, one row of C per lane) every lane holds each of
//          its gate values and the matching up value;
//   GEMM2: B0, B1 = two consecutive 128-row blocks of W_down.
// The epilogues take transposed tiles: a lane's sixteen values of a block are then
// columns of one row in groups of four, which the epilogues stage as 8-byte LDS writes.
//
// Data movement per K step of 64 (128 bytes per row, whole cache lines): 64 KB of A and
// B move from global memory straight into LDS with gfx950's direct-to-LDS loads
// (global_load_lds_dwordx4) through a two-stage ring.  Measured on MI355X, the L2 -> CU
// path delivers about 36 bytes per clock per CU for whole 128-byte row segments but
// only about 23 for half lines, and the 256 x 256 tile needs 32 bytes per MFMA-cycle, so
// whole-line steps and the largest tile the LDS holds are what bound this kernel.  Per
// step each wave multiplies four 16-deep slices, reading the next slice's fragments
// under the current slice's MFMAs; before the last slice it waits for the next step's
// loads, meets the other waves at one barrier, starts the loads two steps ahead into
// the stage just drained, and reads the next step's first fragments.  The loads are
// inline asm: the compiler's wait-count pass cannot tell the stages apart and would
// otherwise wait for every stage before each LDS read.
//
// LDS rows are 8 chunks of 16 bytes; chunk c of row r sits at position
// c ^ (r & 7) ^ ((r >> 3) & 1).  The LDS has 64 four-byte banks, so a 128-byte row covers
// half of them; one ds_read_b128 pass serves 16 lanes = 16 consecutive rows at one
// logical chunk, which this swizzle spreads over all 64 banks.  Direct-to-LDS writes
// are contiguous.
//
// Rows past the valid range are clamped to the last valid row (always in bounds);
// their results are never stored.  Byte offsets stay below 2^32: an A tile spans at
// most 256 rows of at most 65536 bf16, and a weight matrix holds fewer than 2^31 bf16
// (checked on the host).  With COH the A operand is read with
// device-scope
// (sc1) loads: in the persistent kernel the A rows are written by workgroups on other
// XCDs, whose L2s are not coherent with this one.
#pragma once
#include "device.h"
#include "tile_geom.h"

namespace mok {

constexpr int kStageChunks = kBM * 8;  // 16-byte chunks per operand per stage (32 KB)
constexpr int kStageBytes = kStageChunks * 16;

static __shared__ v4u g_lds_a[2 * kStageChunks];  // two stages of A
static __shared__ v4u g_lds_b[2 * kStageChunks];  // two stages of B

template <int S> __device__ __forceinline__ v4u* stage_a() { return g_lds_a + S * kStageChunks; }
template <int S> __device__ __forceinline__ v4u* stage_b() { return g_lds_b + S * kStageChunks; }

__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int lds_chunk(int r, int c) { return r * 8 + (c ^ lds_swz(r)); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)(const_cast<void*>(p))));
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource for byte offsets below 2^32 from `base` (wave-uniform).
__device__ __forceinline__ i32x4_t make_rsrc(const void* base) {
  const uint64_t x = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(int(uint32_t(x)));
  r.y = __builtin_amdgcn_readfirstlane(int(uint32_t(x >> 32) & 0xFFFFu));  // stride 0
  r.z = -16;           // number of records (bytes): all offsets used here are far below
  r.w = 0x00020000;    // raw buffer, 32-bit data
  return r;
}

// The resource, or with `empty` the same one with no records: a load through it reads no
// memory and returns zeros (the loads a K loop issues past its last step).
__device__ __forceinline__ i32x4_t rsrc_or_empty(const i32x4_t& r, bool empty) {
  i32x4_t e = r;
  e.z = empty ? 0 : r.z;
  return e;
}

// Direct-to-LDS load of 16 bytes per lane from rsrc + voff + soff: lane l's bytes land
// at LDS address lds_wave_base + 16 * l (the wave-uniform base travels in M0).  COH adds
// sc1 (device scope).
template <bool COH>
__device__ __forceinline__ void dma16_at(const i32x4_t& rsrc, uint32_t voff, uint32_t soff,
                                         uint32_t lds_wave_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_addr);
  soff = __builtin_amdgcn_readfirstlane(soff);  // uniform; kept in an SGPR for the asm
  if (COH)
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen sc1 lds" ::"v"(voff),
                 "s"(rsrc), "s"(soff), "s"(m0)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff),
                 "s"(rsrc), "s"(soff), "s"(m0)
                 : "memory", "m0");
}
template <bool COH>
__device__ __forceinline__ void dma16(const i32x4_t& rsrc, uint32_t voff, uint32_t soff,
                                      const v4u* lds_wave_base) {
  dma16_at<COH>(rsrc, voff, soff, lds_addr(lds_wave_base));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(0) lgkmcnt(0): every load of this wave has landed, global and LDS.
// Before the barrier that frees a stage this matters for the LDS reads too: once past
// the barrier, other waves start direct-to-LDS loads into the stage those reads use.
__device__ __forceinline__ void wait_loads_and_lds() {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0 << 8) | (0 << 14));
}

struct TileAcc {
  f32x16_t c[4][2];
};

// Sources of this lane's 8 A and 8 B direct-to-LDS loads: one buffer resource per
// operand (based at its first row / the weight matrix's first row) and a fixed,
// non-negative per-lane byte offset (tile_geom.h); the K step travels in the scalar
// offset.  Load p of wave w fills LDS positions [(4p + w) * 64, +64): rows
// (4p + w) * 8 + l/8 at physical position l % 8, i.e. logical chunk (l % 8) ^
// lds_swz(row), and for those rows lds_swz(row) = (l / 8) ^ (w % 2).  Which B matrix
// a load reads depends on the B layout (geom::b_matrix): per load p for kSplit, per
// wave for kPaired.
struct TileSrc {
  i32x4_t ra, rb0, rb1;
  uint32_t oa[geom::kLoads], ob[geom::kLoads];
  int layout;
};

__device__ __forceinline__ void tile_src_init(TileSrc& s, int layout, const uint16_t* A,
                                              int64_t lda, int rows_valid, const uint16_t* B0,
                                              const uint16_t* B1, int64_t ldb, int nb0, int nb1,
                                              int N) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  s.layout = layout;
  s.ra = make_rsrc(A);
  s.rb0 = make_rsrc(B0);
  s.rb1 = make_rsrc(B1);
#pragma unroll
  for (int p = 0; p < geom::kLoads; ++p) {
    s.oa[p] = uint32_t(geom::a_offset(p, w, l, rows_valid, lda));
    s.ob[p] = uint32_t(geom::b_offset(layout, p, w, l, nb0, nb1, N, ldb));
  }
}

// As tile_src_init, with the A rows gathered: tile row r (clamped to rows_valid - 1) is
// row rowmap[r] / k of X [*, ldx] (rowmap = the schedule's perm from the tile's first
// routed row: pair index t*k + j, token t).  Offsets are taken from X's base, so X must
// hold fewer than 2^31 elements (checked on the host).
__device__ __forceinline__ void tile_src_init_gather(TileSrc& s, int layout, const uint16_t* X,
                                                     int64_t ldx, const int32_t* rowmap, int k,
                                                     int rows_valid, const uint16_t* B0,
                                                     const uint16_t* B1, int64_t ldb, int nb0,
                                                     int nb1, int N) {
  tile_src_init(s, layout, X, ldx, rows_valid, B0, B1, ldb, nb0, nb1, N);
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int p = 0; p < geom::kLoads; ++p) {
    int r = geom::dma_row(p, w, l);
    if (r > rows_valid - 1) r = rows_valid - 1;
    const int64_t src = rowmap[r] / k;
    s.oa[p] = uint32_t((src * ldx + geom::dma_chunk(w, l) * 8) * 2);
  }
}

template <bool COH, int STAGE>
__device__ __forceinline__ void tile_issue(const TileSrc& s, int k0) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const uint32_t kb = uint32_t(k0) * 2;
#pragma unroll
  for (int p = 0; p < geom::kLoads; ++p)
    dma16<COH>(s.ra, s.oa[p], kb, stage_a<STAGE>() + (p * 8 + w) * 64);
  const bool paired_up = s.layout == geom::kPaired && ((w >> 1) & 1);
#pragma unroll
  for (int p = 0; p < geom::kLoads; ++p) {
    const bool use_b1 = s.layout == geom::kPaired ? paired_up : (p >= 2);
    dma16<false>(use_b1 ? s.rb1 : s.rb0, s.ob[p], kb, stage_b<STAGE>() + (p * 8 + w) * 64);
  }
}

// B row (within the 256-row tile) of MFMA block j (0..1) of wave column wn (0..3).
__device__ __forceinline__ int brow_of(int j, int wn) { return wn * 64 + j * 32; }

struct TileFrag {
  v4u a[4], b[2];
};

typedef __attribute__((address_space(3))) const v4u lds_cv4u;

// Per-lane LDS byte addresses of the fragment reads of slice ks in stage 0: A rows
// 128 * wm + r32 (+32 i), B rows 64 * wn + r32 (+32 j), chunk (2 ks + l/32) swizzled.
// The swizzle only depends on r32, so block and stage offsets are immediates.
struct FragAddr {
  uint32_t a[4], b[4];
};

__device__ __forceinline__ void frag_addr_init(FragAddr& fa) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int r32 = lane & 31;
  const int sw = lds_swz(r32);
  const uint32_t a0 = lds_addr(g_lds_a) + uint32_t(wm * 128 + r32) * 128;
  const uint32_t b0 = lds_addr(g_lds_b) + uint32_t(wn * 64 + r32) * 128;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t ch = uint32_t(((ks * 2 + (lane >> 5)) ^ sw) * 16);
    fa.a[ks] = a0 + ch;
    fa.b[ks] = b0 + ch;
  }
}

// Fragments of slice ks (16 deep) of stage S.
template <int S>
__device__ __forceinline__ void frag_load(TileFrag& f, const FragAddr& fa, int ks) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i] = *reinterpret_cast<lds_cv4u*>(uintptr_t(fa.a[ks] + S * kStageBytes + i * 32 * 128));
#pragma unroll
  for (int j = 0; j < 2; ++j)
    f.b[j] = *reinterpret_cast<lds_cv4u*>(uintptr_t(fa.b[ks] + S * kStageBytes + j * 32 * 128));
}

// One MFMA block: C += A B^T, or with TR its transpose C^T += B A^T (the B fragment
// takes the MFMA's A slot).  Transposed, lane l of block (i, j) holds tile row
// 32 i + l % 32 (+ 128 wm) at B rows brow_of(j, wn) + 8 (v / 4) + 4 (l / 32) + v % 4:
// sixteen columns of one row, in groups of four consecutive ones.
template <bool TR>
__device__ __forceinline__ f32x16_t mma_blk(v4u a, v4u b, f32x16_t c) {
  return TR ? mfma32x32x16(b, a, c) : mfma32x32x16(a, b, c);
}

template <bool TR = false>
__device__ __forceinline__ void frag_mma(const TileFrag& f, TileAcc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc.c[i][j] = mma_blk<TR>(f.a[i], f.b[j], acc.c[i][j]);
}

// 8 KB of LDS that takes the loads a step issues past the last step (one 1 KB block
// per wave), so the step body has no branch around its loads.
static __shared__ v4u g_lds_dummy[(kThreads / 64) * 64];

// One direct-to-LDS load (q = 0..3: A load q; 4..7: B load q - 4) into stage STAGE, or,
// with `dummy`, into the scratch area through an empty resource (loads past the last
// step: no branch in the step and no memory read).
template <bool COH, int STAGE>
__device__ __forceinline__ void tile_issue_sel(const TileSrc& s, int k0, int q, bool dummy) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t kb = uint32_t(k0) * 2;
  // the destination is selected as an LDS address (selecting generic pointers to LDS
  // makes the compiler emit an invalid null check of the shared aperture)
  uint32_t dst = q < 4 ? lds_addr(stage_a<STAGE>() + (q * 8 + w) * 64)
                       : lds_addr(stage_b<STAGE>() + ((q - 4) * 8 + w) * 64);
  dst = dummy ? lds_addr(g_lds_dummy) + uint32_t(w) * 1024u : dst;
  if (q < 4) {
    dma16_at<COH>(rsrc_or_empty(s.ra, dummy), s.oa[q], kb, dst);
  } else {
    const int p = q - 4;
    const bool paired_up = s.layout == geom::kPaired && ((w >> 1) & 1);
    const bool use_b1 = s.layout == geom::kPaired ? paired_up : (p >= 2);
    dma16_at<false>(rsrc_or_empty(use_b1 ? s.rb1 : s.rb0, dummy), s.ob[p], kb, dst);
  }
}

// One K step kb held in stage S (S = kb % 2).  On entry f0 holds slice 0 of step kb.
// After the barrier that ends the reads of stage S, the eight loads of step kb + 2 are
// issued one per MFMA of the last slice rather than in one burst: a burst fills the
// vector-memory command queue and holds up the MFMAs behind it (measured on MI355X:
// 1091 -> 1121 TFLOP/s on a plain 16384 x 4096 x 7168 GEMM).  That needs a step body
// without a branch around the MFMAs (with one, the compiler spills), so the loads are
// always issued; past the last step they go to g_lds_dummy through an empty resource
// (no memory read).
template <bool COH, int S, bool TR>
__device__ __forceinline__ void tile_step(const TileSrc& src, const FragAddr& fa, int kb, int nk,
                                          TileFrag& f0, TileFrag& f1, TileAcc& acc) {
  constexpr int SN = S ^ 1;
  frag_load<S>(f1, fa, 1);
  __builtin_amdgcn_sched_barrier(0);
  frag_mma<TR>(f0, acc);
  __builtin_amdgcn_sched_barrier(0);
  frag_load<S>(f0, fa, 2);
  __builtin_amdgcn_sched_barrier(0);
  frag_mma<TR>(f1, acc);
  __builtin_amdgcn_sched_barrier(0);
  frag_load<S>(f1, fa, 3);
  __builtin_amdgcn_sched_barrier(0);
  frag_mma<TR>(f0, acc);
  __builtin_amdgcn_sched_barrier(0);
  if (kb + 1 < nk) {
    wait_loads_and_lds();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  __builtin_amdgcn_sched_barrier(0);
  // loads of step kb + 2; past the end they go to the scratch area and read nothing
  const bool past = kb + 2 >= nk;
  const int kn = __builtin_amdgcn_readfirstlane(past ? kb * kBK : (kb + 2) * kBK);
  frag_load<SN>(f0, fa, 0);  // past the last step: stale, unused
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = q >> 1, j = q & 1;
    acc.c[i][j] = mma_blk<TR>(f1.a[i], f1.b[j], acc.c[i][j]);
    tile_issue_sel<COH, S>(src, kn, q, past);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Full K loop (K a multiple of kBK); with TR the accumulators hold C^T (see mma_blk).
// Ends with a barrier, so the stages may be reused as soon as it returns.
template <bool COH, bool TR = false>
__device__ __forceinline__ void tile_gemm(const TileSrc& src, int K, TileAcc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.f;
  const int nk = K / kBK;
  if (nk == 0) return;  // empty contraction: the tile is zero
  asm volatile("" ::: "memory");
  tile_issue<COH, 0>(src, 0);
  if (nk > 1) {
    tile_issue<COH, 1>(src, kBK);
    wait_vmcnt<2 * geom::kLoads>();
  } else {
    wait_vmcnt<0>();
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  FragAddr fa;
  frag_addr_init(fa);
  TileFrag f0, f1;
  frag_load<0>(f0, fa, 0);
  for (int kb = 0; kb < nk; kb += 2) {
    tile_step<COH, 0, TR>(src, fa, kb, nk, f0, f1, acc);
    if (kb + 1 < nk) tile_step<COH, 1, TR>(src, fa, kb + 1, nk, f0, f1, acc);
  }
  wait_vmcnt<0>();  // the loads issued past the last step
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------------------------
// Tiles with K-major operands
// ------------------------------------------------------------------------------------
// The backward contracts over dimensions that are not contiguous in memory: over the
// rows of the weights (dX, dH: the B columns are contiguous along a weight row) and over
// the routed rows (dW: both operands).  Such an operand is staged K-major (tile_geom.h:
// 64 K rows of 256 columns per stage, swizzled in 4-chunk groups) and its MFMA fragments
// are read with ds_read_b64_tr_b16.  That instruction transposes 16-bit elements within
// each group of 16 lanes: lane i of a group receives element i % 4 of the 8-byte chunks
// addressed by lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 (measured on MI355X).
// So if lane s of a group addresses K row kb + s / 4 at column cb + 4 (s % 4), lane i
// receives K rows kb .. kb + 3 of column cb + i: half of an MFMA operand; a second read
// at K + 4 gives the other half.  Per read, the 16 lanes of a group touch 4 K rows
// whose swizzle groups differ, so the 64 lanes hit every bank exactly twice.
//
// Operand kinds:
//   kKC  K-contiguous rows (the tile above; rows may be gathered);
//   kKCD kKC read at device scope (sc1): rows written earlier in the same launch by
//        workgroups on other XCDs;
//   kKW  K-major weight matrix [K rows][ld]: tile column n is column n of every row;
//        K rows past ksplit come from a second matrix (dX stacks W_gate over W_up);
//   kKR  K-major routed rows of a row matrix: K index q is routed row r = rbeg + q at
//        byte r * row bytes;
//   kKRD kKR read at device scope (rows written earlier in the same launch);
//   kKG  K-major routed rows gathered: row r starts at byte rowb[r] of the resource.
//        The offsets are staged in LDS per window of kRowTabLds rows (loaded at the
//        start and every kRowTabLds rows): reading them from memory in the load loop
//        would share the in-order vector-memory counter with the operand loads, so that
//        every wait for the one also waits for the other.
// For kKR and kKG, rows at or past rend read zero (bit 31 of the offset, against a 2 GB
// resource).
enum KmKind { kKC = 0, kKW = 1, kKR = 2, kKG = 3, kKCD = 4, kKRD = 5 };
constexpr bool km_kcontig(int kind) { return kind == kKC || kind == kKCD; }
constexpr uint32_t kKmOutOfRange = 0x80000000u;
constexpr int kKmRowBytes = 512;  // one staged K row: 256 bf16

struct KmOp {
  i32x4_t r0, r1;
  uint32_t off[geom::kLoads];  // kKC / kKW: per-lane byte offsets; kKR: column bytes
  uint32_t ld2;                // kKW: bytes per K row; kKR: bytes per source row
  int ksplit;                  // kKW
  const uint32_t* rowb;        // kKG: byte offset of each routed row
  int rbeg, rend;              // kKR, kKG
  uint32_t nxt[geom::kLoads];  // kKG: offsets of the rows of the next step to issue
};

__device__ __forceinline__ i32x4_t make_rsrc_2g_km(const void* base) {
  i32x4_t r = make_rsrc(base);
  r.z = int(kKmOutOfRange);
  return r;
}

// K-contiguous rows [rows_valid, lda] from A (kKC), as tile_src_init's A operand.
__device__ __forceinline__ void km_init_kc(KmOp& o, const uint16_t* A, int64_t lda,
                                           int rows_valid) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  o.r0 = make_rsrc(A);
#pragma unroll
  for (int p = 0; p < geom::kLoads; ++p)
    o.off[p] = uint32_t(geom::a_offset(p, w, l, rows_valid, lda));
}

// As km_init_kc with the rows gathered: tile row r (clamped to rows_valid - 1) is row
// rowmap[r] / k of X (fewer than 2^31 elements, checked on the host).
__device__ __forceinline__ void km_init_kc_gather(KmOp& o, const uint16_t* X, int64_t ldx,
                                                  const int32_t* rowmap, int k, int rows_valid) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  o.r0 = make_rsrc(X);
#pragma unroll
  for (int p = 0; p < geom::kLoads; ++p) {
    int r = geom::dma_row(p, w, l);
    if (r > rows_valid - 1) r = rows_valid - 1;
    o.off[p] = uint32_t((int64_t(rowmap[r] / k) * ldx + geom::dma_chunk(w, l) * 8) * 2);
  }
}

// K-major weights: rows [0, ksplit) of W0, then rows of W1; tile columns n0 .. n0+255
// of N (ld elements per row).
__device__ __forceinline__ void km_init_weights(KmOp& o, const uint16_t* W0, const uint16_t* W1,
                                                int ksplit, int64_t ld, int n0, int N) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  o.r0 = make_rsrc(W0);
  o.r1 = make_rsrc(W1);
  o.ld2 = uint32_t(ld * 2);
  o.ksplit = ksplit;
#pragma unroll
  for (int p = 0; p < geom::kLoads; ++p)
    o.off[p] = uint32_t((int64_t(geom::km_row(p, w, l)) * ld + geom::km_col(w, l, n0, N)) * 2);
}

constexpr int kRowTabLds = 4096;  // routed-row offsets per LDS window (64 K steps)
static __shared__ uint32_t g_lds_rowtab[kRowTabLds];

// Window of row offsets [rbeg + q0, rbeg + q0 + kRowTabLds) into LDS (zero past rend).
// Every thread of the workgroup calls it; it ends with a barrier.
__device__ __forceinline__ void km_load_rowtab(const KmOp& o, int q0) {
  for (int i = threadIdx.x; i < kRowTabLds; i += kThreads) {
    const int r = o.rbeg + q0 + i;
    g_lds_rowtab[i] = r < o.rend ? o.rowb[r] : 0u;
  }
  __syncthreads();
}

// K-major routed rows [rbeg, rend) of base (kKR: row r at r * ld * 2; kKG: at rowb[r]);
// tile columns n0 .. n0+255 of N (col0 added to every column).  For kKG every thread of
// the workgroup must call this (it stages the first window of offsets).
template <int KIND>
__device__ __forceinline__ void km_init_rows(KmOp& o, const void* base, int64_t ld, int col0,
                                             int n0, int N, const uint32_t* rowb, int rbeg,
                                             int rend) {
  static_assert(KIND == kKR || KIND == kKRD || KIND == kKG, "routed-row operand");
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  o.r0 = make_rsrc_2g_km(base);
  o.ld2 = uint32_t(ld * 2);
  o.rowb = rowb;
  o.rbeg = rbeg;
  o.rend = rend;
#pragma unroll
  for (int p = 0; p < geom::kLoads; ++p)
    o.off[p] = uint32_t((col0 + geom::km_col(w, l, n0, N)) * 2);
  if (KIND == kKG) {
    km_load_rowtab(o, 0);
#pragma unroll
    for (int p = 0; p < geom::kLoads; ++p) o.nxt[p] = g_lds_rowtab[geom::km_row(p, w, l)];
  }
}

template <int KIND, int STAGE>
__device__ __forceinline__ void km_issue(KmOp& o, int k0, v4u* lds) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (km_kcontig(KIND)) {
#pragma unroll
    for (int p = 0; p < geom::kLoads; ++p)
      dma16<KIND == kKCD>(o.r0, o.off[p], uint32_t(k0) * 2,
                          lds + STAGE * kStageChunks + (p * 8 + w) * 64);
  } else if (KIND == kKW) {
    const bool second = k0 >= o.ksplit;
    const uint32_t so = uint32_t(second ? k0 - o.ksplit : k0) * o.ld2;
#pragma unroll
    for (int p = 0; p < geom::kLoads; ++p)
      dma16<false>(second ? o.r1 : o.r0, o.off[p], so,
                   lds + STAGE * kStageChunks + (p * 8 + w) * 64);
  } else {
    const int l = threadIdx.x & 63;
    uint32_t voff[geom::kLoads];
#pragma unroll
    for (int p = 0; p < geom::kLoads; ++p) {
      const int r = o.rbeg + k0 + geom::km_row(p, w, l);
      // row index and row bytes below 2^24 (checked on the host); kKG offsets were read
      // from LDS at the previous issue, so no wait holds up these loads
      const uint32_t rb = KIND == kKG ? o.nxt[p] : __umul24(uint32_t(r), o.ld2);
      voff[p] = r < o.rend ? rb + o.off[p] : kKmOutOfRange;
    }
#pragma unroll
    for (int p = 0; p < geom::kLoads; ++p)
      dma16<KIND == kKRD>(o.r0, voff[p], 0u, lds + STAGE * kStageChunks + (p * 8 + w) * 64);
    if (KIND == kKG) {
      // offsets of the next step; a next step that starts a new window reloads it (every
      // wave read its offsets from the old one at the previous issue, before the barrier
      // that preceded this one)
      const int kn = k0 + kBK;
      if (kn % kRowTabLds == 0) km_load_rowtab(o, kn);
#pragma unroll
      for (int p = 0; p < geom::kLoads; ++p)
        o.nxt[p] = g_lds_rowtab[(kn + geom::km_row(p, w, l)) % kRowTabLds];
    }
  }
}

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s;

// 8 K-consecutive bf16 of a K-major operand: two transposing reads, K rows +0..3, +4..7.
__device__ __forceinline__ v4u km_frag(uint32_t addr) {
  const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4s*>(uintptr_t(addr)));
  const v4s_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4s*>(uintptr_t(addr + 4 * kKmRowBytes)));
  typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));
  const v2u_t a = __builtin_bit_cast(v2u_t, lo), b = __builtin_bit_cast(v2u_t, hi);
  return v4u{a.x, a.y, b.x, b.y};
}

// Per-lane LDS byte address of the K-major fragment of 32-column block `blk` (columns
// cw + 32 blk ..) for slice 0, read 0 of stage 0; slice ks adds 16 K rows, read 1 adds 4.
__device__ __forceinline__ uint32_t km_frag_addr(uint32_t base, int cw, int blk) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, s = lane & 15;
  const int col = cw + 32 * blk + 16 * (g & 1) + 4 * (s & 3);
  const int kk = 8 * (g >> 1) + (s >> 2);
  const int pos = (col >> 3) ^ (4 * (kk & 3));
  return base + uint32_t(kk * kKmRowBytes + pos * 16 + (col & 7) * 2);
}

struct KmFragAddr {
  uint32_t a[4], b[2];  // kKC A: per slice; K-major A: per block i; B: per block j
};

template <int AK>
__device__ __forceinline__ void km_frag_addr_init(KmFragAddr& fa) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 2, wn = w & 3;
  if (km_kcontig(AK)) {
    const int r32 = lane & 31;
    const uint32_t a0 = lds_addr(g_lds_a) + uint32_t(wm * 128 + r32) * 128;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      fa.a[ks] = a0 + uint32_t(((ks * 2 + (lane >> 5)) ^ lds_swz(r32)) * 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa.a[i] = km_frag_addr(lds_addr(g_lds_a), wm * 128, i);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) fa.b[j] = km_frag_addr(lds_addr(g_lds_b), wn * 64, j);
}

template <int AK, int S>
__device__ __forceinline__ void km_frag_load(TileFrag& f, const KmFragAddr& fa, int ks) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (km_kcontig(AK))
      f.a[i] = *reinterpret_cast<lds_cv4u*>(uintptr_t(fa.a[ks] + S * kStageBytes + i * 32 * 128));
    else
      f.a[i] = km_frag(fa.a[i] + S * kStageBytes + ks * 16 * kKmRowBytes);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) f.b[j] = km_frag(fa.b[j] + S * kStageBytes + ks * 16 * kKmRowBytes);
}

template <int AK, int BK, int S>
__device__ __forceinline__ void km_issue_step(KmOp& a, KmOp& b, int k0) {
  km_issue<AK, S>(a, k0, g_lds_a);
  km_issue<BK, S>(b, k0, g_lds_b);
}

// Load p (0..3) of one K step of a non-gathered K-major or K-contiguous operand, into
// stage STAGE of lds, or with `dummy` into g_lds_dummy through an empty resource (loads
// past the last step: they read no memory).
template <int KIND, int STAGE>
__device__ __forceinline__ void km_issue_one(const KmOp& o, int k0, int p, v4u* lds, bool dummy) {
  static_assert(KIND != kKG, "gathered operands are issued per step (km_issue)");
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t dst = dummy ? lds_addr(g_lds_dummy) + uint32_t(w) * 1024u
                             : lds_addr(lds + STAGE * kStageChunks + (p * 8 + w) * 64);
  if (km_kcontig(KIND)) {
    dma16_at<KIND == kKCD>(rsrc_or_empty(o.r0, dummy), o.off[p], uint32_t(k0) * 2, dst);
  } else if (KIND == kKW) {
    const bool second = k0 >= o.ksplit;
    const uint32_t so = uint32_t(second ? k0 - o.ksplit : k0) * o.ld2;
    dma16_at<false>(rsrc_or_empty(second ? o.r1 : o.r0, dummy), o.off[p], so, dst);
  } else {
    const int l = threadIdx.x & 63;
    const int r = o.rbeg + k0 + geom::km_row(p, w, l);
    const uint32_t voff = r < o.rend ? __umul24(uint32_t(r), o.ld2) + o.off[p] : kKmOutOfRange;
    dma16_at<KIND == kKRD>(rsrc_or_empty(o.r0, dummy), voff, 0u, dst);
  }
}

// One K step kb in stage S, as tile_step: after the barrier, the loads of step kb + 2 of
// each non-gathered operand go out one per MFMA of the last slice (past the last step
// into g_lds_dummy, so the MFMAs sit in no branch); a gathered operand's loads, which
// read their offsets from the LDS row table, go out in one group before them.
template <int AK, int BK, int S, bool TR>
__device__ __forceinline__ void km_step(KmOp& a, KmOp& b, const KmFragAddr& fa, int kb, int nk,
                                        TileFrag& f0, TileFrag& f1, TileAcc& acc) {
  constexpr int SN = S ^ 1;
  km_frag_load<AK, S>(f1, fa, 1);
  __builtin_amdgcn_sched_barrier(0);
  frag_mma<TR>(f0, acc);
  __builtin_amdgcn_sched_barrier(0);
  km_frag_load<AK, S>(f0, fa, 2);
  __builtin_amdgcn_sched_barrier(0);
  frag_mma<TR>(f1, acc);
  __builtin_amdgcn_sched_barrier(0);
  km_frag_load<AK, S>(f1, fa, 3);
  __builtin_amdgcn_sched_barrier(0);
  frag_mma<TR>(f0, acc);
  __builtin_amdgcn_sched_barrier(0);
  if (kb + 1 < nk) {
    wait_loads_and_lds();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kb + 2 < nk) {
      if (AK == kKG) km_issue<AK, S>(a, (kb + 2) * kBK, g_lds_a);
      if (BK == kKG) km_issue<BK, S>(b, (kb + 2) * kBK, g_lds_b);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const bool past = kb + 2 >= nk;
  const int kn = __builtin_amdgcn_readfirstlane(past ? kb * kBK : (kb + 2) * kBK);
  km_frag_load<AK, SN>(f0, fa, 0);  // past the last step: stale, unused
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = q >> 1, j = q & 1;
    acc.c[i][j] = mma_blk<TR>(f1.a[i], f1.b[j], acc.c[i][j]);
    if (q < 4) {
      if (AK != kKG) km_issue_one<AK == kKG ? kKC : AK, S>(a, kn, q, g_lds_a, past);
    } else {
      if (BK != kKG) km_issue_one<BK == kKG ? kKW : BK, S>(b, kn, q - 4, g_lds_b, past);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// K loop of nk steps over operands a (kind AK: kKC, kKCD, kKR or kKG) and b (kind BK: kKW,
// kKR or kKG; at most one kKG operand: they share the LDS offset table).
// C = A B^T as for tile_gemm, with A's tile row m / B's tile row n read as column m / n
// of a K-major operand; with TR the accumulators hold C^T (see mma_blk).  Ends with a
// barrier.
template <int AK, int BK, bool TR = false>
__device__ __forceinline__ void tile_gemm_km(KmOp& a, KmOp& b, int nk, TileAcc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.f;
  if (nk <= 0) return;
  asm volatile("" ::: "memory");
  km_issue_step<AK, BK, 0>(a, b, 0);
  if (nk > 1) {
    km_issue_step<AK, BK, 1>(a, b, kBK);
    wait_vmcnt<2 * geom::kLoads>();
  } else {
    wait_vmcnt<0>();
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  KmFragAddr fa;
  km_frag_addr_init<AK>(fa);
  TileFrag f0, f1;
  km_frag_load<AK, 0>(f0, fa, 0);
  for (int kb = 0; kb < nk; kb += 2) {
    km_step<AK, BK, 0, TR>(a, b, fa, kb, nk, f0, f1, acc);
    if (kb + 1 < nk) km_step<AK, BK, 1, TR>(a, b, fa, kb + 1, nk, f0, f1, acc);
  }
  wait_vmcnt<0>();  // the loads issued past the last step
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A value the compiler must treat as produced here: epilogue address arithmetic derived
// from it cannot be hoisted above the K loop, where it would hold registers.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Row (within the 256-row tile) held by accumulator element v of block i for a lane
// with index tid in the workgroup.
__device__ __forceinline__ int acc_row(int tid, int i, int v) {
  const int lane = tid & 63;
  const int wm = (tid >> 6) >> 2;
  return wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// silu(a) = a / (1 + e^-a), with the hardware exponential and reciprocal (about 1 ulp
// each; H is rounded to bf16 or e4m3 right after).
__device__ __forceinline__ float silu_f(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

}  // namespace mok
