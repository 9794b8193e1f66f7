// bf16 grouped-GEMM tile for gfx950: one workgroup (4 waves) computes a 128 x 256 fp32
// tile C = A * B^T with A [rows, K] and B [256 rows, K] both K-contiguous, using
// v_mfma_f32_32x32x16_bf16.  Each wave owns 64 rows x 128 columns (2 x 4 MFMA blocks).
//
// The 256 B rows come from two 128-row halves (B0, B1) so the same tile serves
//   GEMM1: B0 = W_gate rows, B1 = W_up rows of the same 128 intermediate columns
//          (the SwiGLU epilogue pairs gate and up values held by the same lane);
//   GEMM2: B0, B1 = two consecutive 128-row blocks of W_down.
//
// Global -> LDS uses gfx950's direct-to-LDS loads (global_load_lds_dwordx4) in a
// three-stage ring: the loads of K step k+2 are issued while step k is multiplied, and
// each step waits only for its own loads (explicit vmcnt, then a bare s_barrier, so the
// later stages stay in flight).  A direct-to-LDS load writes 64 consecutive 16-byte
// chunks per wave; each lane picks the global chunk that belongs at its LDS position.
// LDS rows are 64 bf16 = 8 chunks and chunk c of row r sits at position c ^ (r & 7),
// so the 32 rows read by one MFMA operand fetch spread over all banks.  The three
// stages are separate LDS objects so the compiler can tell a stage being loaded from
// a stage being read.
//
// Rows past the valid range are clamped to the last valid row (always in bounds);
// their results are never stored.  With kCoherent the A operand is read with
// device-scope (sc1) loads: the persistent kernel's A rows are written by workgroups on
// other XCDs, whose L2s are not coherent with this one.
#pragma once
#include "device.h"

namespace mok {

constexpr int kStages = 3;

static __shared__ v4u g_lds_a0[kBM * 8], g_lds_a1[kBM * 8], g_lds_a2[kBM * 8];  // 3 x 16 KB
static __shared__ v4u g_lds_b0[256 * 8], g_lds_b1[256 * 8], g_lds_b2[256 * 8];  // 3 x 32 KB

// Stage arrays named at compile time (never through a runtime select), so every LDS
// access carries the identity of its array.
template <int S> __device__ __forceinline__ v4u* stage_a();
template <int S> __device__ __forceinline__ v4u* stage_b();
template <> __device__ __forceinline__ v4u* stage_a<0>() { return g_lds_a0; }
template <> __device__ __forceinline__ v4u* stage_a<1>() { return g_lds_a1; }
template <> __device__ __forceinline__ v4u* stage_a<2>() { return g_lds_a2; }
template <> __device__ __forceinline__ v4u* stage_b<0>() { return g_lds_b0; }
template <> __device__ __forceinline__ v4u* stage_b<1>() { return g_lds_b1; }
template <> __device__ __forceinline__ v4u* stage_b<2>() { return g_lds_b2; }

__device__ __forceinline__ int lds_chunk(int r, int c) { return r * 8 + (c ^ (r & 7)); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)(const_cast<void*>(p))));
}

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes land at LDS address
// lds_wave_base + 16 * l (the base is wave-uniform and travels in M0).  Written as
// inline asm so the compiler's wait-count pass, which cannot tell the three stages
// apart, does not force every outstanding stage to land before each LDS read; the
// tile's own vmcnt waits order the stages instead.  COHERENT adds the sc1 (device
// scope) cache policy.
template <bool COHERENT>
__device__ __forceinline__ void dma16(const void* src, v4u* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  if (COHERENT)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off sc1" ::"v"(src), "s"(m0)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
                 : "memory", "m0");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

struct TileAcc {
  f32x16_t c[2][4];
};

// Global source of this lane's chunk for each of its 4 A and 8 B direct-to-LDS loads.
struct TileSrc {
  const uint16_t* pa[4];
  const uint16_t* pb[8];
};

// Load p of wave w fills LDS chunk positions [(4p + w) * 64, +64): rows (4p + w) * 8 + l/8,
// physical chunk l % 8, i.e. logical chunk (l % 8) ^ (row % 8).
__device__ __forceinline__ void tile_src_init(TileSrc& s, const uint16_t* A, int64_t lda,
                                              int rows_valid, const uint16_t* B0,
                                              const uint16_t* B1, int64_t ldb, int nb0, int nb1,
                                              int N) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = (l & 7) ^ ((l >> 3) & 7);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = min((p * 4 + w) * 8 + (l >> 3), rows_valid - 1);
    s.pa[p] = A + int64_t(r) * lda + c * 8;
  }
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = (p * 4 + w) * 8 + (l >> 3);
    if (r < 128) {
      s.pb[p] = B0 + int64_t(min(nb0 + r, N - 1)) * ldb + c * 8;
    } else {
      s.pb[p] = B1 + int64_t(min(nb1 + r - 128, N - 1)) * ldb + c * 8;
    }
  }
}

template <bool COH_A, int STAGE>
__device__ __forceinline__ void tile_issue(const TileSrc& s, int k0) {
  const int w = threadIdx.x >> 6;
  v4u* a = stage_a<STAGE>();
  v4u* b = stage_b<STAGE>();
#pragma unroll
  for (int p = 0; p < 4; ++p) dma16<COH_A>(s.pa[p] + k0, a + (p * 4 + w) * 64);
#pragma unroll
  for (int p = 0; p < 8; ++p) dma16<false>(s.pb[p] + k0, b + (p * 4 + w) * 64);
}

// B row (within the 256-row tile) of MFMA block j for wave column wn.
__device__ __forceinline__ int brow_of(int j, int wn) {
  return (j < 2) ? (wn * 64 + j * 32) : (128 + wn * 64 + (j - 2) * 32);
}

template <int STAGE>
__device__ __forceinline__ void tile_compute(TileAcc& acc) {
  const v4u* sa = stage_a<STAGE>();
  const v4u* sb = stage_b<STAGE>();
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int r32 = lane & 31;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = ks * 2 + (lane >> 5);
    v4u a[2], b[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = sa[lds_chunk(wm * 64 + i * 32 + r32, c)];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = sb[lds_chunk(brow_of(j, wn) + r32, c)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc.c[i][j] = mfma32x32x16(a[i], b[j], acc.c[i][j]);
  }
}

// One K step: wait for this step's loads (the next step's may stay in flight), meet,
// start the loads two steps ahead into the stage freed by the previous step, multiply.
template <bool COH_A, int CS, int IS>
__device__ __forceinline__ void tile_step(const TileSrc& src, int kb, int nk, TileAcc& acc) {
  if (kb + 1 < nk) wait_vmcnt<12>();
  else wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (kb + 2 < nk) tile_issue<COH_A, IS>(src, (kb + 2) * kBK);
  tile_compute<CS>(acc);
}

// Full K loop (K a multiple of kBK).  Ends with a barrier, so the stages may be
// reused as soon as it returns.
template <bool kCoherent>
__device__ __forceinline__ void tile_gemm(const TileSrc& src, int K, TileAcc& acc) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.f;
  const int nk = K / kBK;
  asm volatile("" ::: "memory");
  tile_issue<kCoherent, 0>(src, 0);
  if (nk > 1) tile_issue<kCoherent, 1>(src, kBK);
  for (int kb = 0; kb < nk; kb += 3) {
    tile_step<kCoherent, 0, 2>(src, kb, nk, acc);
    if (kb + 1 < nk) tile_step<kCoherent, 1, 0>(src, kb + 1, nk, acc);
    if (kb + 2 < nk) tile_step<kCoherent, 2, 1>(src, kb + 2, nk, acc);
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Row (within the 128-row tile) held by accumulator element v of block i for this lane.
__device__ __forceinline__ int acc_row(int i, int v) {
  const int lane = threadIdx.x & 63;
  const int wm = (threadIdx.x >> 6) >> 1;
  return wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

}  // namespace mok
