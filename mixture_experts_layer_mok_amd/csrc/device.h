// Device-side helpers shared by the layer's kernels: bf16 conversion, vector types,
// MFMA wrappers, and the release/acquire handoff primitives of the persistent kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace mok {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // 16-byte chunk (native vector)

// ------------------------------------------------------------------------------------
// bf16 (carried as uint16 bit patterns)
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}
// Round to nearest, ties to even.  Values here are finite.
// float32 -> bf16, round to nearest even, with gfx950's v_cvt_pk_bf16_f32 (one
// instruction per pair; every value rounded here is finite).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(v4u v) { return __builtin_bit_cast(bf16x8_t, v); }

// 32x32x16 bf16 MFMA: C[32x32] += A[32x16] * B[16x32].  Lane l supplies A row (l%32),
// K elements 8*(l/32) .. +8, and B column (l%32), the same K elements.  Lane l receives
// C column (l%32), rows 8*(v/4) + 4*(l/32) + (v%4) for v = 0..15.
__device__ __forceinline__ f32x16_t mfma32x32x16(v4u a, v4u b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ------------------------------------------------------------------------------------
// Cross-workgroup handoff inside the persistent kernels.
//
// MI355X has 8 XCDs, each with its own L2; plain stores may sit in the producer's L2 and
// plain loads may hit a stale line in the consumer's L2.  Instead of agent-scope
// release/acquire fences (which write back and invalidate the whole L2 of the XCD on
// every handoff and so destroy the weight reuse of every workgroup on it), all data
// that crosses workgroups inside a kernel is written with device-scope stores and read
// with device-scope loads (the sc1 cache policy), which are coherent on their own.
// The counters are agent-scope atomics.
//   producer: device-scope data stores; wait for them (vmcnt 0); meet; one thread adds.
//   consumer: one thread polls the counter; meet; device-scope data loads.
// Waits are bounded: on expiry the waiter sets MOK_DEV_TIMEOUT and the abort word,
// and every loop of the persistent kernels exits once the abort word is set.
// ------------------------------------------------------------------------------------
constexpr uint64_t kWaitTicks = 200000000ull;  // 2 s of the 100 MHz constant clock
constexpr uint64_t kShortWaitTicks = 100ull;   // 1 us: MOK_FLAG_SHORT_WAITS

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void or_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// device-scope (coherent across XCDs) data movement
__device__ __forceinline__ void st_dev_u16(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u8(uint8_t* p, uint8_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u64(void* p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_b128(void* p, v4u v) {
  uint64_t* q = static_cast<uint64_t*>(p);
  __hip_atomic_store(q, uint64_t(v.x) | (uint64_t(v.y) << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, uint64_t(v.z) | (uint64_t(v.w) << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// Row access through a buffer resource: the hardware checks every access against the
// row's length, so loads past the end read zero and stores past it are dropped, which
// lets a row loop run without per-chunk branches.  The base is made wave-uniform.
// kCpolDev (sc1) makes an access device scope, as the handoff protocol above requires.
// kCpolStream (nt) marks an access non-temporal, for rows written once and read once by
// a later step (results, saved activations): they then do not displace the L2 lines
// that the GEMM tiles re-read (measured on MI355X: the MXFP8 forward at config 4 4.70 ->
// 4.50 ms, the config-4 combine as its own launch 320 -> 265 us).  It combines with sc1.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kCpolPlain = 0;
constexpr int kCpolDev = 16;
constexpr int kCpolStream = 2;

__device__ __forceinline__ rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  const uint64_t x = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(x >> 32));
  void* b = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, 0, int(__builtin_amdgcn_readfirstlane(bytes)),
                                           0x00020000);
}
template <int CPOL>
__device__ __forceinline__ v4u buf_ld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL);
}
template <int CPOL>
__device__ __forceinline__ void buf_st16(rsrc_t r, uint32_t off, v4u v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CPOL);
}
template <int CPOL>
__device__ __forceinline__ void buf_st8(rsrc_t r, uint32_t off, uint64_t v) {
  typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(v2u_t{uint32_t(v), uint32_t(v >> 32)}, r, off, 0, CPOL);
}
template <int CPOL>
__device__ __forceinline__ void buf_st4(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, CPOL);
}
template <int CPOL>
__device__ __forceinline__ void buf_st1(rsrc_t r, uint32_t off, uint8_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, off, 0, CPOL);
}

__device__ __forceinline__ v4u ld_dev_b128(const void* p) {
  const uint64_t* q = static_cast<const uint64_t*>(p);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v4u{uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi), uint32_t(hi >> 32)};
}

// Whole workgroup: wait until *p >= target.  Returns false when aborted/timed out.
__device__ __forceinline__ bool wg_wait_geq(const uint32_t* p, uint32_t target, uint32_t* hdr,
                                            uint64_t limit) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    int ok = 1;
    if (ld_relaxed(p) < target) {
      const uint64_t t0 = wall_clock64();
      while (ld_relaxed(p) < target) {
        if (ld_relaxed(hdr + kHdrAbort)) { ok = 0; break; }
        if (wall_clock64() - t0 > limit) {
          or_relaxed(hdr + kHdrStatus, MOK_DEV_TIMEOUT);
          __hip_atomic_store(hdr + kHdrAbort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    s_ok = ok;
  }
  __syncthreads();
  const bool ok = s_ok != 0;
  __syncthreads();  // s_ok may be rewritten by the next wait
  return ok;
}

// Whole workgroup: this workgroup's device-scope stores are complete, then *p += v.
__device__ __forceinline__ void wg_signal_add(uint32_t* p, uint32_t v) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) fetch_add_relaxed(p, v);
}

__device__ __forceinline__ bool aborted(const uint32_t* hdr) { return ld_relaxed(hdr + kHdrAbort) != 0; }

// MOK_FLAG_PERTURB: a pseudo-random pause of 0-7 s_sleep(127) (about 4 us each) chosen
// from `salt`, taken by every wave of the workgroup.  It shifts when a signal is
// published or a chunk is taken, and so the interleaving of the workgroups, never what
// is computed.
__device__ __forceinline__ void perturb_pause(bool on, uint32_t salt) {
  if (!on) return;
  uint32_t h = salt * 0x9E3779B1u;
  h ^= h >> 15;
  h *= 0x85EBCA77u;
  h ^= h >> 13;
  for (uint32_t i = 0; i < (h & 7u); ++i) __builtin_amdgcn_s_sleep(127);
}

}  // namespace mok
