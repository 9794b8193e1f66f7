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
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(v4u v) { return __builtin_bit_cast(bf16x8_t, v); }

// 32x32x16 bf16 MFMA: C[32x32] += A[32x16] * B[16x32].  Lane l supplies A row (l%32),
// K elements 8*(l/32) .. +8, and B column (l%32), the same K elements.  Lane l receives
// C column (l%32), rows 8*(v/4) + 4*(l/32) + (v%4) for v = 0..15.
__device__ __forceinline__ f32x16_t mfma32x32x16(v4u a, v4u b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ------------------------------------------------------------------------------------
// Cross-workgroup handoff.  Producers: every thread fences its own stores at agent
// scope (so they leave this XCD's L2), the workgroup meets at a barrier, and one
// thread publishes with an agent-scope release add.  Consumers: one thread waits with
// agent-scope acquire loads, then the workgroup meets and every thread acquires.
// Waits are bounded: on expiry the waiter sets MOK_DEV_TIMEOUT and the abort word,
// and every loop of the persistent kernels exits once the abort word is set.
// ------------------------------------------------------------------------------------
constexpr uint64_t kWaitTicks = 200000000ull;  // 2 s of the 100 MHz constant clock

__device__ __forceinline__ uint32_t ld_acquire(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_release(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void or_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whole workgroup: wait until *p >= target.  Returns false when aborted/timed out.
__device__ __forceinline__ bool wg_wait_geq(const uint32_t* p, uint32_t target, uint32_t* hdr) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    int ok = 1;
    if (ld_acquire(p) < target) {
      const uint64_t t0 = wall_clock64();
      while (ld_acquire(p) < target) {
        if (ld_relaxed(hdr + kHdrAbort)) { ok = 0; break; }
        if (wall_clock64() - t0 > kWaitTicks) {
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
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();  // s_ok may be rewritten by the next wait
  return ok;
}

// Whole workgroup: publish this workgroup's stores, then *p += v.
__device__ __forceinline__ void wg_signal_add(uint32_t* p, uint32_t v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) add_release(p, v);
}

__device__ __forceinline__ bool aborted(const uint32_t* hdr) { return ld_relaxed(hdr + kHdrAbort) != 0; }

}  // namespace mok
