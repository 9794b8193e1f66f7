// MXFP8 encoding on the device: OCP MX blocks of 32 elements with an e8m0 shared scale
// and e4m3 elements (bias 7, largest finite 448, no infinities).  The shared exponent
// is the smallest n with amax * 2^-n <= 448 (clamped to [-127, 127], -127 for an
// all-zero block); each element is v * 2^-n rounded to nearest even, saturating.
// Implemented on float32 bit patterns; every step after reading the float32 value is
// exact.
#pragma once
#include "device.h"

namespace mok {

// Shared exponent of a block from its largest magnitude (float32).
__device__ __forceinline__ int mx_shared_exp(float amax) {
  const uint32_t b = __float_as_uint(amax) & 0x7FFFFFFFu;
  const int ef = int(b >> 23);
  if (ef == 0) return -127;  // zero or float32-subnormal: below 448 * 2^-127
  const int E = ef - 127;
  const int n = E - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);  // mantissa above 1.75
  return max(-127, min(127, n));
}

// e4m3 code of x (already scaled), round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;        // |x| >= 448
  if (a < 0x3C800000u) {                             // |x| < 2^-6: multiples of 2^-9
    const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | uint32_t(q);                       // q == 8 is the smallest normal
  }
  const uint32_t e = (a >> 23) - 127u + 7u;         // 1..15
  const uint32_t m = a & 0x7FFFFFu;
  uint32_t q = m >> 20;
  const uint32_t rem = m & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
  uint32_t code = (e << 3) + q;                      // a mantissa carry bumps the exponent
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

// Maximum over each group of 4 (quad) or 16 (DPP row) consecutive lanes, with DPP lane
// moves: quad_perm [1,0,3,2] and [2,3,0,1], then row_half_mirror and row_mirror, which
// pair quad 0 with quad 1 and the two halves of a row.  Every lane of a group must be
// active.
template <int CTRL>
__device__ __forceinline__ float dpp_max_step(float v) {
  const float t = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
  return fmaxf(v, t);
}
__device__ __forceinline__ float quad_max(float v) {
  v = dpp_max_step<0xB1>(v);  // quad_perm [1,0,3,2]
  return dpp_max_step<0x4E>(v);  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float row16_max(float v) {
  v = quad_max(v);
  v = dpp_max_step<0x141>(v);  // row_half_mirror
  return dpp_max_step<0x140>(v);  // row_mirror
}

// Eight e4m3 codes of v[0..7] * 2^-n, packed little-endian.
__device__ __forceinline__ uint64_t e4m3_pack8(const float (&v)[8], int n) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo |= e4m3_rne(ldexpf(v[j], -n)) << (8 * j);
    hi |= e4m3_rne(ldexpf(v[4 + j], -n)) << (8 * j);
  }
  return uint64_t(lo) | (uint64_t(hi) << 32);
}

// One wave quantises one row of D bf16 values (D a multiple of 32) into MX: codes[0..D)
// and scales[0..D/32).  Lane l handles 8-element chunks c = l, l + 64, ..., loading 8 of
// them before quantising any; the 4 lanes of a quad hold one 32-element block, whose
// largest magnitude they share over DPP (a quad is wholly inside or outside the row,
// since D / 8 is a multiple of 4).  With kCoherent the outputs are written at device
// scope (handoff data).
template <bool kCoherent>
__device__ __forceinline__ void wave_quant_row(uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales,
                                               const uint16_t* __restrict__ src, int D) {
  constexpr int kB = 8;
  const int lane = threadIdx.x & 63;
  const int nch = D >> 3;
  const v4u* s = reinterpret_cast<const v4u*>(src);
  for (int c0 = lane; c0 < nch; c0 += 64 * kB) {
    v4u raw[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (c0 + 64 * u < nch) raw[u] = s[c0 + 64 * u];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int c = c0 + 64 * u;
      if (c < nch) {
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
        float v[8];
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = bf16_to_f32(uint16_t(w[j] & 0xFFFF));
          v[2 * j + 1] = bf16_to_f32(uint16_t(w[j] >> 16));
          amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
        }
        amax = quad_max(amax);
        const int n = mx_shared_exp(amax);
        const uint64_t packed = e4m3_pack8(v, n);
        if (kCoherent) st_dev_u64(codes + int64_t(c) * 8, packed);
        else *reinterpret_cast<uint64_t*>(codes + int64_t(c) * 8) = packed;
        if ((lane & 3) == 0) {
          if (kCoherent) st_dev_u8(scales + (c >> 2), uint8_t(n + 127));
          else scales[c >> 2] = uint8_t(n + 127);
        }
      }
    }
  }
}

}  // namespace mok
