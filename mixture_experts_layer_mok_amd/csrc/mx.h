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

// One lane quantises one 32-element block of bf16: src points at the block, codes at
// its 32 output bytes, returns the scale byte.
__device__ __forceinline__ uint8_t mx_block_bf16(const uint16_t* __restrict__ src,
                                                 uint8_t* __restrict__ codes) {
  const v4u* s = reinterpret_cast<const v4u*>(src);
  v4u v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = s[i];
  float f[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[i * 8 + 2 * j] = bf16_to_f32(uint16_t(w[j] & 0xFFFF));
      f[i * 8 + 2 * j + 1] = bf16_to_f32(uint16_t(w[j] >> 16));
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
  const int n = mx_shared_exp(amax);
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t wd = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) wd |= e4m3_rne(ldexpf(f[i * 4 + j], -n)) << (8 * j);
    out[i] = wd;
  }
  v4u* d = reinterpret_cast<v4u*>(codes);
  d[0] = v4u{out[0], out[1], out[2], out[3]};
  d[1] = v4u{out[4], out[5], out[6], out[7]};
  return uint8_t(n + 127);
}

}  // namespace mok
