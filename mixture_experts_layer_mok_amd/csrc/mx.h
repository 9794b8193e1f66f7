// MXFP8 encoding on the device: OCP MX blocks of 32 elements with an e8m0 shared scale
// and e4m3 elements (bias 7, largest finite 448, no infinities).  The shared exponent
// is the smallest n with amax * 2^-n <= 448 (clamped to [-127, 127], -127 for an
// all-zero block); each element is v * 2^-n rounded to nearest even.  The exponent is
// read from float32 bit patterns and the scaling by 2^-n is exact, so only the final
// conversion rounds.
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

// e4m3 codes of two already-scaled values (byte 0: a, byte 1: b) from gfx950's
// conversion instruction: OCP e4m3, round to nearest even, subnormals kept.  The shared
// exponent bounds every scaled magnitude by 448, the largest finite code, so no value
// reaches the instruction's overflow handling.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
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

// Sum over a 16-lane DPP row, the same butterfly as row16_max; every lane of the row
// ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_sum_step(float v) {
  const float t = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
  return v + t;
}
__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_sum_step<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_sum_step<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_sum_step<0x141>(v);  // row_half_mirror
  return dpp_sum_step<0x140>(v);  // row_mirror
}

// Eight e4m3 codes of v[0..7] * 2^-n, packed little-endian.
__device__ __forceinline__ uint64_t e4m3_pack8(const float (&v)[8], int n) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -n), ldexpf(v[1], -n), 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -n), ldexpf(v[3], -n), lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4], -n), ldexpf(v[5], -n), 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[6], -n), ldexpf(v[7], -n), hi, true);
  return uint64_t(uint32_t(lo)) | (uint64_t(uint32_t(hi)) << 32);
}

// MX quantisation of one pass of a row: lane l holds 8-element chunks c = b + l + 64u
// (u < kQuantBatch) in raw; the 4 lanes of a quad hold one 32-element block, whose
// largest magnitude they share over DPP.  Codes and scales go through row-length buffer
// resources (codes: D bytes, scales: D / 32 bytes), so chunks past the row's end are
// quantised from zeros and their stores dropped: every lane stays active for the DPP
// steps.
constexpr int kQuantBatch = 16;

template <int kPol>
__device__ __forceinline__ void quant_store_pass(const v4u (&raw)[kQuantBatch], rsrc_t rc,
                                                 rsrc_t rsc, uint32_t b) {
  const uint32_t lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kQuantBatch; ++u) {
    const uint32_t c = b + lane + 64 * u;
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
    buf_st8<kPol>(rc, c * 8, e4m3_pack8(v, n));
    if ((lane & 3) == 0) buf_st1<kPol>(rsc, c >> 2, uint8_t(n + 127));
  }
}

// One wave quantises one row of D bf16 values (D a multiple of 32) into MX: codes[0..D)
// and scales[0..D/32), kQuantBatch chunks per lane loaded before any is quantised.  With
// kCoherent the outputs are written at device scope (handoff data); kLdPol is the cache
// policy of the source loads (kCpolDev for rows written by other workgroups of the same
// launch).
template <bool kCoherent, int kLdPol = kCpolPlain>
__device__ __forceinline__ void wave_quant_row(uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales,
                                               const uint16_t* __restrict__ src, int D) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t nch = uint32_t(D) >> 3;
  const rsrc_t rs = row_rsrc(src, uint32_t(D) * 2);
  const rsrc_t rc = row_rsrc(codes, uint32_t(D));
  const rsrc_t rsc = row_rsrc(scales, uint32_t(D) >> 5);
  for (uint32_t b = 0; b < nch; b += 64 * kQuantBatch) {
    v4u raw[kQuantBatch];
#pragma unroll
    for (int u = 0; u < kQuantBatch; ++u)
      raw[u] = buf_ld16<kLdPol>(rs, (b + lane + 64 * u) * 16);
    quant_store_pass<kCoherent ? kCpolDev : kCpolPlain>(raw, rc, rsc, b);
  }
}

}  // namespace mok
