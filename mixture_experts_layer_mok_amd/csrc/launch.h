// Device pointers into the workspace (derived from Layout) and the launchers the C ABI
// calls.  Host and device code share this header.
#pragma once
#include <hip/hip_runtime.h>

#include "layout.h"

namespace mok {

struct Ptrs {
  uint32_t* hdr;
  int32_t* counts;
  int32_t* offsets;
  int32_t* blk;
  int32_t* perm;
  int32_t* pos;
  int4* mt_tab;       // [n_mb_max][mt_max] = (first row, rows, local expert, 0)
  int32_t* mt_cnt;    // [n_mb_max]
  int32_t* tile_base; // [n_mb_max + 1]
  int32_t* mb_start;  // [n_mb_max + 1]: first row of each minibatch; [n_mb] = R
  uint32_t* sync;     // device counters
  uint32_t* bsync;    // backward counters: dH tiles done per m-tile
  uint16_t* obuf;     // [T*k, D] bf16: expert output of pair t*k + j
  uint8_t* ring;      // S slots
  uint8_t* full_x;    // unfused: [T*k, D] dispatched rows (bf16 or MX codes)
  uint8_t* full_xs;   // unfused MX scales
  uint8_t* full_h;    // unfused: [T*k, I] hidden rows
  uint8_t* full_hs;
  uint8_t* wsg;       // MXFP8 weight scales repacked to the tile's stride (when needed)
  uint8_t* wsu;
  uint8_t* wsd;
  // backward
  uint16_t* bab;      // [T*k, 2I] gate / up pre-activations
  uint16_t* bdab;     // [T*k, 2I] their gradients
  uint16_t* dxbuf;    // [T*k, D] per-pair dX contributions (pair-indexed)
  float* dgpart;      // [T*k, nNdh] router-weight gradient partials per dH n-tile
  uint16_t* gh;       // [T*k, I] gate weight times h per routed row (dW_down operand)
  uint32_t* dyb;      // [T*k] byte offset of each routed row's dY row in dy
  uint32_t* xb;       // [T*k] byte offset of each routed row's X row (ring or x)
  uint8_t* dyq;       // MXFP8 backward: dY rows quantised along D, [T*k, D] codes
  uint8_t* dyqs;      //   and [T*k, xs_ld] scales
  uint8_t* dabq;      //   [da | db] rows quantised along I: [T*k, 2I] codes
  uint8_t* dabqs;     //   and [T*k, 2I / 32] scales
  uint8_t* wdts;      //   W_down^T scales repacked to the tile's stride (D % 128 != 0)
  uint32_t* trace;    // MOK_FLAG_TRACE: tile records, then workgroup records; else null
};

inline Ptrs make_ptrs(const Layout& L, void* ws) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  Ptrs P;
  P.hdr = reinterpret_cast<uint32_t*>(b + L.off_hdr);
  P.counts = reinterpret_cast<int32_t*>(b + L.off_counts);
  P.offsets = reinterpret_cast<int32_t*>(b + L.off_offsets);
  P.blk = reinterpret_cast<int32_t*>(b + L.off_blk);
  P.perm = reinterpret_cast<int32_t*>(b + L.off_perm);
  P.pos = reinterpret_cast<int32_t*>(b + L.off_pos);
  P.mt_tab = reinterpret_cast<int4*>(b + L.off_mt_tab);
  P.mt_cnt = reinterpret_cast<int32_t*>(b + L.off_mt_cnt);
  P.tile_base = reinterpret_cast<int32_t*>(b + L.off_tile_base);
  P.mb_start = reinterpret_cast<int32_t*>(b + L.off_mb_start);
  P.sync = reinterpret_cast<uint32_t*>(b + L.off_sync);
  P.bsync = reinterpret_cast<uint32_t*>(b + L.off_sync + L.sync_bwd);
  P.obuf = reinterpret_cast<uint16_t*>(b + L.off_obuf);
  P.ring = b + L.off_ring;
  P.full_x = L.unfused ? b + L.off_full_x : nullptr;
  P.full_xs = L.unfused ? b + L.off_full_xs : nullptr;
  P.full_h = L.unfused ? b + L.off_full_h : nullptr;
  P.full_hs = L.unfused ? b + L.off_full_hs : nullptr;
  P.wsg = L.repack_wg ? b + L.off_wsg : nullptr;
  P.wsu = L.repack_wg ? b + L.off_wsu : nullptr;
  P.wsd = L.repack_wd ? b + L.off_wsd : nullptr;
  auto u16 = [&](size_t off) { return L.save ? reinterpret_cast<uint16_t*>(b + off) : nullptr; };
  P.bab = u16(L.off_bab);
  P.bdab = u16(L.off_bdab);
  P.dxbuf = u16(L.off_dxbuf);
  P.dgpart = L.save ? reinterpret_cast<float*>(b + L.off_dgpart) : nullptr;
  P.gh = u16(L.off_gh);
  P.dyb = L.save ? reinterpret_cast<uint32_t*>(b + L.off_dyb) : nullptr;
  P.xb = L.save ? reinterpret_cast<uint32_t*>(b + L.off_xb) : nullptr;
  P.trace = L.trace ? reinterpret_cast<uint32_t*>(b + L.off_trace) : nullptr;
  const bool mxb = L.mx && L.save;
  P.dyq = mxb ? b + L.off_dyq : nullptr;
  P.dyqs = mxb ? b + L.off_dyqs : nullptr;
  P.dabq = mxb ? b + L.off_dabq : nullptr;
  P.dabqs = mxb ? b + L.off_dabqs : nullptr;
  P.wdts = L.repack_wdt ? b + L.off_wdts : nullptr;
  return P;
}

// Layer inputs of one forward/backward call.
struct FwdArgs {
  const uint16_t* x;
  const int32_t* ids;
  const float* gates;
  const void* wg;
  const void* wu;
  const void* wd;
  const uint8_t* sg;
  const uint8_t* su;
  const uint8_t* sd;
  uint16_t* y;
  int comm_cus;
};

mok_status_t launch_schedule(const Layout& L, const Ptrs& P, const int32_t* ids, hipStream_t st);
mok_status_t launch_forward(const Layout& L, const Ptrs& P, const FwdArgs& a, hipStream_t st);

// Layer inputs and outputs of one backward call.
struct BwdArgs {
  const uint16_t* dy;
  const uint16_t* x;
  const int32_t* ids;
  const float* gates;
  const uint16_t* wg;
  const uint16_t* wu;
  const uint16_t* wd;
  uint16_t* dx;
  float* dg;
  float* dwg;
  float* dwu;
  float* dwd;
  // MXFP8 backward: W_down^T codes [E_loc, I, D] + scales [E_loc, I, D/32], and
  // [W_gate; W_up]^T codes [E_loc, D, 2I] + scales [E_loc, D, 2I/32] (null for bf16)
  const uint8_t* wdt;
  const uint8_t* wdts;
  const uint8_t* wgut;
  const uint8_t* wguts;
};
mok_status_t launch_backward(const Layout& L, const Ptrs& P, const BwdArgs& a, hipStream_t st);
// Weight scale rows of src_ld bytes copied to rows of dst_ld >= src_ld bytes (the MX
// tile's stride of one dword per 128-wide K step), padding with 127 (scale 1).
void launch_mx_repack(const uint8_t* src, int64_t rows, int src_ld, uint8_t* dst, int dst_ld,
                      hipStream_t st);
mok_status_t launch_quantize_mx_t(const uint16_t* src, int64_t batch, int32_t rows, int32_t cols,
                                  uint8_t* codes, int64_t ldc, uint8_t* scales, int64_t lds,
                                  hipStream_t st);
mok_status_t launch_quantize_mx(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes,
                                uint8_t* scales, hipStream_t st);

}  // namespace mok
