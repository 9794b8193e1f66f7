// C ABI of the layer library: argument checks (all before any HIP runtime call),
// workspace layout, and the launches.  Declarations and contracts: include/mok.h.
#include <algorithm>

#include "../../include/mok.h"
#include "launch.h"

using namespace mok;

namespace {

bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

mok_status_t check_ws(const Layout& L, const void* ws, size_t ws_bytes) {
  if (!ws) return MOK_E_NULL;
  if (ws_bytes < L.total) return MOK_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return MOK_E_SHAPE;
  return MOK_OK;
}

}  // namespace

extern "C" {

mok_status_t mok_workspace_size(const mok_desc_t* desc, size_t* bytes) {
  if (!desc || !bytes) return MOK_E_NULL;
  Layout L;
  const mok_status_t s = make_layout(desc, &L);
  if (s != MOK_OK) return s;
  *bytes = L.total;
  return MOK_OK;
}

mok_status_t mok_trace_layout(const mok_desc_t* desc, size_t* offset_bytes, size_t* words) {
  if (!desc || !offset_bytes || !words) return MOK_E_NULL;
  Layout L;
  const mok_status_t s = make_layout(desc, &L);
  if (s != MOK_OK) return s;
  if (!L.trace) return MOK_E_UNSUPPORTED;
  *offset_bytes = L.off_trace;
  *words = L.trace_words;
  return MOK_OK;
}

mok_status_t mok_schedule(const mok_desc_t* desc, const int32_t* topk_ids, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!desc || !topk_ids) return MOK_E_NULL;
  Layout L;
  mok_status_t s = make_layout(desc, &L);
  if (s != MOK_OK) return s;
  if ((s = check_ws(L, ws, ws_bytes)) != MOK_OK) return s;
  return launch_schedule(L, make_ptrs(L, ws), topk_ids, static_cast<hipStream_t>(stream));
}

mok_status_t mok_schedule_tables(const mok_desc_t* desc, const void* ws, size_t ws_bytes,
                                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                                 int32_t* hdr, void* stream) {
  if (!desc) return MOK_E_NULL;
  Layout L;
  mok_status_t s = make_layout(desc, &L);
  if (s != MOK_OK) return s;
  if ((s = check_ws(L, ws, ws_bytes)) != MOK_OK) return s;
  const Ptrs P = make_ptrs(L, const_cast<void*>(ws));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipMemcpyKind k = hipMemcpyDeviceToDevice;
  if (counts && hipMemcpyAsync(counts, P.counts, L.nl * 4, k, st) != hipSuccess) return MOK_E_DEVICE;
  if (offsets && hipMemcpyAsync(offsets, P.offsets, (L.nl + 1) * 4, k, st) != hipSuccess)
    return MOK_E_DEVICE;
  if (perm && hipMemcpyAsync(perm, P.perm, L.TK * 4, k, st) != hipSuccess) return MOK_E_DEVICE;
  if (pos && hipMemcpyAsync(pos, P.pos, L.TK * 4, k, st) != hipSuccess) return MOK_E_DEVICE;
  if (hdr) {
    if (hipMemcpyAsync(hdr, P.hdr + kHdrR, 3 * 4, k, st) != hipSuccess) return MOK_E_DEVICE;
    if (hipMemcpyAsync(hdr + 3, P.hdr + kHdrStatus, 4, k, st) != hipSuccess) return MOK_E_DEVICE;
  }
  return MOK_OK;
}

mok_status_t mok_quantize_mx(const void* src_bf16, int64_t rows, int32_t cols, uint8_t* codes,
                             uint8_t* scales, void* stream) {
  if (!src_bf16 || !codes || !scales) return MOK_E_NULL;
  if (rows < 0 || cols < 32 || cols % 32 != 0) return MOK_E_SHAPE;
  if (!aligned(src_bf16, 16) || !aligned(codes, 16)) return MOK_E_SHAPE;
  return launch_quantize_mx(static_cast<const uint16_t*>(src_bf16), rows, cols, codes, scales,
                            static_cast<hipStream_t>(stream));
}

mok_status_t mok_moe_fwd(const mok_desc_t* desc, const void* x, const int32_t* topk_ids,
                         const float* topk_w, const void* w_gate, const void* w_up,
                         const void* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                         const uint8_t* s_down, void* y, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!desc || !x || !topk_ids || !topk_w || !w_gate || !w_up || !w_down || !y) return MOK_E_NULL;
  Layout L;
  mok_status_t s = make_layout(desc, &L);
  if (s != MOK_OK) return s;
  if ((s = check_ws(L, ws, ws_bytes)) != MOK_OK) return s;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w_gate, 16) || !aligned(w_up, 16) ||
      !aligned(w_down, 16))
    return MOK_E_SHAPE;
  if (L.mx) {
    if (!s_gate || !s_up || !s_down) return MOK_E_NULL;
    if (!aligned(s_gate, 4) || !aligned(s_up, 4) || !aligned(s_down, 4)) return MOK_E_SHAPE;
  } else if (s_gate || s_up || s_down) {
    return MOK_E_SHAPE;
  }
  FwdArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.ids = topk_ids;
  a.gates = topk_w;
  a.wg = w_gate; a.wu = w_up; a.wd = w_down;
  a.sg = s_gate; a.su = s_up; a.sd = s_down;
  a.y = static_cast<uint16_t*>(y);
  a.comm_cus = desc->comm_cus;
  return launch_forward(L, make_ptrs(L, ws), a, static_cast<hipStream_t>(stream));
}

mok_status_t mok_moe_bwd(const mok_desc_t* desc, const void* dy, const void* x,
                         const int32_t* topk_ids, const float* topk_w, const void* w_gate,
                         const void* w_up, const void* w_down, void* dx, float* d_topk_w,
                         float* dw_gate, float* dw_up, float* dw_down, void* ws,
                         size_t ws_bytes, void* stream) {
  if (!desc || !dy || !x || !topk_ids || !topk_w || !w_gate || !w_up || !w_down || !dx ||
      !d_topk_w || !dw_gate || !dw_up || !dw_down)
    return MOK_E_NULL;
  Layout L;
  mok_status_t s = make_layout(desc, &L);
  if (s != MOK_OK) return s;
  if ((s = check_ws(L, ws, ws_bytes)) != MOK_OK) return s;
  if (!L.save || L.mx) return MOK_E_UNSUPPORTED;  // needs a bf16 forward that saved (MXFP8:
                                                  // mok_moe_bwd_mx)
  if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(w_gate, 16) || !aligned(w_up, 16) ||
      !aligned(w_down, 16) || !aligned(dx, 16))
    return MOK_E_SHAPE;
  BwdArgs a;
  a.dy = static_cast<const uint16_t*>(dy);
  a.x = static_cast<const uint16_t*>(x);
  a.ids = topk_ids;
  a.gates = topk_w;
  a.wg = static_cast<const uint16_t*>(w_gate);
  a.wu = static_cast<const uint16_t*>(w_up);
  a.wd = static_cast<const uint16_t*>(w_down);
  a.dx = static_cast<uint16_t*>(dx);
  a.dg = d_topk_w;
  a.dwg = dw_gate;
  a.dwu = dw_up;
  a.dwd = dw_down;
  a.wdt = a.wdts = a.wgut = a.wguts = nullptr;
  return launch_backward(L, make_ptrs(L, ws), a, static_cast<hipStream_t>(stream));
}

mok_status_t mok_moe_bwd_mx(const mok_desc_t* desc, const void* dy, const void* x,
                            const int32_t* topk_ids, const float* topk_w, const uint8_t* wd_t,
                            const uint8_t* wd_t_scales, const uint8_t* wgu_t,
                            const uint8_t* wgu_t_scales, void* dx, float* d_topk_w,
                            float* dw_gate, float* dw_up, float* dw_down, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!desc || !dy || !x || !topk_ids || !topk_w || !wd_t || !wd_t_scales || !wgu_t ||
      !wgu_t_scales || !dx || !d_topk_w || !dw_gate || !dw_up || !dw_down)
    return MOK_E_NULL;
  Layout L;
  mok_status_t s = make_layout(desc, &L);
  if (s != MOK_OK) return s;
  if ((s = check_ws(L, ws, ws_bytes)) != MOK_OK) return s;
  if (!L.save || !L.mx) return MOK_E_UNSUPPORTED;  // needs a MXFP8 forward that saved
  if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(wd_t, 16) || !aligned(wgu_t, 16) ||
      !aligned(dx, 16) || !aligned(wd_t_scales, 4) || !aligned(wgu_t_scales, 4))
    return MOK_E_SHAPE;
  BwdArgs a;
  a.dy = static_cast<const uint16_t*>(dy);
  a.x = static_cast<const uint16_t*>(x);
  a.ids = topk_ids;
  a.gates = topk_w;
  a.wg = a.wu = a.wd = nullptr;
  a.dx = static_cast<uint16_t*>(dx);
  a.dg = d_topk_w;
  a.dwg = dw_gate;
  a.dwu = dw_up;
  a.dwd = dw_down;
  a.wdt = wd_t;
  a.wdts = wd_t_scales;
  a.wgut = wgu_t;
  a.wguts = wgu_t_scales;
  return launch_backward(L, make_ptrs(L, ws), a, static_cast<hipStream_t>(stream));
}

mok_status_t mok_quantize_mx_t(const void* src_bf16, int64_t batch, int32_t rows, int32_t cols,
                               uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                               int64_t ld_scales, void* stream) {
  if (!src_bf16 || !codes || !scales) return MOK_E_NULL;
  if (batch < 0 || rows < 32 || rows % 32 != 0 || cols < 1 || ld_codes < rows ||
      ld_codes % 16 != 0 || ld_scales < rows / 32)
    return MOK_E_SHAPE;
  if (!aligned(src_bf16, 2) || !aligned(codes, 16)) return MOK_E_SHAPE;
  return launch_quantize_mx_t(static_cast<const uint16_t*>(src_bf16), batch, rows, cols, codes,
                              ld_codes, scales, ld_scales, static_cast<hipStream_t>(stream));
}

mok_status_t mok_read_device_status(const void* ws, void* stream, uint32_t* out) {
  if (!ws || !out) return MOK_E_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return MOK_E_DEVICE;
  if (hipMemcpy(out, static_cast<const uint32_t*>(ws) + kHdrStatus, 4, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return MOK_E_DEVICE;
  return MOK_OK;
}

const char* mok_status_string(mok_status_t s) {
  switch (s) {
    case MOK_OK: return "ok";
    case MOK_E_NULL: return "null pointer argument";
    case MOK_E_SHAPE: return "size out of range or inconsistent";
    case MOK_E_UNSUPPORTED: return "unsupported mode";
    case MOK_E_WORKSPACE: return "workspace too small";
    case MOK_E_LAUNCH: return "kernel launch failed";
    case MOK_E_DEVICE: return "device or runtime error";
  }
  return "unknown status";
}

int32_t mok_device_cus(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

}  // extern "C"
