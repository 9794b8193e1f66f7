// Schedule + forward with the workspace in a static device-memory area, for callers that
// cannot allocate device memory.  The kernels are the ones mok_schedule and mok_moe_fwd
// launch; only the workspace's address differs.
//
// `scratch` is a file-scope device array: each GPU that runs this code holds its own copy
// from the first call on that GPU until the process ends.  In host code its name is only
// a host-side stand-in, so its device address is looked up once per device (with that
// device current) and kept; kernels receive that address, never the name.
#include <mutex>

#include "../../include/mok.h"
#include "launch.h"

using namespace mok;

namespace {

static_assert(MOK_NOALLOC_SCRATCH_BYTES % 256 == 0, "the area keeps the workspace's alignment");
static __device__ __align__(256) uint8_t scratch[MOK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The area's device address on the current device (looked up on the first call there).
mok_status_t scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOK_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOK_E_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOK_OK;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }
bool aligned4(const void* p) { return reinterpret_cast<uintptr_t>(p) % 4 == 0; }

}  // namespace

extern "C" mok_status_t mok_moe_fwd_noalloc(const mok_desc_t* desc, const void* x,
                                            const int32_t* topk_ids, const float* topk_w,
                                            const void* w_gate, const void* w_up,
                                            const void* w_down, const uint8_t* s_gate,
                                            const uint8_t* s_up, const uint8_t* s_down, void* y,
                                            uint32_t* dev_status, void* stream) {
  if (!desc || !x || !topk_ids || !topk_w || !w_gate || !w_up || !w_down || !y) return MOK_E_NULL;
  Layout L;
  mok_status_t s = make_layout(desc, &L);
  if (s != MOK_OK) return s;
  if (L.save || L.trace) return MOK_E_UNSUPPORTED;  // their results stay in the workspace
  if (L.total > MOK_NOALLOC_SCRATCH_BYTES) return MOK_E_WORKSPACE;
  if (!aligned16(x) || !aligned16(y) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down))
    return MOK_E_SHAPE;
  if (L.mx) {
    if (!s_gate || !s_up || !s_down) return MOK_E_NULL;
    if (!aligned4(s_gate) || !aligned4(s_up) || !aligned4(s_down)) return MOK_E_SHAPE;
  } else if (s_gate || s_up || s_down) {
    return MOK_E_SHAPE;
  }
  if (dev_status && !aligned4(dev_status)) return MOK_E_SHAPE;
  void* ws = nullptr;
  if ((s = scratch_on_current_device(&ws)) != MOK_OK) return s;
  const Ptrs P = make_ptrs(L, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = launch_schedule(L, P, topk_ids, st)) != MOK_OK) return s;
  FwdArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.ids = topk_ids;
  a.gates = topk_w;
  a.wg = w_gate; a.wu = w_up; a.wd = w_down;
  a.sg = s_gate; a.su = s_up; a.sd = s_down;
  a.y = static_cast<uint16_t*>(y);
  a.comm_cus = desc->comm_cus;
  if ((s = launch_forward(L, P, a, st)) != MOK_OK) return s;
  if (dev_status &&
      hipMemcpyAsync(dev_status, P.hdr + kHdrStatus, 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return MOK_E_LAUNCH;
  return MOK_OK;
}
