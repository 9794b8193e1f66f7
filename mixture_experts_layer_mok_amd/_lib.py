"""ctypes binding of libmok.so (the C ABI declared in include/mok.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
Functions keep the C names.  Tensor arguments may be torch tensors (their data_ptr is
passed) or raw integer device addresses; streams may be torch streams, raw handles or
None (the current torch stream when torch is importable, else the default stream).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmok.so")

MOK_OK = 0
MOK_E_NULL = 1
MOK_E_SHAPE = 2
MOK_E_UNSUPPORTED = 3
MOK_E_WORKSPACE = 4
MOK_E_LAUNCH = 5
MOK_E_DEVICE = 6

MOK_PREC_BF16 = 0
MOK_PREC_MXFP8 = 1
MOK_FLAG_SAVE_FOR_BWD = 0x1
MOK_FLAG_UNFUSED = 0x2
MOK_FLAG_SHORT_WAITS = 0x4
MOK_FLAG_PERTURB = 0x8
MOK_FLAG_TRACE = 0x10
MOK_FLAG_OVERLAP_NEXT = 0x20
MOK_TRACE_MAX_WORKGROUPS = 1024
MOK_DEV_BAD_ID = 0x1
MOK_DEV_TIMEOUT = 0x2

# exported entry points, in header order
EXPORTS = (
    "mok_workspace_size", "mok_schedule", "mok_schedule_tables", "mok_quantize_mx",
    "mok_moe_fwd", "mok_moe_bwd", "mok_read_device_status", "mok_status_string",
    "mok_device_cus", "mok_trace_layout", "mok_moe_fwd_noalloc", "mok_quantize_mx_t",
    "mok_moe_bwd_mx",
)


class mok_desc_t(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("expert_begin", ctypes.c_int32),
        ("num_local_experts", ctypes.c_int32),
        ("minibatch_rows", ctypes.c_int32),
        ("ring_slots", ctypes.c_int32),
        ("comm_cus", ctypes.c_int32),
        ("precision", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class MokError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {code} ({status_string(code)})")


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m mixture_experts_layer_mok_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32p, u8p, f32p = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p)
    D = ctypes.POINTER(mok_desc_t)
    sig = {
        "mok_workspace_size": (ctypes.c_int, [D, ctypes.POINTER(ctypes.c_size_t)]),
        "mok_schedule": (ctypes.c_int, [D, i32p, vp, sz, vp]),
        "mok_schedule_tables": (ctypes.c_int, [D, vp, sz, i32p, i32p, i32p, i32p, i32p, vp]),
        "mok_quantize_mx": (ctypes.c_int, [vp, ctypes.c_int64, ctypes.c_int32, u8p, u8p, vp]),
        "mok_moe_fwd": (ctypes.c_int, [D, vp, i32p, f32p, vp, vp, vp, u8p, u8p, u8p, vp, vp, sz,
                                       vp]),
        "mok_moe_bwd": (ctypes.c_int, [D, vp, vp, i32p, f32p, vp, vp, vp, vp, f32p, f32p, f32p,
                                       f32p, vp, sz, vp]),
        "mok_read_device_status": (ctypes.c_int, [vp, vp, ctypes.POINTER(ctypes.c_uint32)]),
        "mok_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "mok_device_cus": (ctypes.c_int32, []),
        "mok_trace_layout": (ctypes.c_int, [D, ctypes.POINTER(ctypes.c_size_t),
                                            ctypes.POINTER(ctypes.c_size_t)]),
        "mok_moe_fwd_noalloc": (ctypes.c_int, [D, vp, i32p, f32p, vp, vp, vp, u8p, u8p, u8p, vp,
                                               vp, vp]),
        "mok_quantize_mx_t": (ctypes.c_int, [vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             u8p, ctypes.c_int64, u8p, ctypes.c_int64, vp]),
        "mok_moe_bwd_mx": (ctypes.c_int, [D, vp, vp, i32p, f32p, u8p, u8p, u8p, u8p, vp, f32p,
                                          f32p, f32p, f32p, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(code: int) -> str:
    try:
        return load().mok_status_string(int(code)).decode()
    except Exception:  # pragma: no cover
        return "?"


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except Exception:  # pragma: no cover
            pass
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn: str, code: int) -> None:
    if code != MOK_OK:
        raise MokError(fn, code)


def make_desc(T, D, I, E, k, *, e0=0, E_loc=0, M=32, S=2, comm_cus=32, precision=0,
              flags=0) -> mok_desc_t:
    return mok_desc_t(T, D, I, E, k, e0, E_loc if E_loc > 0 else E, M, S, comm_cus, precision,
                      flags)


def desc_from_config(cfg, *, flags=0, comm_cus=None, M=None, S=None, precision=None):
    return make_desc(cfg.T, cfg.D, cfg.I, cfg.E, cfg.k, e0=cfg.e0, E_loc=cfg.n_local,
                     M=cfg.M if M is None else M, S=cfg.S if S is None else S,
                     comm_cus=cfg.comm_cus if comm_cus is None else comm_cus,
                     precision=cfg.precision if precision is None else precision, flags=flags)


# ---------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------
def mok_workspace_size(desc: mok_desc_t) -> int:
    n = ctypes.c_size_t(0)
    _check("mok_workspace_size", load().mok_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def mok_schedule(desc, topk_ids, ws, ws_bytes=None, stream=None) -> None:
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("mok_schedule", load().mok_schedule(ctypes.byref(desc), _ptr(topk_ids), _ptr(ws),
                                               ws_bytes, _stream(stream)))


def mok_schedule_tables(desc, ws, counts=None, offsets=None, perm=None, pos=None, hdr=None,
                        ws_bytes=None, stream=None) -> None:
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("mok_schedule_tables", load().mok_schedule_tables(
        ctypes.byref(desc), _ptr(ws), ws_bytes, _ptr(counts), _ptr(offsets), _ptr(perm),
        _ptr(pos), _ptr(hdr), _stream(stream)))


def mok_quantize_mx(src, rows, cols, codes, scales, stream=None) -> None:
    _check("mok_quantize_mx", load().mok_quantize_mx(_ptr(src), int(rows), int(cols),
                                                     _ptr(codes), _ptr(scales), _stream(stream)))


def mok_moe_fwd(desc, x, topk_ids, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, y, ws,
                ws_bytes=None, stream=None) -> None:
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("mok_moe_fwd", load().mok_moe_fwd(
        ctypes.byref(desc), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(y), _ptr(ws), ws_bytes,
        _stream(stream)))


def mok_moe_bwd(desc, dy, x, topk_ids, topk_w, w_gate, w_up, w_down, dx, d_topk_w, dw_gate,
                dw_up, dw_down, ws, ws_bytes=None, stream=None) -> None:
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("mok_moe_bwd", load().mok_moe_bwd(
        ctypes.byref(desc), _ptr(dy), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(dx), _ptr(d_topk_w), _ptr(dw_gate), _ptr(dw_up),
        _ptr(dw_down), _ptr(ws), ws_bytes, _stream(stream)))


def mok_moe_fwd_noalloc(desc, x, topk_ids, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down,
                        y, dev_status=None, stream=None) -> None:
    _check("mok_moe_fwd_noalloc", load().mok_moe_fwd_noalloc(
        ctypes.byref(desc), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(y), _ptr(dev_status),
        _stream(stream)))


def mok_quantize_mx_t(src, batch, rows, cols, codes, ld_codes, scales, ld_scales,
                      stream=None) -> None:
    _check("mok_quantize_mx_t", load().mok_quantize_mx_t(
        _ptr(src), int(batch), int(rows), int(cols), _ptr(codes), int(ld_codes), _ptr(scales),
        int(ld_scales), _stream(stream)))


def mok_moe_bwd_mx(desc, dy, x, topk_ids, topk_w, wd_t, wd_t_scales, wgu_t, wgu_t_scales, dx,
                   d_topk_w, dw_gate, dw_up, dw_down, ws, ws_bytes=None, stream=None) -> None:
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("mok_moe_bwd_mx", load().mok_moe_bwd_mx(
        ctypes.byref(desc), _ptr(dy), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(wd_t),
        _ptr(wd_t_scales), _ptr(wgu_t), _ptr(wgu_t_scales), _ptr(dx), _ptr(d_topk_w),
        _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _ptr(ws), ws_bytes, _stream(stream)))


def mok_read_device_status(ws, stream=None) -> int:
    out = ctypes.c_uint32(0)
    _check("mok_read_device_status", load().mok_read_device_status(_ptr(ws), _stream(stream),
                                                                   ctypes.byref(out)))
    return out.value


def mok_device_cus() -> int:
    return int(load().mok_device_cus())


def mok_trace_layout(desc: mok_desc_t) -> tuple[int, int]:
    """(byte offset, uint32 words) of the trace region of a MOK_FLAG_TRACE workspace."""
    off, words = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("mok_trace_layout", load().mok_trace_layout(ctypes.byref(desc), ctypes.byref(off),
                                                       ctypes.byref(words)))
    return off.value, words.value
