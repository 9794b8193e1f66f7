"""C ABI checks that need no GPU: the library loads, exports every entry point the header
declares, and rejects bad arguments synchronously (before any HIP runtime call)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_mok_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # never dereferenced: every call below fails its host checks first


def _header_functions():
    src = open(os.path.join(ROOT, "include", "mok.h")).read()
    return re.findall(r"^\s*(?:mok_status_t|const char\*|int32_t)\s+(mok_\w+)\(", src, re.M)


def test_library_exports_every_declared_function():
    lib = L.load()
    names = _header_functions()
    assert sorted(names) == sorted(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(7):
        assert L.status_string(code)
    assert L.status_string(L.MOK_E_WORKSPACE) == "workspace too small"


def _desc(**kw):
    base = dict(T=128, D=128, I=64, E=4, k=2, M=32, S=2, comm_cus=8)
    base.update(kw)
    T, D, I, E, k = (base.pop(x) for x in ("T", "D", "I", "E", "k"))
    return L.make_desc(T, D, I, E, k, **base)


def _ws_code(desc):
    n = ctypes.c_size_t(0)
    return L.load().mok_workspace_size(ctypes.byref(desc), ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,code", [
    (dict(D=100), L.MOK_E_SHAPE), (dict(D=0), L.MOK_E_SHAPE), (dict(I=96), L.MOK_E_SHAPE),
    (dict(k=5), L.MOK_E_SHAPE), (dict(k=0), L.MOK_E_SHAPE), (dict(E_loc=5), L.MOK_E_SHAPE),
    (dict(e0=3, E_loc=2), L.MOK_E_SHAPE), (dict(M=0), L.MOK_E_SHAPE), (dict(S=0), L.MOK_E_SHAPE),
    (dict(comm_cus=0), L.MOK_E_SHAPE), (dict(T=0), L.MOK_E_SHAPE),
    (dict(precision=7), L.MOK_E_UNSUPPORTED), (dict(flags=0x80), L.MOK_E_UNSUPPORTED),
])
def test_workspace_size_rejects(kw, code):
    assert _ws_code(_desc(**kw))[0] == code


def test_workspace_size_null_and_growth():
    lib = L.load()
    n = ctypes.c_size_t(0)
    assert lib.mok_workspace_size(None, ctypes.byref(n)) == L.MOK_E_NULL
    assert lib.mok_workspace_size(ctypes.byref(_desc()), None) == L.MOK_E_NULL
    c0, b0 = _ws_code(_desc())
    c1, b1 = _ws_code(_desc(S=4))
    c2, b2 = _ws_code(_desc(flags=L.MOK_FLAG_UNFUSED))
    c3, b3 = _ws_code(_desc(flags=L.MOK_FLAG_SAVE_FOR_BWD))
    c4, b4 = _ws_code(_desc(flags=L.MOK_FLAG_SHORT_WAITS))
    assert c0 == c1 == c2 == c3 == c4 == L.MOK_OK
    assert b0 < b1 and b0 < b2 and b0 < b3 and b0 % 256 == 0
    assert b4 == b0  # the wait limit needs no memory
    # the result buffer alone is T*k*D bf16
    assert b0 > 128 * 2 * 128 * 2


def test_entry_points_fail_before_touching_memory():
    lib = L.load()
    d = _desc()
    ok, need = _ws_code(d)
    assert ok == L.MOK_OK
    small = need - 256
    dp = ctypes.byref(d)
    assert lib.mok_schedule(dp, None, FAKE, need, None) == L.MOK_E_NULL
    assert lib.mok_schedule(dp, FAKE, None, need, None) == L.MOK_E_NULL
    assert lib.mok_schedule(dp, FAKE, FAKE, small, None) == L.MOK_E_WORKSPACE
    assert lib.mok_schedule(dp, FAKE, FAKE + 8, need, None) == L.MOK_E_SHAPE  # misaligned
    args = [FAKE] * 6
    assert lib.mok_moe_fwd(dp, *args, None, None, None, FAKE, FAKE, small, None) == \
        L.MOK_E_WORKSPACE
    assert lib.mok_moe_fwd(dp, None, *args[1:], None, None, None, FAKE, FAKE, need, None) == \
        L.MOK_E_NULL
    assert lib.mok_moe_fwd(dp, *args, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == L.MOK_E_SHAPE
    dmx = _desc(precision=1)
    ok, need_mx = _ws_code(dmx)
    assert lib.mok_moe_fwd(ctypes.byref(dmx), *args, None, None, None, FAKE, FAKE, need_mx,
                           None) == L.MOK_E_NULL
    # misaligned operands are refused before anything is enqueued
    assert lib.mok_moe_fwd(dp, FAKE + 2, *args[1:], None, None, None, FAKE, FAKE, need,
                           None) == L.MOK_E_SHAPE
    assert lib.mok_moe_fwd(dp, *args, None, None, None, FAKE + 8, FAKE, need, None) == \
        L.MOK_E_SHAPE
    assert lib.mok_moe_fwd(ctypes.byref(dmx), *args, FAKE + 1, FAKE, FAKE, FAKE, FAKE, need_mx,
                           None) == L.MOK_E_SHAPE
    assert lib.mok_quantize_mx(FAKE + 4, 4, 64, FAKE, FAKE, None) == L.MOK_E_SHAPE
    assert lib.mok_quantize_mx(FAKE, 4, 48, FAKE, FAKE, None) == L.MOK_E_SHAPE
    assert lib.mok_quantize_mx(None, 4, 64, FAKE, FAKE, None) == L.MOK_E_NULL
    assert lib.mok_read_device_status(None, None, None) == L.MOK_E_NULL
    assert lib.mok_schedule_tables(dp, FAKE, small, None, None, None, None, None, None) == \
        L.MOK_E_WORKSPACE
    bw = [FAKE] * 7
    assert lib.mok_moe_bwd(dp, *bw, None, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == L.MOK_E_NULL
    assert lib.mok_moe_bwd(dp, *bw, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, small, None) == \
        L.MOK_E_WORKSPACE
    # the MXFP8 backward: its own entry point, on a MXFP8 workspace that saved
    dmxs = _desc(precision=1, flags=L.MOK_FLAG_SAVE_FOR_BWD)
    ok, need_mxs = _ws_code(dmxs)
    assert ok == L.MOK_OK and need_mxs > _ws_code(dmx)[1]
    bmx = [FAKE] * 9
    assert lib.mok_moe_bwd(ctypes.byref(dmxs), *bw, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need_mxs,
                           None) == L.MOK_E_UNSUPPORTED
    assert lib.mok_moe_bwd_mx(dp, *bmx, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == \
        L.MOK_E_UNSUPPORTED
    assert lib.mok_moe_bwd_mx(ctypes.byref(dmxs), *bmx, FAKE, FAKE, FAKE, None, FAKE, need_mxs,
                              None) == L.MOK_E_NULL
    assert lib.mok_moe_bwd_mx(ctypes.byref(dmxs), *bmx, FAKE, FAKE, FAKE, FAKE, FAKE,
                              need_mxs - 256, None) == L.MOK_E_WORKSPACE
    assert lib.mok_moe_bwd_mx(ctypes.byref(dmxs), *bmx[:7], FAKE + 1, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, need_mxs, None) == L.MOK_E_SHAPE
    # the transposing quantiser's shape checks
    assert lib.mok_quantize_mx_t(FAKE, 2, 48, 64, FAKE, 48, FAKE, 2, None) == L.MOK_E_SHAPE
    assert lib.mok_quantize_mx_t(FAKE, 2, 64, 64, FAKE, 72, FAKE, 2, None) == L.MOK_E_SHAPE
    assert lib.mok_quantize_mx_t(FAKE, 2, 64, 64, FAKE, 64, FAKE, 1, None) == L.MOK_E_SHAPE
    assert lib.mok_quantize_mx_t(FAKE, 2, 64, 64, FAKE + 8, 64, FAKE, 2, None) == L.MOK_E_SHAPE
    assert lib.mok_quantize_mx_t(None, 2, 64, 64, FAKE, 64, FAKE, 2, None) == L.MOK_E_NULL


def test_trace_layout():
    """The trace region exists only with MOK_FLAG_TRACE, lies inside the workspace, and
    holds 8 words per possible forward tile plus 8 per workgroup."""
    with pytest.raises(L.MokError) as e:
        L.mok_trace_layout(_desc())
    assert e.value.code == L.MOK_E_UNSUPPORTED
    d = _desc(flags=L.MOK_FLAG_TRACE)
    off, words = L.mok_trace_layout(d)
    total = L.mok_workspace_size(d)
    assert off % 256 == 0 and off + words * 4 <= total
    assert total > L.mok_workspace_size(_desc())
    assert words > L.MOK_TRACE_MAX_WORKGROUPS * 8 and (words - L.MOK_TRACE_MAX_WORKGROUPS * 8) % 8 == 0
