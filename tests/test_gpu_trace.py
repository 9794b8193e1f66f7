"""The fused forward's in-kernel trace (MOK_FLAG_TRACE): tracing does not change the
output, every tile ticket has one record from a real workgroup with ordered timestamps,
and the decoded shares of the compute workgroups' time add up to one."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import gen
from mixture_experts_layer_mok_amd import trace as TR
from tests.gpu_util import DevInputs, run_forward, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [gen.CONFIGS[2], gen.small_config(
    "ragged", T=300, D=192, I=192, E=6, k=2, M=96, S=2, comm_cus=8)], ids=lambda c: c.name)
def test_trace_records(cfg):
    say(f"[trace] {cfg.name}")
    d = gen.make_inputs(cfg, seed=9)
    dev = DevInputs(d)
    y0, _ = run_forward(cfg, dev)
    y1, layer = run_forward(cfg, dev, flags=L.MOK_FLAG_TRACE)
    assert layer.status() == 0
    assert torch.equal(y0, y1)
    tab = layer.tables()
    nN1, nN2 = (cfg.I + 127) // 128, (cfg.D + 255) // 256
    tiles = tab["n_mtiles"] * (nN1 + nN2)
    cus = L.mok_device_cus()
    recs, wgs = TR.read(layer, tiles, cus)
    wg = recs[:, 0]
    assert ((wg >= cfg.comm_cus) & (wg < cus)).all()  # tiles run on compute workgroups
    t = recs[:, 2:6].astype(np.int64)
    steps = (t[:, 1:] - t[:, :-1]) & 0xFFFFFFFF
    assert (steps < 10**8).all()  # ticket <= ready <= K loop done <= end, under 1 s apart
    g2 = recs[:, 1] & 1
    assert int((g2 == 0).sum()) == tab["n_mtiles"] * nN1
    assert int((g2 == 1).sum()) == tab["n_mtiles"] * nN2
    assert int(recs[:, 1].max() >> 1) < tab["n_mb"]
    assert (wgs[:cfg.comm_cus, 4] == 1).all() and (wgs[cfg.comm_cus:, 4] == 0).all()
    s = TR.summarize(recs, wgs, cfg.comm_cus)
    say(f"  {s['span_us']} us, compute shares {s['compute_share']}")
    assert abs(sum(s["compute_share"].values()) - 1.0) < 0.02


@pytest.mark.parametrize("precision", [L.MOK_PREC_BF16, L.MOK_PREC_MXFP8], ids=["bf16", "mxfp8"])
def test_unfused_phase_clock(precision):
    """With MOK_FLAG_UNFUSED | MOK_FLAG_TRACE the four launches record per-workgroup start
    and end times: the output is unchanged, every phase has a positive span, and the four
    spans fit inside the forward's own time measured with HIP events."""
    from mixture_experts_layer_mok_amd.layer import MoKLayer
    cfg = gen.CONFIGS[2]
    d = gen.make_inputs(cfg, seed=19)
    dev = DevInputs(d)
    flags = L.MOK_FLAG_UNFUSED
    layers = [MoKLayer(L.desc_from_config(cfg, flags=f, precision=precision))
              for f in (flags, flags | L.MOK_FLAG_TRACE)]
    w = (dev.wg, dev.wu, dev.wd)
    sc = (None, None, None)
    if precision == L.MOK_PREC_MXFP8:
        q = [layers[0].quantize_weights(t) for t in w]
        w, sc = tuple(c for c, _ in q), tuple(s for _, s in q)
    ys = []
    for layer in layers:
        layer.schedule(dev.ids)
        ys.append(layer.forward(dev.x, dev.ids, dev.gates, *w, scales=sc))
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    layers[1].forward(dev.x, dev.ids, dev.gates, *w, scales=sc, y=ys[1])
    e1.record(st)
    torch.cuda.synchronize()
    ph = TR.read_phases(layers[1])
    total_us = e0.elapsed_time(e1) * 1e3
    say(f"[phases] {ph}, events {total_us:.1f} us")
    assert all(v > 0 for v in ph.values())
    assert sum(ph.values()) <= total_us * 1.02 + 5.0
    assert layers[1].status() == 0
