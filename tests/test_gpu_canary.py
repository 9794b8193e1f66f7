"""Canary check of every buffer the layer writes: the workspace and each output are carved
out of a larger allocation whose bytes before and after them hold a known pattern.  After
schedule, forward and backward the patterns must be intact, so no kernel wrote outside
its buffers (the per-access bounds of the buffer resources are what this checks), and a
second run on fresh buffers gives the same results bit for bit."""
import pytest
import torch

from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import gen
from tests.gpu_util import DevInputs, say

pytestmark = pytest.mark.gpu

GUARD = 1 << 16  # bytes of pattern on each side
PAT = 0xA5


class Guarded:
    """A device buffer of `nbytes` with GUARD pattern bytes on each side."""

    def __init__(self, nbytes: int, dev):
        self.raw = torch.full((nbytes + 2 * GUARD,), PAT, dtype=torch.uint8, device=dev)
        self.n = nbytes

    def view(self, dtype, shape):
        return self.raw[GUARD:GUARD + self.n].view(dtype).view(shape)

    def intact(self) -> bool:
        return bool((self.raw[:GUARD] == PAT).all()) and bool((self.raw[GUARD + self.n:] == PAT).all())


def _run(cfg, dev, flags):
    desc = L.desc_from_config(cfg, flags=flags)
    wsb = L.mok_workspace_size(desc)
    T, D, I, k, nl = cfg.T, cfg.D, cfg.I, cfg.k, cfg.n_local
    def mk(n):
        return Guarded(n, dev.x.device)

    bufs = {"ws": mk(wsb), "y": mk(T * D * 2)}
    ws = bufs["ws"].view(torch.uint8, (wsb,))
    y = bufs["y"].view(torch.bfloat16, (T, D))
    L.mok_schedule(desc, dev.ids, ws, wsb)
    L.mok_moe_fwd(desc, dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd, None, None, None, y,
                  ws, wsb)
    out = {"y": y}
    if flags & L.MOK_FLAG_SAVE_FOR_BWD:
        for name, n in (("dx", T * D * 2), ("dg", T * k * 4), ("dwg", nl * I * D * 4),
                        ("dwu", nl * I * D * 4), ("dwd", nl * D * I * 4)):
            bufs[name] = mk(n)
        out["dx"] = bufs["dx"].view(torch.bfloat16, (T, D))
        out["dg"] = bufs["dg"].view(torch.float32, (T, k))
        out["dwg"] = bufs["dwg"].view(torch.float32, (nl, I, D))
        out["dwu"] = bufs["dwu"].view(torch.float32, (nl, I, D))
        out["dwd"] = bufs["dwd"].view(torch.float32, (nl, D, I))
        L.mok_moe_bwd(desc, dev.dy, dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd, out["dx"],
                      out["dg"], out["dwg"], out["dwu"], out["dwd"], ws, wsb)
    torch.cuda.synchronize()
    assert L.mok_read_device_status(ws) == 0
    return bufs, out


@pytest.mark.parametrize("cfg", [
    gen.small_config("ragged", T=300, D=192, I=192, E=6, k=2, M=96, S=2, comm_cus=8),
    gen.small_config("e0", T=257, D=128, I=128, E=16, k=4, e0=5, E_loc=6, M=64, S=3, comm_cus=16),
    gen.CONFIGS[2],
], ids=lambda c: c.name)
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_no_writes_outside_buffers(cfg, fused):
    say(f"[canary] {cfg.name} fused={fused}")
    d = gen.make_inputs(cfg, seed=21, with_dy=True)
    dev = DevInputs(d)
    flags = L.MOK_FLAG_SAVE_FOR_BWD | (0 if fused else L.MOK_FLAG_UNFUSED)
    bufs, out = _run(cfg, dev, flags)
    for name, b in bufs.items():
        assert b.intact(), f"pattern around {name} overwritten"
    _, ref = _run(cfg, dev, flags)  # a second run on fresh buffers
    for name in out:
        assert torch.equal(out[name], ref[name]), name
