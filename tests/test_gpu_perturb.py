"""Race check of the persistent kernels' handoffs: with MOK_FLAG_PERTURB every workgroup
pauses for a pseudo-random time before each cross-workgroup signal and each drain or
row-sum chunk, which reorders the workgroups.  What is computed does not depend on that
order (every reduction has one owner and a fixed order), so the forward output and every
gradient must be bitwise equal to those of an unperturbed run; a handoff that published
before its data was visible would show up as a difference."""
import pytest
import torch

from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import gen
from mixture_experts_layer_mok_amd.layer import MoKLayer
from tests.gpu_util import DevInputs, say

pytestmark = pytest.mark.gpu

CASES = [
    gen.CONFIGS[1],
    gen.small_config("ragged", T=300, D=192, I=192, E=6, k=2, M=96, S=2, comm_cus=8),
    gen.small_config("zipf", T=512, D=256, I=320, E=8, k=3, M=200, S=1, comm_cus=8, zipf_s=1.2),
    gen.CONFIGS[2],
]


def _fwd_bwd(cfg, dev, flags):
    layer = MoKLayer(L.desc_from_config(cfg, flags=flags | L.MOK_FLAG_SAVE_FOR_BWD))
    layer.schedule(dev.ids)
    y = layer.forward(dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd)
    g = layer.backward(dev.dy, dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd)
    torch.cuda.synchronize()
    assert layer.status() == 0
    return y, g


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_perturbed_interleaving_is_bitwise_neutral(cfg):
    say(f"[perturb] {cfg.name}")
    d = gen.make_inputs(cfg, seed=5, with_dy=True)
    dev = DevInputs(d)
    y0, g0 = _fwd_bwd(cfg, dev, 0)
    y1, g1 = _fwd_bwd(cfg, dev, L.MOK_FLAG_PERTURB)
    assert torch.equal(y0, y1)
    for k in g0:
        assert torch.equal(g0[k], g1[k]), k


def test_perturbed_mxfp8_forward_is_bitwise_neutral():
    cfg = gen.small_config("mx-ragged", T=300, D=192, I=192, E=6, k=2, M=96, S=2, comm_cus=8,
                           precision=L.MOK_PREC_MXFP8)
    say(f"[perturb] {cfg.name}")
    d = gen.make_inputs(cfg, seed=6)
    dev = DevInputs(d)
    ys = []
    for flags in (0, L.MOK_FLAG_PERTURB):
        layer = MoKLayer(L.desc_from_config(cfg, flags=flags))
        sc = []
        w = []
        for t in (dev.wg, dev.wu, dev.wd):
            c, s = layer.quantize_weights(t)
            w.append(c)
            sc.append(s)
        layer.schedule(dev.ids)
        y = layer.forward(dev.x, dev.ids, dev.gates, *w, scales=tuple(sc))
        torch.cuda.synchronize()
        assert layer.status() == 0
        ys.append(y)
    assert torch.equal(ys[0], ys[1])
