"""Macrobatch interleave (MOK_FLAG_OVERLAP_NEXT): successive forwards on two workspaces
and two streams, each one's final combine overlapping the next one's dispatch, give the
same outputs bit for bit as separate calls, in bf16 and MXFP8; the flag alone changes
no output."""
import pytest
import torch

from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import gen
from mixture_experts_layer_mok_amd.layer import MoKLayer, forward_macrobatches
from tests.gpu_util import DevInputs, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("precision", [L.MOK_PREC_BF16, L.MOK_PREC_MXFP8], ids=["bf16", "mxfp8"])
def test_macrobatches_interleaved_equal_separate_calls(precision):
    cfg = gen.CONFIGS[2].replace(S=2, M=1024)
    n = 4
    devs = [DevInputs(gen.make_inputs(cfg, seed=60 + i)) for i in range(n)]
    q = MoKLayer(L.desc_from_config(cfg, precision=precision))
    batches, refs = [], []
    for dv in devs:
        if precision == L.MOK_PREC_MXFP8:
            cs = [q.quantize_weights(t) for t in (dv.wg, dv.wu, dv.wd)]
            w, sc = tuple(c for c, _ in cs), tuple(s for _, s in cs)
        else:
            w, sc = (dv.wg, dv.wu, dv.wd), (None, None, None)
        batches.append((dv.x, dv.ids, dv.gates, *w, sc))
        ref_layer = MoKLayer(L.desc_from_config(cfg, precision=precision))
        ref_layer.schedule(dv.ids)
        refs.append(ref_layer.forward(dv.x, dv.ids, dv.gates, *w, scales=sc))
    torch.cuda.synchronize()
    layers = [MoKLayer(L.desc_from_config(cfg, precision=precision,
                                          flags=L.MOK_FLAG_OVERLAP_NEXT)) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for rep in range(2):
        ys = [torch.empty_like(r) for r in refs]
        forward_macrobatches(layers, streams, batches, ys)
        torch.cuda.synchronize()
        say(f"[macrobatch] precision={precision} repeat {rep}")
        for lay in layers:
            assert lay.status() == 0
        for i in range(n):
            assert torch.equal(ys[i], refs[i]), f"macrobatch {i} differs"
