"""The layer inside a HIP graph: schedule, forward and backward captured once on the current
stream (torch.cuda.graph), then replayed with new routing, activations, gates and output
gradients written into the captured input tensors in place, with eager launches of the
library (on another workspace) and synchronisations between the replays.  Every replay
must equal the eager calls on the same inputs bit for bit, in bf16 and MXFP8: the
launches read the routed-row count, the minibatch count and every tile count from the
workspace on the device, and no step of the path enqueues a memset or a host copy."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import gen
from mixture_experts_layer_mok_amd.layer import MoKLayer
from tests.gpu_util import DevInputs, say

pytestmark = pytest.mark.gpu

CASES = [
    gen.CONFIGS[2],  # 16 minibatches on 2 ring slots: slot reuse and GEMM1 replay
    gen.small_config("ragged", T=300, D=192, I=192, E=6, k=2, M=96, S=2, comm_cus=8),
]


class Step:
    """Schedule + forward + backward of one layer on static device tensors."""

    def __init__(self, cfg, dev: DevInputs, precision):
        self.mx = precision == L.MOK_PREC_MXFP8
        self.layer = MoKLayer(L.desc_from_config(cfg, flags=L.MOK_FLAG_SAVE_FOR_BWD,
                                                 precision=precision))
        self.dev = dev
        if self.mx:
            q = [self.layer.quantize_weights(t) for t in (dev.wg, dev.wu, dev.wd)]
            self.w = tuple(c for c, _ in q)
            self.sc = tuple(s for _, s in q)
            self.wt = self.layer.quantize_weights_bwd(dev.wg, dev.wu, dev.wd)
        else:
            self.w = (dev.wg, dev.wu, dev.wd)
            self.sc = (None, None, None)

    def __call__(self):
        d = self.dev
        self.layer.schedule(d.ids)
        y = self.layer.forward(d.x, d.ids, d.gates, *self.w, scales=self.sc)
        if self.mx:
            g = self.layer.backward_mx(d.dy, d.x, d.ids, d.gates, self.wt)
        else:
            g = self.layer.backward(d.dy, d.x, d.ids, d.gates, *self.w)
        return {"y": y, **g}


def _load(dst: DevInputs, d: dict):
    """Write the activations, routing, gates and output gradients of d into dst in place."""
    src = DevInputs(d)
    for name in ("x", "ids", "gates", "dy"):
        getattr(dst, name).copy_(getattr(src, name))


@pytest.mark.parametrize("precision", [L.MOK_PREC_BF16, L.MOK_PREC_MXFP8], ids=["bf16", "mxfp8"])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_graph_replays_equal_eager(cfg, precision):
    say(f"[graph] {cfg.name} precision={precision}: capture")
    dev = DevInputs(gen.make_inputs(cfg, seed=70, with_dy=True))
    step = Step(cfg, dev, precision)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    torch.cuda.synchronize()
    # the eager reference: the same weights, its own layer and workspace, fresh inputs
    ref_dev = DevInputs(gen.make_inputs(cfg, seed=70, with_dy=True))
    ref_step = Step(cfg, ref_dev, precision)
    for i, seed in enumerate((71, 72, 73)):
        d = gen.make_inputs(cfg, seed=seed, with_dy=True)
        if i == 1:  # masked slots and an expert without rows
            d["ids"] = gen.mask_ids(d["ids"], 0.3, seed=seed)
            d["ids"][d["ids"] == 1] = -1
        _load(ref_dev, d)
        ref = ref_step()
        torch.cuda.synchronize()
        assert ref_step.layer.status() == 0
        _load(dev, d)
        graph.replay()
        torch.cuda.synchronize()
        assert step.layer.status() == 0, f"replay {i}: device status"
        say(f"[graph] {cfg.name} replay {i} (seed {seed}, "
            f"{int(np.count_nonzero(d['ids'] >= 0))} routed pairs) against eager")
        for name, t in ref.items():
            assert torch.equal(out[name], t), f"replay {i}: {name} differs from eager"
