"""GPU parity of the bf16 backward against the float64 oracle: dX, router-weight
gradient dG, dW_gate, dW_up, dW_down (relative Frobenius error < 1e-2 each), plus
bitwise run-to-run determinism and edge cases (masked slots, experts with no rows)."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import gen
from mixture_experts_layer_mok_amd.layer import MoKLayer, bf16_values
from tests.gpu_util import DevInputs, rel_fro, row_errors, say

pytestmark = pytest.mark.gpu
TOL_BF16 = 1e-2


def run_fwd_bwd(cfg, dev, flags=L.MOK_FLAG_SAVE_FOR_BWD, **over):
    desc = L.desc_from_config(cfg, flags=flags, **over)
    layer = MoKLayer(desc)
    layer.schedule(dev.ids)
    y = layer.forward(dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd)
    g = layer.backward(dev.dy, dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd)
    torch.cuda.synchronize()
    return y, g, layer


def _compare(cfg, d, ids, g, tag):
    ref = O.backward(d["dy"], d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0,
                     E=cfg.E, M=cfg.M)
    errs = {
        "dx": rel_fro(bf16_values(g["dx"]), ref["dx"]),
        "dg": rel_fro(g["dg"].cpu().numpy(), ref["dg"]),
        "dwg": rel_fro(g["dwg"].cpu().numpy(), ref["dwg"]),
        "dwu": rel_fro(g["dwu"].cpu().numpy(), ref["dwu"]),
        "dwd": rel_fro(g["dwd"].cpu().numpy(), ref["dwd"]),
    }
    _, worst, stray = row_errors(bf16_values(g["dx"]), ref["dx"])
    say(f"  {tag} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) +
        f" dx worst row={worst:.2e}")
    for k, v in errs.items():
        assert v < TOL_BF16, (k, v)
    assert worst < TOL_BF16 and stray == 0, (worst, stray)
    # non-local slots carry no gradient
    assert np.all(g["dg"].cpu().numpy()[ref["schedule"].pos.reshape(ids.shape) < 0] == 0)
    return ref


SMALL = [
    gen.CONFIGS[1],
    gen.small_config("ragged", T=300, D=192, I=192, E=6, k=2, M=96, S=2, comm_cus=8),
    gen.small_config("e0", T=257, D=128, I=128, E=16, k=4, e0=5, E_loc=6, M=64, S=3, comm_cus=16),
    gen.small_config("zipf", T=512, D=256, I=320, E=8, k=3, M=200, S=1, comm_cus=8, zipf_s=1.2),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_backward_small_parity(cfg):
    say(f"[bwd-small] {cfg.name}")
    d = gen.make_inputs(cfg, seed=202, with_dy=True)
    dev = DevInputs(d)
    _, g, layer = run_fwd_bwd(cfg, dev)
    assert layer.status() == 0
    _compare(cfg, d, d["ids"], g, cfg.name)


def test_backward_edge_cases():
    cfg = gen.small_config("bedge", T=200, D=128, I=128, E=8, k=2, M=64, S=2, comm_cus=8)
    d = gen.make_inputs(cfg, seed=7, with_dy=True)
    # expert 5 receives nothing, a third of the slots are masked
    ids = gen.mask_ids(d["ids"], 0.3, seed=3)
    ids[ids == 5] = -1
    dev = DevInputs(d, ids=ids)
    _, g, layer = run_fwd_bwd(cfg, dev)
    assert layer.status() == 0
    _compare(cfg, d, ids, g, "masked+empty-expert")
    for name in ("dwg", "dwu", "dwd"):
        assert torch.count_nonzero(g[name][5]).item() == 0
    # nothing local at all: every gradient is zero
    none = np.full_like(d["ids"], -1)
    dev = DevInputs(d, ids=none)
    _, g, layer = run_fwd_bwd(cfg, dev)
    assert layer.status() == 0
    for name, t in g.items():
        assert torch.count_nonzero(t).item() == 0, name


@pytest.mark.parametrize("S", [2, 8], ids=["replay", "all-resident"])
def test_backward_expert_longer_than_row_table(S):
    """Expert 1 holds 9000 routed rows: the dW tiles run past two windows of the row
    offset table (4096 rows each); with 8 ring slots every minibatch stays resident and
    the X rows come from the ring, with 2 the early ones are replayed and X is gathered."""
    cfg = gen.small_config("long", T=9000, D=128, I=128, E=4, k=2, M=4096, S=S, comm_cus=8)
    d = gen.make_inputs(cfg, seed=21, with_dy=True)
    ids = d["ids"].copy()
    ids[:, 0] = 1
    ids[:, 1] = np.where(ids[:, 1] == 1, 2, ids[:, 1])
    dev = DevInputs(d, ids=ids)
    _, g, layer = run_fwd_bwd(cfg, dev)
    assert layer.status() == 0
    assert int(layer.tables()["counts"][1]) == 9000
    _compare(cfg, d, ids, g, f"long-expert S={S}")


def test_backward_outputs_ordered_on_caller_stream():
    """The backward runs on the caller's stream: work enqueued after it on a non-default
    stream (copies of its outputs) sees every output complete, call after call."""
    cfg = SMALL[1]
    d = gen.make_inputs(cfg, seed=13, with_dy=True)
    dev = DevInputs(d)
    _, ref, _ = run_fwd_bwd(cfg, dev)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        layer = MoKLayer(L.desc_from_config(cfg, flags=L.MOK_FLAG_SAVE_FOR_BWD))
        layer.schedule(dev.ids, stream=s.cuda_stream)
        layer.forward(dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd, stream=s.cuda_stream)
        for _ in range(3):
            g = layer.backward(dev.dy, dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd,
                               stream=s.cuda_stream)
            # copies enqueued on the same stream see finished outputs
            got = {k: v.clone() for k, v in g.items()}
    s.synchronize()
    for k in ref:
        assert torch.equal(got[k], ref[k]), k


def test_backward_config5_full_and_deterministic():
    """Config 5 against the oracle (the whole Y row by row, every gradient), then ten
    forward + backward runs in all, each on a new workspace, bitwise equal in Y and every
    gradient."""
    cfg = gen.CONFIGS[5]
    say("[c5] generating")
    d = gen.make_inputs(cfg, with_dy=True)
    dev = DevInputs(d)
    y1, g1, layer = run_fwd_bwd(cfg, dev)
    assert layer.status() == 0
    del layer
    say("[c5] oracle forward (float64)")
    ref_y = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0,
                      E=cfg.E, M=cfg.M)
    fro, worst, stray = row_errors(bf16_values(y1), ref_y)
    say(f"  c5 y rel_fro={fro:.3e} worst row={worst:.3e} stray rows={stray}")
    assert fro < TOL_BF16 and worst < TOL_BF16 and stray == 0
    del ref_y
    say("[c5] oracle backward (float64)")
    _compare(cfg, d, d["ids"], g1, "c5")
    for run in range(2, 11):
        y, g, layer = run_fwd_bwd(cfg, dev)
        assert layer.status() == 0
        del layer
        assert torch.equal(y1, y), f"y differs in run {run}"
        for k in g1:
            assert torch.equal(g1[k], g[k]), f"{k} differs in run {run}"
    say("[c5] 10 runs bitwise identical")


@pytest.mark.parametrize("cfg", SMALL[1:3], ids=lambda c: c.name)
def test_backward_after_fused_and_unfused_forward_agree(cfg):
    """The backward takes a, b from the forward where it still holds them (ring slots
    after a fused forward, every row after an unfused one) and replays GEMM1 elsewhere;
    replayed and held values come from the same tile arithmetic, so the gradients are
    bitwise equal, and equal again with a one-slot ring (everything but the last
    minibatch replayed)."""
    d = gen.make_inputs(cfg, seed=77, with_dy=True)
    dev = DevInputs(d)
    _, g_f, _ = run_fwd_bwd(cfg, dev)
    _, g_u, _ = run_fwd_bwd(cfg, dev, flags=L.MOK_FLAG_SAVE_FOR_BWD | L.MOK_FLAG_UNFUSED)
    _, g_1, _ = run_fwd_bwd(cfg, dev, S=1)
    for name in g_f:
        assert torch.equal(g_f[name], g_u[name]), name
        assert torch.equal(g_f[name], g_1[name]), name


def test_backward_wait_timeout_exits_and_recovers():
    """dX tiles wait for the dH tiles of their m-tile inside one launch.  With
    MOK_FLAG_SHORT_WAITS such a wait expires after 1 us, well before a dH tile with
    K = 1024 ends, so the backward must time out after an (unfused, wait-free) forward:
    the launch still exits, the status word carries MOK_DEV_TIMEOUT, and the next
    schedule, forward and backward on the same workspace are correct again."""
    cfg = gen.small_config("bwd-timeout", T=512, D=1024, I=512, E=4, k=2, M=256, S=2,
                           comm_cus=8)
    d = gen.make_inputs(cfg, seed=14, with_dy=True)
    dev = DevInputs(d)
    say("[bwd-timeout] short waits")
    flags = L.MOK_FLAG_SAVE_FOR_BWD | L.MOK_FLAG_UNFUSED
    _, _, layer = run_fwd_bwd(cfg, dev, flags=flags | L.MOK_FLAG_SHORT_WAITS)
    assert layer.status() & L.MOK_DEV_TIMEOUT
    say("[bwd-timeout] recovery run")
    layer.desc = L.desc_from_config(cfg, flags=flags)
    layer.schedule(dev.ids)
    layer.forward(dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd)
    g = layer.backward(dev.dy, dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd)
    torch.cuda.synchronize()
    assert layer.status() == 0
    _compare(cfg, d, d["ids"], g, cfg.name)
