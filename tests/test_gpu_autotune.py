"""GPU test of the per-shape tuner on the config-2 shape: the choice comes from the grid it
was given, the forward with the chosen minibatch and split is bitwise equal to the forward
with the starting ones and matches the oracle, and a second call is served from the cache."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import autotune as A
from mixture_experts_layer_mok_amd import gen
from tests.gpu_util import DevInputs, rel_fro, run_forward, say, y_values

pytestmark = pytest.mark.gpu


def test_tune_config2_choice_is_bitwise_neutral(tmp_path):
    cfg = gen.CONFIGS[2]
    say(f"[autotune] {cfg.name}")
    d = gen.make_inputs(cfg)
    dev = DevInputs(d)
    desc = L.desc_from_config(cfg)
    cache = str(tmp_path / "tune.json")
    m_grid, comm_grid = [512, 1024, 2048], [16, 32]
    ch = A.tune(desc, dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd, steps=2, warmup=1,
                cache_path=cache, comm_grid=comm_grid, m_grid=m_grid)
    say(f"  choice M={ch.minibatch_rows} comm_cus={ch.comm_cus} fwd_ms={ch.fwd_ms}")
    assert ch.minibatch_rows in m_grid + [cfg.M] and ch.comm_cus in comm_grid
    assert ch.fwd_ms == min(t["fwd_ms"] for t in ch.trials)
    y0, l0 = run_forward(cfg, dev)
    y1, l1 = run_forward(cfg, dev, M=ch.minibatch_rows, comm_cus=ch.comm_cus)
    assert l0.status() == 0 and l1.status() == 0
    b0 = y0.view(torch.int16).cpu().numpy()
    b1 = y1.view(torch.int16).cpu().numpy()
    assert np.array_equal(b0, b1)
    ref = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0, E=cfg.E,
                    M=cfg.M)
    assert rel_fro(y_values(y1), ref) < 1e-2
    again = A.tune(desc, dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd, cache_path=cache,
                   comm_grid=[8], m_grid=[4096])  # served from the cache: grids unused
    assert (again.minibatch_rows, again.comm_cus) == (ch.minibatch_rows, ch.comm_cus)
