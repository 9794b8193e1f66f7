"""GPU parity of the schedule and the bf16 forward against the float64 oracle.

Schedule tables are compared bit-exactly.  Layer outputs are compared by relative
Frobenius error against the oracle's float64 result (bound 1e-2 for bf16): the GPU reads
bf16 inputs, accumulates in fp32, rounds H and the expert outputs to bf16 and the layer
output once to bf16, so the expected error is a few 1e-3 at most."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import gen
from mixture_experts_layer_mok_amd.layer import MoKLayer
from tests.gpu_util import DevInputs, rel_fro, row_errors, run_forward, say, y_values

pytestmark = pytest.mark.gpu
TOL_BF16 = 1e-2


def _check_schedule(cfg, d, ids, layer):
    tab = layer.tables()
    s = O.schedule(ids, cfg.e0, cfg.n_local, cfg.E, cfg.M)
    assert tab["R"] == s.R
    assert tab["n_mb"] == s.n_mb
    assert np.array_equal(tab["counts"], s.counts)
    assert np.array_equal(tab["offsets"], s.offsets)
    assert np.array_equal(tab["perm"], s.perm)
    assert np.array_equal(tab["pos"], s.pos)
    return tab


@pytest.mark.parametrize("T,k,E,e0,nl", [
    (3000, 4, 64, 3, 40),      # 17..64 local experts: ranking rounds, bases in registers
    (2000, 6, 300, 10, 200),   # more than 64: bases in LDS
    (70000, 8, 32, 0, 16),     # count table above the fused-scan size: separate scan launch
    (70000, 8, 128, 5, 40),    # the same with ranking rounds
], ids=["nl40", "nl200", "big-nl16", "big-nl40"])
def test_schedule_paths_bit_exact(T, k, E, e0, nl):
    """mok_schedule against the oracle bit for bit on every placement path: one ballot per
    expert (<= 16 local experts, the other tests), ranking rounds with the next rows in
    registers (<= 64) or in LDS (more), and count tables too large for the scan to be
    folded into the place kernel; with masked and out-of-range ids."""
    rng = np.random.default_rng(T + nl)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids = gen.mask_ids(ids, 0.05, seed=nl)
    ids[::97, 0] = E + 1  # out of range: flagged and skipped
    cfg = gen.small_config("sched", T=T, D=64, I=64, E=E, k=k, e0=e0, E_loc=nl, M=512, S=2)
    say(f"[schedule] T={T} k={k} E={E} nl={nl}")
    layer = MoKLayer(L.desc_from_config(cfg))
    layer.schedule(torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    tab = _check_schedule(cfg, None, ids, layer)
    assert tab["status"] == L.MOK_DEV_BAD_ID


SMALL = [
    gen.CONFIGS[1],
    gen.small_config("ragged", T=300, D=192, I=192, E=6, k=2, M=96, S=2, comm_cus=8),
    gen.small_config("e0", T=257, D=128, I=128, E=16, k=4, e0=5, E_loc=6, M=64, S=3, comm_cus=16),
    gen.small_config("zipf", T=512, D=256, I=320, E=8, k=3, M=200, S=1, comm_cus=8, zipf_s=1.2),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_forward_small_parity(cfg, fused):
    say(f"[fwd-small] {cfg.name} fused={fused}")
    d = gen.make_inputs(cfg, seed=101)
    dev = DevInputs(d)
    y, layer = run_forward(cfg, dev, flags=0 if fused else L.MOK_FLAG_UNFUSED)
    assert layer.status() == 0
    _check_schedule(cfg, d, d["ids"], layer)
    ref = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0, E=cfg.E,
                    M=cfg.M)
    err = rel_fro(y_values(y), ref)
    say(f"  rel_fro={err:.3e}")
    assert err < TOL_BF16


@pytest.mark.parametrize("S", [1, 2, 4])
def test_forward_c1_ring_slots(S):
    cfg = gen.CONFIGS[1]
    d = gen.make_inputs(cfg)
    dev = DevInputs(d)
    ys = []
    for comm in (1, 8, 24):
        y, layer = run_forward(cfg, dev, S=S, comm_cus=comm)
        assert layer.status() == 0
        ys.append(y.clone())
    ref = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=cfg.E, M=32)
    assert rel_fro(y_values(ys[0]), ref) < TOL_BF16
    # error against the unrounded float32 draws, for information
    if d["x_raw"] is not None:
        ref_raw = O.forward(d["x_raw"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0,
                            E=cfg.E, M=32)
        say(f"  c1 vs unrounded draws: {rel_fro(y_values(ys[0]), ref_raw):.3e}")
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


def test_forward_edge_cases():
    cfg = gen.small_config("edge", T=200, D=128, I=128, E=8, k=2, M=64, S=2, comm_cus=8)
    d = gen.make_inputs(cfg, seed=5)
    ref_args = (d["x"], None, d["gates"], d["wg"], d["wu"], d["wd"])
    cases = {
        "none_local": np.full_like(d["ids"], -1),
        "all_to_one": np.stack([np.full(200, 3), np.full(200, -1)], 1).astype(np.int32),
        "masked": gen.mask_ids(d["ids"], 0.4, seed=1),
    }
    for name, ids in cases.items():
        say(f"[edge] {name}")
        dev = DevInputs(d, ids=ids)
        y, layer = run_forward(cfg, dev)
        assert layer.status() == 0
        _check_schedule(cfg, d, ids, layer)
        ref = O.forward(ref_args[0], ids, *ref_args[2:], e0=0, E=cfg.E, M=cfg.M)
        yv = y_values(y)
        if name == "none_local":
            assert np.all(yv == 0)
        else:
            assert rel_fro(yv, ref) < TOL_BF16
    # out-of-range ids are flagged and skipped
    bad = d["ids"].copy()
    bad[::7, 0] = cfg.E + 3
    bad[1::11, 1] = -5
    dev = DevInputs(d, ids=bad)
    y, layer = run_forward(cfg, dev)
    assert layer.status() == L.MOK_DEV_BAD_ID
    ref = O.forward(d["x"], bad, d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=cfg.E, M=cfg.M)
    assert rel_fro(y_values(y), ref) < TOL_BF16


def test_forward_config2_full():
    cfg = gen.CONFIGS[2]
    say("[c2] generating")
    d = gen.make_inputs(cfg)
    dev = DevInputs(d)
    y, layer = run_forward(cfg, dev)
    assert layer.status() == 0
    tab = _check_schedule(cfg, d, d["ids"], layer)
    assert tab["R"] == cfg.T * cfg.k
    ref = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=cfg.E,
                    M=cfg.M)
    err = rel_fro(y_values(y), ref)
    say(f"  c2 rel_fro={err:.3e}")
    assert err < TOL_BF16
    y2, _ = run_forward(cfg, dev, flags=L.MOK_FLAG_UNFUSED)
    assert torch.equal(y, y2)


@pytest.fixture(scope="module")
def c3_inputs():
    cfg = gen.CONFIGS[3]
    say("[c3] generating inputs")
    d = gen.make_inputs(cfg)
    return cfg, d, DevInputs(d)


def test_forward_config3_full_and_deterministic(c3_inputs):
    """The whole config-3 output against the oracle, row by row: the relative Frobenius
    error and the largest per-row relative error are both below 1e-2, and tokens without a
    local slot are exactly zero.  Then bitwise repeats and invariance."""
    cfg, d, dev = c3_inputs
    y, layer = run_forward(cfg, dev)
    assert layer.status() == 0
    _check_schedule(cfg, d, d["ids"], layer)
    say("[c3] oracle forward (float64)")
    ref = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=cfg.E,
                    M=cfg.M)
    fro, worst, stray = row_errors(y_values(y), ref)
    say(f"  c3 rel_fro={fro:.3e} worst row={worst:.3e} stray rows={stray}")
    assert fro < TOL_BF16 and worst < TOL_BF16 and stray == 0
    del ref
    y_again, _ = run_forward(cfg, dev)
    assert torch.equal(y, y_again)
    # per-row arithmetic does not depend on the minibatch split, the ring or the CU split
    for over in (dict(M=512, S=2, comm_cus=16), dict(M=4096, S=1, comm_cus=64)):
        say(f"  invariance {over}")
        y_o, lay = run_forward(cfg, dev, **over)
        assert lay.status() == 0
        assert torch.equal(y, y_o)
    y_u, _ = run_forward(cfg, dev, flags=L.MOK_FLAG_UNFUSED)
    assert torch.equal(y, y_u)


@pytest.mark.parametrize("precision", [0, 1], ids=["bf16", "mxfp8"])
def test_forward_reuses_workspace_with_new_inputs(precision):
    """Successive forwards on one workspace with different inputs: each must equal a fresh
    unfused run bit for bit, with as many ring slots as minibatches and with fewer (slots
    rewritten within a launch): no data of an earlier call or minibatch may survive."""
    cfg = gen.small_config("reuse", T=1024, D=256, I=256, E=8, k=2, M=256, S=8, comm_cus=16)
    for S in (8, 2):
        layer = MoKLayer(L.desc_from_config(cfg, S=S, precision=precision))
        for seed in (31, 32, 33):
            d = gen.make_inputs(cfg, seed=seed)
            dev = DevInputs(d)
            scales = (None, None, None)
            wg, wu, wd = dev.wg, dev.wu, dev.wd
            if precision:
                (wg, sg), (wu, su), (wd, sd) = (layer.quantize_weights(w) for w in (wg, wu, wd))
                scales = (sg, su, sd)
            layer.schedule(dev.ids)
            y = layer.forward(dev.x, dev.ids, dev.gates, wg, wu, wd, scales=scales)
            ref_layer = MoKLayer(L.desc_from_config(cfg, S=S, precision=precision,
                                                    flags=L.MOK_FLAG_UNFUSED))
            ref_layer.schedule(dev.ids)
            yr = ref_layer.forward(dev.x, dev.ids, dev.gates, wg, wu, wd, scales=scales)
            torch.cuda.synchronize()
            assert layer.status() == 0
            assert torch.equal(y, yr), (S, seed)


@pytest.mark.parametrize("precision", [L.MOK_PREC_BF16, L.MOK_PREC_MXFP8], ids=["bf16", "mxfp8"])
def test_forward_wait_timeout_exits_and_recovers(precision):
    """With MOK_FLAG_SHORT_WAITS every bounded wait of the fused forward expires after
    1 us, so a run with more minibatches than ring slots must time out: the kernel
    still exits (the synchronize returns), the status word carries MOK_DEV_TIMEOUT, and
    the next schedule and forward on the same workspace are correct again."""
    cfg = gen.small_config("timeout", T=512, D=256, I=256, E=4, k=2, M=64, S=1, comm_cus=8)
    d = gen.make_inputs(cfg, seed=12)
    dev = DevInputs(d)
    mx = precision == L.MOK_PREC_MXFP8
    desc = L.desc_from_config(cfg, flags=L.MOK_FLAG_SHORT_WAITS, precision=precision)
    layer = MoKLayer(desc)
    ws = (layer.quantize_weights(dev.wg), layer.quantize_weights(dev.wu),
          layer.quantize_weights(dev.wd)) if mx else None
    w = (ws[0][0], ws[1][0], ws[2][0]) if mx else (dev.wg, dev.wu, dev.wd)
    sc = (ws[0][1], ws[1][1], ws[2][1]) if mx else (None, None, None)
    say(f"[timeout] {'mxfp8' if mx else 'bf16'} short waits")
    layer.schedule(dev.ids)
    layer.forward(dev.x, dev.ids, dev.gates, *w, scales=sc)
    torch.cuda.synchronize()
    assert layer.status() & L.MOK_DEV_TIMEOUT
    say("[timeout] recovery run")
    layer.desc = L.desc_from_config(cfg, precision=precision)
    layer.schedule(dev.ids)
    y = layer.forward(dev.x, dev.ids, dev.gates, *w, scales=sc)
    torch.cuda.synchronize()
    assert layer.status() == 0
    ref = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0, E=cfg.E,
                    M=cfg.M, mxfp8=mx)
    assert rel_fro(y_values(y), ref) < (5e-2 if mx else TOL_BF16)
