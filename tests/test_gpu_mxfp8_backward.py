"""GPU parity of the MXFP8 backward (mok_moe_bwd_mx) against the float64 oracle that
applies the same MX round trips (oracle.backward(mxfp8=True): a, b as saved bf16 rows; dY
and W_down along D for u, da / db from their bf16 rows and W_gate / W_up along I for the
dX rows; weight gradients unquantised): relative Frobenius error below 1e-2 on dX, dG and
the three weight gradients, and below 5e-2 for the largest per-row error of dX; the transposing weight quantiser bit-exact against the
oracle's quantiser; bitwise repeats and fused / unfused forwards giving the same
gradients."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import gen
from mixture_experts_layer_mok_amd.layer import MoKLayer, bf16_tensor, bf16_values
from tests.gpu_util import DevInputs, rel_fro, row_errors, say
from tests.test_gpu_mxfp8 import _edge_matrix

pytestmark = pytest.mark.gpu
# Relative Frobenius bar: the MX oracle applies the same round trips, and each code is
# decided from values of the precision the kernels hold, so what is left is bf16 rounding
# of stored values and float32 accumulation order, the bf16 bar.  A row can still hold a
# code that the two accumulation orders put on either side of an e4m3 rounding midpoint
# (one element off by one e4m3 step, up to 2^-3 of it), so the per-row bar is wider.
TOL_MX = 1e-2
TOL_MX_ROW = 5e-2


def run_mx_fwd_bwd(cfg, dev, flags=0, **over):
    desc = L.desc_from_config(cfg, flags=flags | L.MOK_FLAG_SAVE_FOR_BWD,
                              precision=L.MOK_PREC_MXFP8, **over)
    layer = MoKLayer(desc)
    q = [layer.quantize_weights(t) for t in (dev.wg, dev.wu, dev.wd)]
    wt = layer.quantize_weights_bwd(dev.wg, dev.wu, dev.wd)
    layer.schedule(dev.ids)
    y = layer.forward(dev.x, dev.ids, dev.gates, *(c for c, _ in q), scales=tuple(s for _, s in q))
    g = layer.backward_mx(dev.dy, dev.x, dev.ids, dev.gates, wt)
    torch.cuda.synchronize()
    return y, g, layer


def _compare(cfg, d, ids, g, tag):
    ref = O.backward(d["dy"], d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0,
                     E=cfg.E, M=cfg.M, mxfp8=True)
    got = {"dx": bf16_values(g["dx"]), **{n: g[n].cpu().numpy() for n in ("dg", "dwg", "dwu", "dwd")}}
    errs = {n: rel_fro(got[n], ref[n]) for n in got}
    _, worst, stray = row_errors(got["dx"], ref["dx"])
    say(f"  {tag} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) +
        f" dx worst row={worst:.2e}")
    for k, v in errs.items():
        assert v < TOL_MX, (k, v)
    assert worst < TOL_MX_ROW and stray == 0, (worst, stray)
    assert np.all(got["dg"][ref["schedule"].pos.reshape(ids.shape) < 0] == 0)


def test_quantize_mx_t_bit_exact():
    """mok_quantize_mx_t = the oracle's quantiser applied to each transposed matrix, also
    into a wider destination at a column offset (the [W_gate; W_up]^T layout)."""
    bits, vals = _edge_matrix(rows=64, cols=96)
    b2 = np.stack([bits, bits[::-1]])                    # batch of 2, [64, 96]
    v2 = np.stack([vals, vals[::-1]])
    dev = torch.device("cuda")
    src = bf16_tensor(b2, dev)
    codes = torch.full((2, 96, 160), 0xAA, dtype=torch.uint8, device=dev)
    scales = torch.full((2, 96, 8), 0xAA, dtype=torch.uint8, device=dev)
    L.mok_quantize_mx_t(src, 2, 64, 96, codes.data_ptr() + 32, 160, scales.data_ptr() + 1, 8)
    torch.cuda.synchronize()
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    for b in range(2):
        rc, rs = O.mx_quantize(np.ascontiguousarray(v2[b].T))
        assert np.array_equal(gc[b, :, 32:96], rc)
        assert np.array_equal(gs[b, :, 1:3], rs)
    assert np.all(gc[:, :, :32] == 0xAA) and np.all(gc[:, :, 96:] == 0xAA)
    assert np.all(gs[:, :, 0] == 0xAA) and np.all(gs[:, :, 3:] == 0xAA)


SMALL = [
    gen.CONFIGS[1],
    gen.small_config("ragged", T=300, D=192, I=192, E=6, k=2, M=96, S=2, comm_cus=8),
    gen.small_config("e0", T=257, D=128, I=128, E=16, k=4, e0=5, E_loc=6, M=64, S=3, comm_cus=16),
    gen.small_config("zipf", T=512, D=256, I=320, E=8, k=3, M=200, S=1, comm_cus=8, zipf_s=1.2),
    gen.small_config("odd-steps", T=200, D=320, I=448, E=4, k=2, M=128, S=2, comm_cus=8),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_backward_mx_small_parity(cfg):
    say(f"[mx-bwd] {cfg.name}")
    d = gen.make_inputs(cfg, seed=404, with_dy=True)
    dev = DevInputs(d)
    _, g, layer = run_mx_fwd_bwd(cfg, dev)
    assert layer.status() == 0
    _compare(cfg, d, d["ids"], g, cfg.name)


def test_backward_mx_edge_cases():
    cfg = gen.small_config("mxbedge", T=200, D=128, I=128, E=8, k=2, M=64, S=2, comm_cus=8)
    d = gen.make_inputs(cfg, seed=8, with_dy=True)
    ids = gen.mask_ids(d["ids"], 0.3, seed=3)
    ids[ids == 5] = -1                                   # an expert with no rows
    dev = DevInputs(d, ids=ids)
    _, g, layer = run_mx_fwd_bwd(cfg, dev)
    assert layer.status() == 0
    _compare(cfg, d, ids, g, "masked+empty-expert")
    for name in ("dwg", "dwu", "dwd"):
        assert torch.count_nonzero(g[name][5]).item() == 0
    dev = DevInputs(d, ids=np.full_like(d["ids"], -1))
    _, g, layer = run_mx_fwd_bwd(cfg, dev)
    assert layer.status() == 0
    for name, t in g.items():
        assert torch.count_nonzero(t).item() == 0, name


def test_backward_mx_config2_full_deterministic_and_fused_unfused():
    """Config 2's shape (every expert local, 16384 routed rows) against the oracle; a
    repeat is bitwise equal, and so is the backward after an unfused MXFP8 forward."""
    cfg = gen.CONFIGS[2]
    say("[mx-bwd c2] generating")
    d = gen.make_inputs(cfg, with_dy=True)
    dev = DevInputs(d)
    _, g1, layer = run_mx_fwd_bwd(cfg, dev)
    assert layer.status() == 0
    say("[mx-bwd c2] oracle backward (float64, MX round trips)")
    _compare(cfg, d, d["ids"], g1, "c2")
    _, g2, _ = run_mx_fwd_bwd(cfg, dev)
    _, g3, layer3 = run_mx_fwd_bwd(cfg, dev, flags=L.MOK_FLAG_UNFUSED)
    assert layer3.status() == 0
    for k in g1:
        assert torch.equal(g1[k], g2[k]), f"{k} differs between repeats"
        assert torch.equal(g1[k], g3[k]), f"{k} differs after the unfused forward"


def test_backward_mx_perturbed_is_bitwise_neutral():
    cfg = SMALL[3]
    d = gen.make_inputs(cfg, seed=55, with_dy=True)
    dev = DevInputs(d)
    _, g0, _ = run_mx_fwd_bwd(cfg, dev)
    _, g1, layer = run_mx_fwd_bwd(cfg, dev, flags=L.MOK_FLAG_PERTURB)
    assert layer.status() == 0
    for k in g0:
        assert torch.equal(g0[k], g1[k]), k


@pytest.mark.parametrize("c", [4, 6], ids=["c4", "c6"])
def test_backward_mx_zipf_shares_sampled(c):
    """Config 4 (MXFP8, Zipf routing, about 86k routed rows) and config 6 (permuted ranks,
    about 3.8k rows in experts of 35 to 2k rows): dX and dG of sampled tokens
    (tokens of every local expert and those owning the rows on both sides of every
    minibatch window boundary) against the MX oracle's backward on the pool of just those
    tokens (a token's dx and dG depend only on its own rows and the weights); and the three
    weight gradients of the local expert with the fewest rows against the oracle's
    backward on the tokens routed to it (their other slots masked)."""
    cfg = gen.CONFIGS[c]
    say(f"[mx-bwd c{c}] generating")
    d = gen.make_inputs(cfg, with_dy=True)
    dev = DevInputs(d)
    _, g, layer = run_mx_fwd_bwd(cfg, dev)
    assert layer.status() == 0
    ids = d["ids"]
    s = O.schedule(ids, cfg.e0, cfg.n_local, cfg.E, cfg.M)
    rng = np.random.default_rng(45)
    rows = set()
    for e in range(cfg.n_local):
        lo, hi = int(s.offsets[e]), int(s.offsets[e + 1])
        if hi > lo:
            rows.update(rng.integers(lo, hi, 4).tolist())
            rows.update((lo, hi - 1))
    for b in range(cfg.M, s.R, cfg.M):
        rows.update(r for r in (b - 1, b) if 0 <= r < s.R)
    toks = np.unique(s.perm[sorted(rows)] // cfg.k)
    say(f"[mx-bwd c{c}] oracle backward on {len(toks)} tokens")
    ref = O.backward(d["dy"][toks], d["x"][toks], ids[toks], d["gates"][toks], d["wg"], d["wu"],
                     d["wd"], e0=cfg.e0, E=cfg.E, M=cfg.M, mxfp8=True)
    dx = bf16_values(g["dx"])[toks]
    fro, worst, stray = row_errors(dx, ref["dx"])
    dg_err = rel_fro(g["dg"].cpu().numpy()[toks], ref["dg"])
    say(f"[mx-bwd c{c}] dx rel_fro {fro:.2e} worst row {worst:.2e}, dg {dg_err:.2e}")
    assert fro < TOL_MX and worst < TOL_MX_ROW and stray == 0 and dg_err < TOL_MX
    e_min = int(np.argmin(np.where(s.counts > 0, s.counts, np.iinfo(np.int64).max)))
    tok_e = np.flatnonzero((ids == cfg.e0 + e_min).any(axis=1))
    ids_e = np.where(ids[tok_e] == cfg.e0 + e_min, ids[tok_e], -1)
    say(f"[mx-bwd c{c}] oracle weight gradients of expert {e_min} ({len(tok_e)} rows)")
    ref_w = O.backward(d["dy"][tok_e], d["x"][tok_e], ids_e, d["gates"][tok_e], d["wg"],
                       d["wu"], d["wd"], e0=cfg.e0, E=cfg.E, M=cfg.M, mxfp8=True)
    for name in ("dwg", "dwu", "dwd"):
        err = rel_fro(g[name][e_min].cpu().numpy(), ref_w[name][e_min])
        say(f"[mx-bwd c{c}] {name}[{e_min}] rel_fro {err:.2e}")
        assert err < TOL_MX, (name, err)
