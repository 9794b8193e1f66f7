"""GPU parity of the MXFP8 forward against the float64 oracle that applies the same MX
round-trips (X at dispatch, the weights, H after SwiGLU; OCP MX blocks of 32 with the
ceil scale rule).

- mok_quantize_mx, which runs the same row quantiser as the forward's dispatch, is
  compared bit for bit with the oracle's quantiser on values that reach every branch of
  the encoding: all-zero blocks, subnormal bf16, amax exactly 448 * 2^n, mantissas
  just above and below 1.75, round-to-nearest-even ties, signs.
- Layer outputs are compared by relative Frobenius error against the MX-emulating
  oracle (bound 1e-2; 5e-2 on a single row); the error against the unquantised oracle
  is printed only.
- Fused and unfused runs, and runs with other minibatch sizes, ring slots and comm CUs,
  must agree bit for bit; the config-4 run is repeated and compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import gen
from mixture_experts_layer_mok_amd.layer import MoKLayer, bf16_tensor
from tests.gpu_util import DevInputs, rel_fro, row_errors, say, y_values

pytestmark = pytest.mark.gpu
# Relative Frobenius bar: the MX oracle applies the same round trips, and each code is
# decided from values of the precision the kernels hold, so what is left is bf16 rounding
# of stored values and float32 accumulation order, the bf16 bar.  A row can still hold a
# code that the two accumulation orders put on either side of an e4m3 rounding midpoint
# (one element off by one e4m3 step, up to 2^-3 of it), so the per-row bar is wider.
TOL_MX = 1e-2
TOL_MX_ROW = 5e-2


class MxWeights:
    def __init__(self, layer: MoKLayer, dev: DevInputs):
        self.g, self.gs = layer.quantize_weights(dev.wg)
        self.u, self.us = layer.quantize_weights(dev.wu)
        self.d, self.ds = layer.quantize_weights(dev.wd)


def run_mx(cfg, dev, flags=0, **over):
    desc = L.desc_from_config(cfg, flags=flags, precision=L.MOK_PREC_MXFP8, **over)
    layer = MoKLayer(desc)
    w = MxWeights(layer, dev)
    layer.schedule(dev.ids)
    y = layer.forward(dev.x, dev.ids, dev.gates, w.g, w.u, w.d, scales=(w.gs, w.us, w.ds))
    torch.cuda.synchronize()
    return y, layer


def _edge_matrix(rows=48, cols=256, seed=5):
    """bf16 values covering the quantiser's branches, as float32."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    v *= np.ldexp(1.0, rng.integers(-20, 20, size=(rows, 1))).astype(np.float32)
    v[0] = 0.0                                            # all-zero blocks
    v[1, :32] = np.float32(-0.0)
    v[2] = np.ldexp(rng.standard_normal(cols), -130).astype(np.float32)  # bf16 subnormals
    v[3, :32] = 448.0 * 4                                 # amax exactly 448 * 2^n
    v[3, 1] = -448.0 * 4
    m = np.float32(1.75)
    v[4, :32] = np.ldexp(m, 9)                            # mantissa exactly 1.75: no carry
    v[5, :32] = np.ldexp(np.float32(1.7578125), 9)        # just above 1.75 (bf16 step)
    v[6, :32] = np.ldexp(np.float32(1.0), 3) * np.arange(32, dtype=np.float32) / 8
    # ties: values halfway between e4m3 neighbours once scaled (x.5 ulp of 3 bits)
    v[7, :32] = np.float32(1.0) + np.float32(1.0 / 16) * (2 * np.arange(32) % 16)
    v[8] = np.ldexp(np.float32(1.0), 120) * rng.standard_normal(cols).astype(np.float32)
    bits = gen.f32_to_bf16_bits(v)
    return bits, gen.bf16_bits_to_f32(bits)


def test_quantize_mx_bit_exact():
    bits, vals = _edge_matrix()
    dev = torch.device("cuda")
    src = bf16_tensor(bits, dev)
    layer = MoKLayer(L.desc_from_config(gen.CONFIGS[1], precision=L.MOK_PREC_MXFP8), device=dev)
    codes, scales = layer.quantize_weights(src)
    torch.cuda.synchronize()
    rc, rs = O.mx_quantize(vals)
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(gs, rs), np.argwhere(gs != rs)[:5]
    assert np.array_equal(gc, rc), np.argwhere(gc != rc)[:5]


SMALL = [
    gen.CONFIGS[1],  # I = 64: GEMM2 is one half step
    gen.small_config("ragged", T=300, D=192, I=192, E=6, k=2, M=96, S=2, comm_cus=8),
    gen.small_config("e0", T=257, D=128, I=128, E=16, k=4, e0=5, E_loc=6, M=64, S=3, comm_cus=16),
    gen.small_config("zipf", T=512, D=256, I=320, E=8, k=3, M=200, S=1, comm_cus=8, zipf_s=1.2),
    gen.small_config("odd-steps", T=200, D=320, I=448, E=4, k=2, M=128, S=2, comm_cus=8),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_forward_mx_small_parity(cfg):
    say(f"[mx-small] {cfg.name}")
    d = gen.make_inputs(cfg, seed=303)
    dev = DevInputs(d)
    y, layer = run_mx(cfg, dev)
    assert layer.status() == 0
    yu, layer_u = run_mx(cfg, dev, flags=L.MOK_FLAG_UNFUSED)
    assert layer_u.status() == 0
    assert torch.equal(y, yu), "fused and unfused MXFP8 forwards differ"
    ref = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0, E=cfg.E,
                    M=cfg.M, mxfp8=True)
    plain = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0,
                      E=cfg.E, M=cfg.M)
    yv = y_values(y)
    err = rel_fro(yv, ref)
    say(f"  vs MX oracle {err:.3e}; vs unquantised oracle {rel_fro(yv, plain):.3e}")
    assert err < TOL_MX


def test_forward_mx_comm_cus_too_large_enqueues_nothing():
    """comm_cus at or above the persistent kernel's grid (one workgroup per CU) is refused
    with MOK_E_SHAPE before anything is enqueued: with D % 128 == 64 the forward would first
    repack the weight scales into the workspace, and the workspace stays untouched."""
    cfg = gen.small_config("mxcomm", T=64, D=192, I=128, E=4, k=2, M=32, S=2, comm_cus=8)
    d = gen.make_inputs(cfg, seed=4)
    dev = DevInputs(d)
    w = MxWeights(MoKLayer(L.desc_from_config(cfg, precision=L.MOK_PREC_MXFP8)), dev)
    layer = MoKLayer(L.desc_from_config(cfg, precision=L.MOK_PREC_MXFP8,
                                        comm_cus=L.mok_device_cus()))
    layer.schedule(dev.ids)
    torch.cuda.synchronize()
    layer.ws.fill_(0x5A)
    torch.cuda.synchronize()
    with pytest.raises(L.MokError) as err:
        layer.forward(dev.x, dev.ids, dev.gates, w.g, w.u, w.d, scales=(w.gs, w.us, w.ds))
    assert err.value.code == L.MOK_E_SHAPE
    torch.cuda.synchronize()
    assert bool((layer.ws == 0x5A).all())


def test_forward_mx_ring_and_split_invariance():
    cfg = SMALL[3]
    d = gen.make_inputs(cfg, seed=17)
    dev = DevInputs(d)
    base, _ = run_mx(cfg, dev)
    for over in (dict(M=64, S=3, comm_cus=4), dict(M=512, S=1, comm_cus=16),
                 dict(M=37, S=2, comm_cus=1)):
        y, layer = run_mx(cfg, dev, **over)
        assert layer.status() == 0
        assert torch.equal(y, base), over


def test_forward_mx_edge_cases():
    cfg = gen.small_config("mxedge", T=160, D=128, I=128, E=8, k=2, M=64, S=2, comm_cus=8)
    d = gen.make_inputs(cfg, seed=9)
    # nothing local: y is zero
    dev = DevInputs(d, ids=np.full_like(d["ids"], -1))
    y, layer = run_mx(cfg, dev)
    assert layer.status() == 0
    assert torch.count_nonzero(y).item() == 0
    # every slot on one expert, a third masked
    ids = gen.mask_ids(np.full_like(d["ids"], 3), 0.3, seed=2)
    ids[:, 1] = np.where(ids[:, 1] >= 0, 5, -1)
    dev = DevInputs(d, ids=ids)
    y, layer = run_mx(cfg, dev)
    assert layer.status() == 0
    ref = O.forward(d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=cfg.E, M=cfg.M,
                    mxfp8=True)
    assert rel_fro(y_values(y), ref) < TOL_MX


@pytest.mark.parametrize("c", [4, 6], ids=["c4", "c6"])
def test_forward_zipf_shares_sampled_and_deterministic(c):
    """Config 4 (MXFP8, Zipf routing, about 86k routed rows) and config 6 (the same skew
    with permuted ranks: about 3.8k rows, experts of 35 to 2k rows) against the
    MX-emulating oracle on sampled tokens: tokens of every local expert, and the tokens
    that own the rows on both sides of every minibatch window boundary and of the first
    m-tile start (256 rows from the expert's first row) at or after it; plus tokens with no
    local slot, which must be exactly zero.  Relative Frobenius error below 1e-2 and the
    largest per-row error below 5e-2.  Then a bitwise repeat."""
    cfg = gen.CONFIGS[c]
    say(f"[c{c}] generating")
    d = gen.make_inputs(cfg)
    dev = DevInputs(d)
    y, layer = run_mx(cfg, dev)
    assert layer.status() == 0
    tab = layer.tables()
    say(f"[c{c}] routed rows {tab['R']}, per expert {tab['counts'].tolist()}")
    y2, _ = run_mx(cfg, dev)
    assert torch.equal(y, y2), "MXFP8 forward not deterministic"
    ids = d["ids"]
    s = O.schedule(ids, cfg.e0, cfg.n_local, cfg.E, cfg.M)
    rng = np.random.default_rng(44)
    rows = set()
    for e in range(cfg.n_local):                      # every local expert
        lo, hi = int(s.offsets[e]), int(s.offsets[e + 1])
        if hi > lo:
            rows.update(rng.integers(lo, hi, 4).tolist())
            rows.update((lo, hi - 1))
    for b in range(cfg.M, s.R, cfg.M):                # every minibatch window boundary
        e = int(np.searchsorted(s.offsets, b, side="right")) - 1
        t0 = int(s.offsets[e]) + -(-(b - int(s.offsets[e])) // 256) * 256
        for r in (b - 1, b, t0 - 1, t0):
            if 0 <= r < s.R:
                rows.add(r)
    toks = np.unique(s.perm[sorted(rows)] // cfg.k)
    local = (ids >= cfg.e0) & (ids < cfg.e0 + cfg.n_local)
    none = np.flatnonzero(~local.any(axis=1))[:8]
    say(f"[c{c}] oracle on {len(toks)} tokens")
    ref = O.forward_tokens(toks, d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0,
                           mxfp8=True)
    yv = y_values(y)
    fro, worst, stray = row_errors(yv[toks], ref)
    say(f"[c{c}] sampled rel_fro vs MX oracle {fro:.3e}, worst row {worst:.3e}")
    assert fro < TOL_MX and worst < TOL_MX_ROW and stray == 0
    assert np.all(yv[none] == 0)
