"""Pins for the CPU oracle: each test checks the oracle against something other than
itself — hand-worked fixtures, library routines (torch autograd, torch.nn.functional,
torch's float8_e4m3fn conversion, NumPy's sort), brute force on tiny inputs,
finite differences, closed forms and invariants."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from mixture_experts_layer_mok_amd import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------------
# schedule
# ---------------------------------------------------------------------------------
def test_schedule_golden():
    for c in _load("schedule_tiny.json")["cases"]:
        ids = np.array(c["ids"], dtype=np.int32)
        s = O.schedule(ids, c["e0"], c["n_local"], c["E"], c["M"])
        assert s.counts.tolist() == c["counts"]
        assert s.offsets.tolist() == c["offsets"]
        assert s.perm.tolist() == c["perm"]
        assert s.pos.tolist() == c["pos"]
        assert [list(x) for x in s.segments()] == c["segments"]
        assert s.bad == c["bad"]


def _brute_schedule(ids, e0, n_local):
    """Python loops: for every local expert in order, walk tokens then slots."""
    T, k = ids.shape
    perm = []
    for e in range(e0, e0 + n_local):
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    perm.append(t * k + j)
    return perm


@pytest.mark.parametrize("T,k,E,e0,nl,mask", [(37, 3, 7, 2, 4, 0.0), (64, 8, 64, 0, 8, 0.0),
                                              (50, 2, 5, 0, 5, 0.3), (16, 4, 4, 3, 1, 0.1)])
def test_schedule_brute_and_invariants(T, k, E, e0, nl, mask):
    rng = np.random.default_rng(T * 31 + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if mask:
        ids = gen.mask_ids(ids, mask, seed=T)
    s = O.schedule(ids, e0, nl, E, M=5)
    assert s.perm.tolist() == _brute_schedule(ids, e0, nl)
    n_local_pairs = int(np.count_nonzero((ids >= e0) & (ids < e0 + nl)))
    assert int(s.counts.sum()) == n_local_pairs == s.R
    # perm is a bijection onto the local pairs, pos inverts it
    assert len(set(s.perm.tolist())) == s.R
    assert np.array_equal(s.pos[s.perm], np.arange(s.R))
    assert np.count_nonzero(s.pos >= 0) == s.R
    # rows sorted by (expert, token, slot)
    key = (ids.reshape(-1)[s.perm].astype(np.int64) * (T * k)) + s.perm
    assert np.all(np.diff(key) > 0)
    # minibatch segments tile [0, R) exactly, each inside one expert and one window
    covered = []
    for mb, e, a, b in s.segments():
        assert mb * 5 <= a < b <= min((mb + 1) * 5, s.R)
        assert s.offsets[e] <= a and b <= s.offsets[e + 1]
        covered.extend(range(a, b))
    assert covered == list(range(s.R))


def test_schedule_all_to_one_and_empty():
    ids = np.full((10, 2), 3, dtype=np.int32)
    s = O.schedule(ids, 0, 6, 6, M=4)
    assert s.counts.tolist() == [0, 0, 0, 20, 0, 0]
    assert s.perm.tolist() == list(range(20))
    s2 = O.schedule(np.full((10, 2), -1, dtype=np.int32), 0, 6, 6, M=4)
    assert s2.R == 0 and s2.n_mb == 0 and s2.bad == 0 and np.all(s2.pos == -1)


# ---------------------------------------------------------------------------------
# MX codec
# ---------------------------------------------------------------------------------
def test_e4m3_decode_matches_spec_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    for v in _load("e4m3_spec_values.json")["values"]:
        got = O.e4m3_decode(np.array([int(v["code"], 16)], dtype=np.uint8))[0]
        if v["value"] == "nan":
            assert np.isnan(got)
        else:
            assert got == v["value"] and np.signbit(got) == np.signbit(v["value"])


def test_e4m3_roundtrip_exhaustive():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes).astype(np.float32)), codes)


def _nearest_even_brute(v):
    """Search the 253 finite non-negative-zero code values for the nearest; on a tie
    take the code with an even mantissa.  Saturates at 448."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.int64)
    vals = O.e4m3_decode(codes.astype(np.uint8))
    out = []
    for x in v:
        x = float(np.float32(x))
        x = min(max(x, -448.0), 448.0)
        same_sign = codes[(np.signbit(vals) == np.signbit(x)) | (vals == 0)]
        cv = O.e4m3_decode(same_sign.astype(np.uint8))
        d = np.abs(cv - x)
        best = same_sign[d == d.min()]
        vb = O.e4m3_decode(best.astype(np.uint8))
        best = best[np.signbit(vb) == np.signbit(x)] if np.any(np.signbit(vb) == np.signbit(x)) else best
        if len(best) > 1:
            best = best[(best & 1) == 0]
        out.append(int(best[0]))
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_vs_torch_and_brute():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(4000) * 50,
        rng.standard_normal(2000) * 0.01,
        (rng.integers(-3000, 3000, 2000) + 0.5) * 2.0 ** -9,   # ties in the subnormal range
        np.ldexp(1.0 + (rng.integers(0, 8, 500) * 2 + 1) / 16.0, rng.integers(-6, 8, 500)),  # ties
        [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10, 1.9375 * 2 ** -7],
    ]).astype(np.float32)
    v = np.clip(v, -448, 448)
    ours = O.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    idx = rng.choice(v.size, 600, replace=False)
    assert np.array_equal(ours[idx], _nearest_even_brute(v[idx]))
    # saturation above the largest finite value
    assert O.e4m3_encode(np.array([1e4, -600.0], np.float32)).tolist() == [0x7E, 0xFE]


def test_mx_blocks_golden():
    for blk in _load("mx_blocks.json")["blocks"]:
        v = np.full(32, blk["fill"], dtype=np.float32)
        for i, x in blk["set"].items():
            v[int(i)] = x
        codes, scales = O.mx_quantize(v[None, :])
        assert scales.tolist() == [[blk["scale"]]]
        for i in range(32):
            want = blk["codes"].get(str(i), blk["codes"]["*"])
            assert codes[0, i] == want, (blk, i)


def test_mx_scale_rule_properties():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((2000, 64)) * np.exp(rng.uniform(-30, 30, (2000, 1)))).astype(
        np.float32)
    v[5] = 0.0
    codes, scales = O.mx_quantize(v)
    amax = np.abs(v.reshape(2000, 2, 32)).max(-1).astype(np.float64)
    n = scales.astype(np.int64) - 127
    nz = amax > 0
    # smallest power of two that brings the block inside the e4m3 range
    assert np.all(amax[nz] * np.ldexp(1.0, -n[nz]) <= 448.0)
    assert np.all(amax[nz] * np.ldexp(1.0, -(n[nz] - 1)) > 448.0)
    assert np.all(scales[~nz] == 0)
    # boundary: exactly 448 * 2^n keeps n, the next float32 up moves to n + 1
    for n0 in (-20, 0, 5):
        a = np.float32(448.0 * 2.0 ** n0)
        assert O.mx_scale_exponent(np.array([a]))[0] == n0
        assert O.mx_scale_exponent(np.array([np.nextafter(a, np.float32(np.inf))]))[0] == n0 + 1
    # dequantised block error is bounded by half an e4m3 step (relative 2^-4) above 2^-6
    deq = O.mx_dequantize(codes, scales)
    big = np.abs(v) * np.ldexp(1.0, -np.repeat(n, 32, axis=1)) >= 2.0 ** -6
    rel = np.abs(deq - v)[big] / np.abs(v)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-12


# ---------------------------------------------------------------------------------
# expert FFN and forward
# ---------------------------------------------------------------------------------
def _torch_layer(x, ids, gates, wg, wu, wd, e0, requires_grad=False):
    """The layer written with torch library ops and per-expert masks (no schedule)."""
    X = torch.tensor(x, dtype=torch.float64, requires_grad=requires_grad)
    G = torch.tensor(gates, dtype=torch.float64, requires_grad=requires_grad)
    Wg = torch.tensor(wg, dtype=torch.float64, requires_grad=requires_grad)
    Wu = torch.tensor(wu, dtype=torch.float64, requires_grad=requires_grad)
    Wd = torch.tensor(wd, dtype=torch.float64, requires_grad=requires_grad)
    Y = torch.zeros_like(X)
    idt = torch.tensor(ids.astype(np.int64))
    for e in range(wg.shape[0]):
        tok, slot = torch.nonzero(idt == e + e0, as_tuple=True)
        if tok.numel() == 0:
            continue
        hid = F.silu(F.linear(X[tok], Wg[e])) * F.linear(X[tok], Wu[e])
        out = F.linear(hid, Wd[e]) * G[tok, slot][:, None]
        Y = Y.index_add(0, tok, out)
    return Y, (X, G, Wg, Wu, Wd)


def _small(T=48, D=64, I=32, E=6, k=2, e0=0, nl=0, M=16, seed=11, zipf=0.0):
    cfg = gen.small_config("t", T, D, I, E, k, M, e0=e0, E_loc=nl, zipf_s=zipf)
    return cfg, gen.make_inputs(cfg, seed=seed, with_dy=True)


def test_dense_swiglu_special_case():
    """E = 1, k = 1, gate 1: the layer is a dense SwiGLU FFN."""
    cfg, d = _small(T=20, D=64, I=32, E=1, k=1, M=8)
    gates = np.ones_like(d["gates"])
    y = O.forward(d["x"], d["ids"], gates, d["wg"], d["wu"], d["wd"], e0=0, E=1, M=8)
    X = torch.tensor(d["x"], dtype=torch.float64)
    ref = F.linear(F.silu(F.linear(X, torch.tensor(d["wg"][0], dtype=torch.float64))) *
                   F.linear(X, torch.tensor(d["wu"][0], dtype=torch.float64)),
                   torch.tensor(d["wd"][0], dtype=torch.float64)).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("args", [dict(), dict(E=8, k=3, e0=2, nl=4), dict(zipf=1.2, E=8, k=4)])
def test_forward_vs_torch_layer(args):
    cfg, d = _small(**args)
    ids = gen.mask_ids(d["ids"], 0.1, seed=5)
    y = O.forward(d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0, E=cfg.E,
                  M=cfg.M)
    ref, _ = _torch_layer(d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], cfg.e0)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-10, atol=1e-13)


def test_forward_config1_and_tokenwise():
    cfg = gen.CONFIGS[1]
    d = gen.make_inputs(cfg)
    y = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=cfg.E,
                  M=cfg.M)
    ref, _ = _torch_layer(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], 0)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-10, atol=1e-13)
    toks = [0, 5, 77, 127]
    yt = O.forward_tokens(toks, d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0)
    np.testing.assert_allclose(yt, y[toks], rtol=1e-12, atol=1e-14)
    # the minibatch size does not change the result
    y2 = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=cfg.E, M=7)
    assert np.array_equal(y, y2)


def test_forward_linear_in_gates_and_permutation_equivariant():
    cfg, d = _small(T=40, E=5, k=2)
    args = (d["wg"], d["wu"], d["wd"])
    y = O.forward(d["x"], d["ids"], d["gates"], *args, e0=0, E=5, M=9)
    y2 = O.forward(d["x"], d["ids"], 2.5 * d["gates"].astype(np.float64), *args, e0=0, E=5, M=9)
    np.testing.assert_allclose(y2, 2.5 * y, rtol=1e-12, atol=1e-14)
    p = np.random.default_rng(0).permutation(40)
    yp = O.forward(d["x"][p], d["ids"][p], d["gates"][p], *args, e0=0, E=5, M=9)
    np.testing.assert_allclose(yp, y[p], rtol=1e-12, atol=1e-14)


def test_forward_mxfp8_oracle():
    cfg, d = _small(T=40, D=64, I=64, E=4, k=2)
    yq, parts = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=4,
                          M=16, mxfp8=True, return_parts=True)
    y = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=4, M=16)
    rel = np.linalg.norm(yq - y) / np.linalg.norm(y)
    assert 1e-3 < rel < 0.15       # MX rounding is visible but bounded
    toks = [1, 17, 39]
    yt = O.forward_tokens(toks, d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0,
                          mxfp8=True)
    np.testing.assert_allclose(yt, yq[toks], rtol=1e-11, atol=1e-13)
    # H was quantised: each row's values are e4m3 values times a power of two
    h = parts["h"]
    codes, scales = O.mx_quantize(h.astype(np.float32))
    assert np.array_equal(O.mx_dequantize(codes, scales), h)


def _torch_mx_roundtrip(v: torch.Tensor) -> torch.Tensor:
    """MX round trip written independently of the oracle, with torch's float8_e4m3fn cast:
    blocks of 32 along the last axis; the shared scale is 2^n for the smallest integer n
    with max|v| 2^-n <= 448 (the largest finite e4m3 value), n clamped to [-127, 127].
    The block values are read as float32 (what the quantisers read)."""
    v32 = v.to(torch.float32).to(torch.float64)
    K = v32.shape[-1]
    blk = v32.reshape(*v32.shape[:-1], K // 32, 32)
    amax = blk.abs().amax(dim=-1)
    _, e = torch.frexp(amax)                      # amax = m 2^e, m in [0.5, 1)
    base = e.to(torch.int64) - 9                  # floor(log2 amax) - 8
    n = base + 1                                  # always large enough
    for cand in (base, base - 1):                 # keep the smallest n that still fits
        ok = amax * torch.exp2(-cand.to(torch.float64)) <= 448.0
        n = torch.where(ok, cand, n)
    n = torch.clamp(n, -127, 127)
    scale = torch.exp2(n.to(torch.float64))[..., None]
    q = (blk / scale).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64) * scale
    return q.reshape(v32.shape)


def _torch_mx_layer(x, ids, gates, wg, wu, wd, e0, transposed=()):
    """The MXFP8 layer as per-expert masked torch products (no schedule), with the MX round
    trip applied where each GEMM reads its operands: X rows and W_gate / W_up along D (their
    K), W_down along I (its K), and H along I after SwiGLU, from its float32 value.
    `transposed` names quantisation points ("x", "wgu", "wd", "h") whose blocks are taken
    along the other axis instead (a planted mistake, to show the comparison notices it)."""
    def q(v, name):
        if name not in transposed:
            return _torch_mx_roundtrip(v)
        n = v.shape[0]
        pad = torch.zeros((v.shape[1], -n % 32), dtype=v.dtype)   # zeros leave amax as is
        return _torch_mx_roundtrip(torch.cat([v.T, pad], dim=1))[:, :n].T

    X = torch.tensor(x, dtype=torch.float64)
    G = torch.tensor(gates, dtype=torch.float64)
    Y = torch.zeros_like(X)
    idt = torch.tensor(ids.astype(np.int64))
    for e in range(wg.shape[0]):
        tok, slot = torch.nonzero(idt == e + e0, as_tuple=True)
        if tok.numel() == 0:
            continue
        Wg = q(torch.tensor(wg[e], dtype=torch.float64), "wgu")   # [I, D], K = D
        Wu = q(torch.tensor(wu[e], dtype=torch.float64), "wgu")
        Wd = q(torch.tensor(wd[e], dtype=torch.float64), "wd")    # [D, I], K = I
        Xq = q(X[tok], "x")
        hid = F.silu(F.linear(Xq, Wg)) * F.linear(Xq, Wu)
        out = F.linear(q(hid.to(torch.float32).to(torch.float64), "h"), Wd) * G[tok, slot][:, None]
        Y = Y.index_add(0, tok, out)
    return Y


def _wide_range_inputs(d):
    """Rescale an input set so that every 32-block along each GEMM's K spans many binades.
    With power-of-two block scales, e4m3 rounds normal-range values the same whatever the
    block, so only the values that a block's scale pushes into the subnormal range (or
    flushes) show which axis the blocks run along; and such a value must meet a large
    partner in its product to reach the output.  So the two operands of each GEMM get
    complementary patterns along K: X columns 2^-(d mod 24), W_gate / W_up columns
    2^-((d + 12) mod 24); W_gate / W_up rows 2^-floor((i mod 24) / 2), which makes H span
    about 24 binades along I; W_down columns 2^-((i + 12) mod 24)."""
    out = dict(d)
    D, I = d["wg"].shape[2], d["wg"].shape[1]
    dd, ii = np.arange(D), np.arange(I)
    px = np.ldexp(1.0, -(dd % 24)).astype(np.float32)
    pwd = np.ldexp(1.0, -((dd + 12) % 24)).astype(np.float32)
    pwi = np.ldexp(1.0, -((ii % 24) // 2)).astype(np.float32)
    pdi = np.ldexp(1.0, -((ii + 12) % 24)).astype(np.float32)
    out["x"] = (d["x"] * px[None, :]).astype(np.float32)
    out["wg"] = (d["wg"] * pwd[None, None, :] * pwi[None, :, None]).astype(np.float32)
    out["wu"] = (d["wu"] * pwd[None, None, :] * pwi[None, :, None]).astype(np.float32)
    out["wd"] = (d["wd"] * pdi[None, None, :]).astype(np.float32)
    return out


@pytest.mark.parametrize("args", [dict(T=40, D=64, I=64, E=4, k=2),
                                  dict(T=64, D=256, I=96, E=8, k=3, e0=2, nl=4, zipf=1.2)])
def test_forward_mxfp8_composition_vs_torch_float8(args):
    """The oracle's MXFP8 forward equals an emulation built from torch's float8 cast and
    per-32-block power-of-two scales along each GEMM's K, on inputs whose blocks span 24
    binades.  Taking any one of the four quantisation points along the other axis moves
    the emulation far beyond the 1e-12 bound, so a wrong block axis (or a missing round
    trip) in the oracle would fail here."""
    cfg, d = _small(**args)
    d = _wide_range_inputs(d)
    ids = gen.mask_ids(d["ids"], 0.1, seed=4)
    y = O.forward(d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0, E=cfg.E,
                  M=cfg.M, mxfp8=True)
    args_t = (d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], cfg.e0)
    ref = _torch_mx_layer(*args_t).numpy()
    nref = np.linalg.norm(ref)
    assert np.linalg.norm(y - ref) <= 1e-12 * nref
    for point in ("x", "wgu", "wd", "h"):
        alt = _torch_mx_layer(*args_t, transposed=(point,)).numpy()
        assert np.linalg.norm(alt - ref) > 1e-9 * nref, point
    # the emulation's quantiser itself agrees with the oracle's codes and scales
    v = np.random.default_rng(3).standard_normal((8, 96)).astype(np.float32) * 7.0
    v *= np.ldexp(1.0, -(np.arange(96) % 24)).astype(np.float32)
    np.testing.assert_array_equal(_torch_mx_roundtrip(torch.tensor(v)).numpy(),
                                  O.mx_roundtrip(v))


# ---------------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("args", [dict(), dict(E=8, k=3, e0=2, nl=4, T=30)])
def test_backward_vs_torch_autograd(args):
    cfg, d = _small(**args)
    ids = gen.mask_ids(d["ids"], 0.1, seed=9)
    g = O.backward(d["dy"], d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0,
                   E=cfg.E, M=cfg.M)
    Y, (X, G, Wg, Wu, Wd) = _torch_layer(d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"],
                                         cfg.e0, requires_grad=True)
    (Y * torch.tensor(d["dy"], dtype=torch.float64)).sum().backward()
    for ours, ref in ((g["dx"], X.grad), (g["dg"], G.grad), (g["dwg"], Wg.grad),
                      (g["dwu"], Wu.grad), (g["dwd"], Wd.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-9, atol=1e-12)


def test_backward_finite_differences():
    cfg, d = _small(T=12, D=32, I=16, E=3, k=2, M=5)
    args = dict(e0=0, E=3, M=5)
    g = O.backward(d["dy"], d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], **args)
    dy = d["dy"].astype(np.float64)

    def loss(x, gates, wg, wu, wd):
        return float(np.sum(O.forward(x, d["ids"], gates, wg, wu, wd, **args) * dy))

    base = [d["x"].astype(np.float64), d["gates"].astype(np.float64),
            d["wg"].astype(np.float64), d["wu"].astype(np.float64), d["wd"].astype(np.float64)]
    names = ["dx", "dg", "dwg", "dwu", "dwd"]
    rng = np.random.default_rng(1)
    h = 1e-6
    for which in range(5):
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in base[which].shape)
            plus = [b.copy() for b in base]
            minus = [b.copy() for b in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - g[names[which]][idx]) <= 1e-6 * max(1.0, abs(fd)), (names[which], idx)


def test_gate_gradient_identity():
    """dG[t, j] = <u, h> equals <dY[t], o> for the same row."""
    cfg, d = _small(T=30, E=4, k=2)
    _, parts = O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=4,
                         M=8, return_parts=True)
    g = O.backward(d["dy"], d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=0, E=4,
                   M=8)
    s = parts["schedule"]
    t = s.perm // 2
    direct = np.sum(d["dy"].astype(np.float64)[t] * parts["o"], axis=1)
    np.testing.assert_allclose(g["dg"].reshape(-1)[s.perm], direct, rtol=1e-10, atol=1e-13)
    assert np.all(g["dg"].reshape(-1)[s.pos < 0] == 0)


def test_two_waves_rule_reproduces_printed_floor():
    """The pages' 2368-token floor for the 7168/2048 shape follows from the two-waves rule
    with 148 compute units and a 128 x 256 tile (tests/golden/two_waves.json)."""
    from mixture_experts_layer_mok_amd.tuning import layer_two_wave_min_rows, two_wave_min_rows
    g = json.load(open(os.path.join(GOLD, "two_waves.json")))
    assert two_wave_min_rows(g["compute_units"], g["tile_m"], g["tile_n"],
                             g["intermediate"]) == g["min_minibatch"]
    # more compute units or a bigger tile raise the floor proportionally
    assert layer_two_wave_min_rows(256, 32, 2048) == 2 * 224 * 256 * 256 / 4096


def test_bf16_round_matches_torch():
    """bf16_round equals torch's float32 -> bfloat16 conversion (round to nearest, ties to
    even) on random values over many binades, on exact ties in both directions, and on
    values whose rounding carries into the exponent."""
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(4096) * np.ldexp(1.0, rng.integers(-60, 60, 4096))).astype(np.float32)
    bits = rng.integers(0, 1 << 16, 512).astype(np.uint32)
    ties = ((bits << 16) | 0x8000).view(np.float32)                 # halfway, both parities
    carry = ((bits << 16) | 0xFFFF).view(np.float32)                # rounds up into the next binade
    for w in (v, ties[np.isfinite(ties)], carry[np.isfinite(carry)], np.float32([0.0, -0.0, 1.0])):
        ref = torch.from_numpy(w).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(O.bf16_round(w), ref)
    # an exact tie with an even kept bit stays, with an odd one rounds away
    assert O.bf16_round(np.float32([1.0 + 2.0 ** -8]))[0] == 1.0
    assert O.bf16_round(np.float32([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def _torch_mx_backward(dy, x, ids, gates, wg, wu, wd, e0, transposed=()):
    """The MXFP8 backward as per-expert masked torch products (no schedule), written apart
    from the oracle: a, b from the MX forward's operands, saved as bfloat16; u from dY rows and W_down^T
    round-tripped along D; dx rows from da, db (rounded to float32, then bfloat16) and
    W_gate^T, W_up^T round-tripped along I; dG and the weight gradients from the unquantised values.  `transposed` names
    quantisation points ("dy", "wdt", "dab", "wgut") taken along the other axis instead."""
    def q(v, name):
        if name not in transposed:
            return _torch_mx_roundtrip(v)
        n = v.shape[0]
        pad = torch.zeros((v.shape[1], -n % 32), dtype=v.dtype)
        return _torch_mx_roundtrip(torch.cat([v.T, pad], dim=1))[:, :n].T

    X = torch.tensor(x, dtype=torch.float64)
    DY = torch.tensor(dy, dtype=torch.float64)
    G = torch.tensor(gates, dtype=torch.float64)
    nl = wg.shape[0]
    dX, dG = torch.zeros_like(X), torch.zeros_like(G)
    dWg, dWu = torch.zeros(wg.shape, dtype=torch.float64), torch.zeros(wu.shape, dtype=torch.float64)
    dWd = torch.zeros(wd.shape, dtype=torch.float64)
    idt = torch.tensor(ids.astype(np.int64))
    for e in range(nl):
        tok, slot = torch.nonzero(idt == e + e0, as_tuple=True)
        if tok.numel() == 0:
            continue
        Wg, Wu, Wd = (torch.tensor(w[e], dtype=torch.float64) for w in (wg, wu, wd))
        Xq = _torch_mx_roundtrip(X[tok])
        a = F.linear(Xq, _torch_mx_roundtrip(Wg)).to(torch.float32).to(torch.bfloat16).double()
        b = F.linear(Xq, _torch_mx_roundtrip(Wu)).to(torch.float32).to(torch.bfloat16).double()
        h = F.silu(a) * b
        u = F.linear(q(DY[tok], "dy"), q(Wd.T, "wdt"))          # [n, I]
        g = G[tok, slot][:, None]
        dG[tok, slot] = (u * h).sum(dim=1)
        sg = torch.sigmoid(a)
        da = g * u * b * sg * (1.0 + a * (1.0 - sg))
        db = g * u * a * sg
        dWd[e] = (g * DY[tok]).T @ h
        dWg[e] = da.T @ X[tok]
        dWu[e] = db.T @ X[tok]
        daq = q(da.to(torch.float32).to(torch.bfloat16).to(torch.float64), "dab")
        dbq = q(db.to(torch.float32).to(torch.bfloat16).to(torch.float64), "dab")
        dx = F.linear(daq, q(Wg.T, "wgut")) + F.linear(dbq, q(Wu.T, "wgut"))
        dX = dX.index_add(0, tok, dx)
    return dict(dx=dX.numpy(), dg=dG.numpy(), dwg=dWg.numpy(), dwu=dWu.numpy(), dwd=dWd.numpy())


def _wide_range_bwd_inputs(d):
    """Inputs whose blocks along each backward GEMM's K span many binades, with
    complementary partners (see _wide_range_inputs): dY columns 2^-(d mod 24) against
    W_down rows 2^-((d + 12) mod 24) along D; W_down columns 2^-floor((i mod 24) / 2), so
    that u, da and db vary widely along I, against W_gate / W_up rows 2^-((i + 12) mod 24)."""
    out = dict(d)
    D, I = d["wg"].shape[2], d["wg"].shape[1]
    dd, ii = np.arange(D), np.arange(I)
    f = lambda v: np.ldexp(1.0, -v).astype(np.float32)  # noqa: E731
    out["dy"] = (d["dy"] * f(dd % 24)[None, :]).astype(np.float32)
    out["wd"] = (d["wd"] * f((dd + 12) % 24)[None, :, None] * f((ii % 24) // 2)[None, None, :]
                 ).astype(np.float32)
    out["wg"] = (d["wg"] * f((ii + 12) % 24)[None, :, None]).astype(np.float32)
    out["wu"] = (d["wu"] * f((ii + 12) % 24)[None, :, None]).astype(np.float32)
    return out


@pytest.mark.parametrize("args", [dict(T=40, D=64, I=64, E=4, k=2),
                                  dict(T=64, D=128, I=96, E=8, k=3, e0=2, nl=4, zipf=1.2)])
def test_backward_mxfp8_vs_torch_float8(args):
    """The oracle's MXFP8 backward equals an independent torch-float8 emulation to 1e-12
    on every gradient, on inputs whose blocks span many binades; taking any one of the
    backward's four quantisation points along the other axis moves some gradient far
    beyond that bound, so a wrong block axis in the oracle would fail here.  Without the
    quantisation points (plain inputs) it also stays close to the unquantised backward."""
    cfg, d = _small(**args)
    d = _wide_range_bwd_inputs(d)
    ids = gen.mask_ids(d["ids"], 0.1, seed=6)
    got = O.backward(d["dy"], d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0,
                     E=cfg.E, M=cfg.M, mxfp8=True)
    targs = (d["dy"], d["x"], ids, d["gates"], d["wg"], d["wu"], d["wd"], cfg.e0)
    ref = _torch_mx_backward(*targs)
    for name in ("dx", "dg", "dwg", "dwu", "dwd"):
        assert np.linalg.norm(got[name] - ref[name]) <= 1e-12 * np.linalg.norm(ref[name]), name
    for point in ("dy", "wdt", "dab", "wgut"):
        alt = _torch_mx_backward(*targs, transposed=(point,))
        moved = max(np.linalg.norm(alt[n] - ref[n]) / np.linalg.norm(ref[n]) for n in ref)
        assert moved > 1e-9, point


def test_backward_mxfp8_near_plain():
    """On ordinary inputs the MX backward is the plain backward up to MX rounding."""
    cfg, d = _small(T=48, D=64, I=64, E=4, k=2)
    args = (d["dy"], d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"])
    mx = O.backward(*args, e0=0, E=4, M=16, mxfp8=True)
    plain = O.backward(*args, e0=0, E=4, M=16)
    for name in ("dx", "dg", "dwg", "dwu", "dwd"):
        rel = np.linalg.norm(mx[name] - plain[name]) / np.linalg.norm(plain[name])
        assert 1e-4 < rel < 0.2, (name, rel)
