"""Seeded synthetic inputs for the MoE layer, shared by the tests, the benchmark and
the oracle's callers.

This module only draws random numbers and converts storage formats.  It holds none
of the layer's arithmetic: the schedule, the expert FFN, the combine and the MX
quantiser live in the HIP library and, independently, in the oracle.

Draw order per configuration (NumPy PCG64, ``default_rng(seed)``; the seed defaults
to the configuration number):  X, router logits, W_gate, W_up, W_down, dY.
All draws are float32 normals; tensors the device reads as bf16 are rounded to
bf16 (round to nearest even) once, here, and both sides read those rounded values.

Routing is upstream of the layer: the generator turns logits into top-k expert ids
(k largest logits, descending, ties to the lower id) and gates (softmax over the
selected logits).  Both the GPU path and the oracle read the same ids and gates.
The Zipf-skewed variant adds ln p_e with p_e proportional to (e+1)^-s to every
token's logits, so low expert ids are the popular ones.  Its permuted-rank variant gives
expert e the popularity rank perm[e] instead, with perm a permutation of the expert ids
drawn from its own generator (``default_rng(zipf_perm_seed)``, outside the draw order
above), so that the local experts hold ranks spread over the whole range.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

PREC_BF16 = 0
PREC_MXFP8 = 1


@dataclass(frozen=True)
class LayerConfig:
    """Shape and launch parameters of one layer call (mirrors ``mok_desc_t``)."""

    name: str
    T: int                  # pool tokens
    D: int                  # hidden size
    I: int                  # expert intermediate size
    E: int                  # total experts
    k: int                  # top-k
    e0: int = 0             # first local expert
    E_loc: int = 0          # local experts (0 -> all E)
    M: int = 32             # minibatch rows
    S: int = 2              # ring slots
    comm_cus: int = 32      # workgroups given to dispatch/combine in the fused kernel
    precision: int = PREC_BF16
    zipf_s: float = 0.0     # 0 -> uniform router logits
    zipf_perm_seed: int = -1  # >= 0: popularity ranks permuted over the expert ids
    x_std: float = 1.0
    w_std: float = 0.02

    @property
    def n_local(self) -> int:
        return self.E_loc if self.E_loc > 0 else self.E

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  c3/c4/c5 are one GPU's share of an expert-parallel layer of
# hidden 7168 / expert intermediate 2048 with 64 experts, top-8, 8 local experts
# and 2048 tokens from each of 8 sources (a 16384-token pool).
CONFIGS = {
    1: LayerConfig("c1-tiny-fwd", T=128, D=128, I=64, E=4, k=2, M=32, S=2, comm_cus=8),
    2: LayerConfig("c2-small-fwd-bf16", T=4096, D=2048, I=1024, E=16, k=4, M=1024, S=2,
                   comm_cus=32),
    # comm_cus: the best of the minibatch x comm-CU sweeps of the fused forward
    3: LayerConfig("c3-share-fwd-bf16", T=16384, D=7168, I=2048, E=64, k=8, E_loc=8, M=2048,
                   S=4, comm_cus=20),
    # the skewed load puts ~86k rows on this GPU, which the data movers quantise and
    # combine (about five slots per token): they need more CUs than the even share
    4: LayerConfig("c4-share-zipf-fwd-mxfp8", T=16384, D=7168, I=2048, E=64, k=8, E_loc=8,
                   M=2048, S=4, comm_cus=32, precision=PREC_MXFP8, zipf_s=1.2),
    # eight ring slots (about 61 MB each) hold every minibatch of this share, so the
    # backward finds a and b of all of them in the ring and replays nothing; with no slot
    # to recycle, the data movers only gather and combine, and 16 of them suffice (the
    # per-shape tuner and a comm-CU sweep of the whole step agree)
    5: LayerConfig("c5-share-fwd-bwd-bf16", T=16384, D=7168, I=2048, E=64, k=8, E_loc=8,
                   M=2048, S=8, comm_cus=16),
    # config 4's skew with the popularity ranks permuted: this GPU's eight experts get
    # ranks spread over the range and hold about 3.8k routed rows, two minibatches; M and
    # comm_cus are the per-shape tuner's choice (forward 0.450 -> 0.434 ms against M = 2048
    # on 32 comm CUs)
    6: LayerConfig("c6-share-zipf-permuted-mxfp8", T=16384, D=7168, I=2048, E=64, k=8,
                   E_loc=8, M=3072, S=4, comm_cus=16, precision=PREC_MXFP8, zipf_s=1.2,
                   zipf_perm_seed=1004),
}


# ---------------------------------------------------------------------------------
# storage conversion (bf16 is carried as uint16 bit patterns)
# ---------------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16, nearest-even; returns uint16 bit patterns.  Inputs here
    are finite normal draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


# ---------------------------------------------------------------------------------
# routing (upstream of the layer; only produces inputs)
# ---------------------------------------------------------------------------------
def route_topk(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-k ids (descending logit, ties to lower id) and softmax gates over them."""
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    sel = sel - sel.max(axis=1, keepdims=True)
    g = np.exp(sel)
    g = g / g.sum(axis=1, keepdims=True)
    return order.astype(np.int32), g.astype(np.float32)


def zipf_bias(E: int, s: float) -> np.ndarray:
    p = (np.arange(E, dtype=np.float64) + 1.0) ** (-s)
    p = p / p.sum()
    return np.log(p).astype(np.float32)


# ---------------------------------------------------------------------------------
# full input set
# ---------------------------------------------------------------------------------
def make_inputs(cfg: LayerConfig, seed: int | None = None, *, with_dy: bool = False) -> dict:
    """Draw one seeded input set for ``cfg``.

    Returns a dict with
      x_bits  uint16 [T, D]          (bf16)      x   float32 [T, D] (same values)
      ids     int32  [T, k]                      gates float32 [T, k]
      wg_bits, wu_bits uint16 [E_loc, I, D]      wg, wu float32
      wd_bits uint16 [E_loc, D, I]               wd  float32
      dy_bits / dy when ``with_dy``
    Only the local experts' weights are drawn; index 0 is expert e0.
    """
    if seed is None:
        seed = int(cfg.name[1]) if cfg.name[:1] == "c" and cfg.name[1:2].isdigit() else 0
    rng = np.random.default_rng(seed)
    T, D, I, E, k = cfg.T, cfg.D, cfg.I, cfg.E, cfg.k
    nl = cfg.n_local
    x = rng.standard_normal((T, D), dtype=np.float32)
    if cfg.x_std != 1.0:
        x *= np.float32(cfg.x_std)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if cfg.zipf_s > 0:
        bias = zipf_bias(E, cfg.zipf_s)
        if cfg.zipf_perm_seed >= 0:
            bias = bias[np.random.default_rng(cfg.zipf_perm_seed).permutation(E)]
        logits = logits + bias[None, :]
    ids, gates = route_topk(logits, k)
    wg = rng.standard_normal((nl, I, D), dtype=np.float32) * np.float32(cfg.w_std)
    wu = rng.standard_normal((nl, I, D), dtype=np.float32) * np.float32(cfg.w_std)
    wd = rng.standard_normal((nl, D, I), dtype=np.float32) * np.float32(cfg.w_std)
    out = {"x_raw": None}
    out["x_bits"] = f32_to_bf16_bits(x)
    out["x"] = bf16_bits_to_f32(out["x_bits"])
    if T * D <= (1 << 16):
        out["x_raw"] = x          # unrounded draws, kept only for tiny configs
    del x
    out["ids"] = ids
    out["gates"] = gates
    for name, w in (("wg", wg), ("wu", wu), ("wd", wd)):
        out[name + "_bits"] = f32_to_bf16_bits(w)
        out[name] = bf16_bits_to_f32(out[name + "_bits"])
    del wg, wu, wd
    if with_dy:
        dy = rng.standard_normal((T, D), dtype=np.float32)
        out["dy_bits"] = f32_to_bf16_bits(dy)
        out["dy"] = bf16_bits_to_f32(out["dy_bits"])
    return out


def mask_ids(ids: np.ndarray, frac: float, seed: int) -> np.ndarray:
    """Return a copy of ids with a random fraction of entries set to -1 (masked)."""
    rng = np.random.default_rng(seed)
    m = rng.random(ids.shape) < frac
    out = ids.copy()
    out[m] = -1
    return out


def small_config(name: str, T: int, D: int, I: int, E: int, k: int, M: int, *, e0: int = 0,
                 E_loc: int = 0, S: int = 2, comm_cus: int = 8, precision: int = PREC_BF16,
                 zipf_s: float = 0.0) -> LayerConfig:
    return LayerConfig(name, T=T, D=D, I=I, E=E, k=k, e0=e0, E_loc=E_loc, M=M, S=S,
                       comm_cus=comm_cus, precision=precision, zipf_s=zipf_s)
