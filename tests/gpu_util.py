"""Helpers for the GPU tests: move seeded inputs to the device and run the library."""
from __future__ import annotations

import sys

import numpy as np
import torch

from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd.layer import MoKLayer, bf16_tensor, bf16_values


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class DevInputs:
    def __init__(self, d: dict, ids: np.ndarray | None = None, device="cuda"):
        self.x = bf16_tensor(d["x_bits"], device)
        self.ids = torch.from_numpy(np.ascontiguousarray(d["ids"] if ids is None else ids)).to(device)
        self.gates = torch.from_numpy(np.ascontiguousarray(d["gates"])).to(device)
        self.wg = bf16_tensor(d["wg_bits"], device)
        self.wu = bf16_tensor(d["wu_bits"], device)
        self.wd = bf16_tensor(d["wd_bits"], device)
        self.dy = bf16_tensor(d["dy_bits"], device) if "dy_bits" in d else None


def run_forward(cfg, dev: DevInputs, *, flags=0, **over):
    desc = L.desc_from_config(cfg, flags=flags, **over)
    layer = MoKLayer(desc)
    layer.schedule(dev.ids)
    y = layer.forward(dev.x, dev.ids, dev.gates, dev.wg, dev.wu, dev.wd)
    torch.cuda.synchronize()
    return y, layer


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def y_values(y: torch.Tensor) -> np.ndarray:
    return bf16_values(y)


def row_errors(got, ref) -> tuple[float, float, int]:
    """(relative Frobenius error, largest per-row relative error over rows whose reference
    is non-zero, number of rows whose reference is zero but got is not).  A row's relative
    error is ||got_t - ref_t|| / ||ref_t||."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rn = np.linalg.norm(ref, axis=1)
    dn = np.linalg.norm(got - ref, axis=1)
    nz = rn > 0
    worst = float((dn[nz] / rn[nz]).max()) if nz.any() else 0.0
    stray = int(np.count_nonzero(np.any(got[~nz] != 0, axis=1)))
    return rel_fro(got, ref), worst, stray
