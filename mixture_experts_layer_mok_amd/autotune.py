"""Per-shape choice of the minibatch size M and the comm/compute CU split.

The best minibatch and the best split between data-moving and matrix-core workgroups
shift with the hidden size, top-k and expert count (news brief on MoK, benchmark
section).  This module measures them on the device for one layer shape and keeps the
result in a JSON cache keyed by that shape, so a caller tunes once per shape and reuses
the choice.  Tuning runs the library's own schedule and forward on the caller's inputs;
it changes launch parameters only, never the arithmetic: the forward output is bitwise
the same for every M and split (m-tiles start at expert offsets, and the combine order
is fixed), which the GPU tests check.

Search: coordinate descent over two small grids, comm CUs first at the starting M, then
M at the best split, then the split again at the best M.  Each candidate is timed as the
median of `steps` schedule + forward calls after `warmup` calls, with HIP events on the
current stream.
"""
from __future__ import annotations

import json
import os
from dataclasses import asdict, dataclass

from . import _lib as L
from .tuning import layer_two_wave_min_rows


@dataclass(frozen=True)
class ShapeKey:
    """What the choice depends on: the layer shape, the precision, the device and the
    routed-row count rounded up to a power of two (routing skew moves R)."""
    T: int
    D: int
    I: int
    E: int
    E_loc: int
    k: int
    precision: int
    r_bucket: int
    device: str
    cus: int

    def text(self) -> str:
        return (f"T{self.T}_D{self.D}_I{self.I}_E{self.E}_L{self.E_loc}_k{self.k}"
                f"_p{self.precision}_R{self.r_bucket}_{self.device}_cu{self.cus}")


def r_bucket(routed_rows: int) -> int:
    """Smallest power of two >= routed_rows (at least 1)."""
    b = 1
    while b < max(1, routed_rows):
        b *= 2
    return b


def shape_key(desc: L.mok_desc_t, routed_rows: int, device: str, cus: int) -> ShapeKey:
    return ShapeKey(desc.num_tokens, desc.hidden, desc.intermediate, desc.num_experts,
                    desc.num_local_experts, desc.top_k, desc.precision, r_bucket(routed_rows),
                    device, cus)


def candidate_minibatches(routed_rows: int, cus: int, comm_cus: int, intermediate: int,
                          m_min: int = 512, m_max: int = 8192) -> list[int]:
    """Minibatch sizes (multiples of 512) around the two-waves threshold: from a quarter
    of it to twice it, within [m_min, m_max] and not above the routed rows rounded up."""
    two = layer_two_wave_min_rows(cus, comm_cus, intermediate)
    hi = min(m_max, max(m_min, -(-max(routed_rows, 1) // 512) * 512))
    out = []
    for f in (0.25, 0.375, 0.5, 0.75, 1.0, 1.5, 2.0):
        m = int(round(two * f / 512.0)) * 512
        m = min(max(m, m_min), hi)
        if m not in out:
            out.append(m)
    return sorted(out)


def candidate_comm_cus(cus: int, precision: int) -> list[int]:
    """Data-mover workgroup counts: multiples of 4 (at least 8), a small share of the CUs;
    MXFP8 quantises on the gather and moves more rows per flop, so its range is higher."""
    lo, hi = (16, cus // 4) if precision == L.MOK_PREC_MXFP8 else (8, cus // 8)
    step = max(4, (hi - lo) // 5 // 4 * 4)
    return [c for c in range(lo, hi + 1, step) if 1 <= c <= cus - 1]


@dataclass
class Choice:
    minibatch_rows: int
    comm_cus: int
    fwd_ms: float
    trials: list

    def to_json(self) -> dict:
        return asdict(self)


def load_cache(path: str | None) -> dict:
    if not path or not os.path.exists(path):
        return {}
    with open(path) as f:
        return json.load(f)


def save_cache(path: str, cache: dict) -> None:
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(cache, f, indent=1, sort_keys=True)
    os.replace(tmp, path)


def tune(desc: L.mok_desc_t, x, ids, gates, wg, wu, wd, scales=(None, None, None), *,
         steps: int = 5, warmup: int = 2, cache_path: str | None = None,
         comm_grid: list[int] | None = None, m_grid: list[int] | None = None) -> Choice:
    """Best (M, comm_cus) for this shape on the current device.  desc gives the shape, the
    ring slots and the starting M / split; inputs are device tensors as for the forward.
    With cache_path, a cached choice for the same ShapeKey is returned without timing, and
    a new choice is written back."""
    import statistics

    import torch

    from .layer import MoKLayer

    dev = x.device
    cus = L.mok_device_cus()
    probe = MoKLayer(desc, device=dev)
    probe.schedule(ids)
    R = probe.tables()["R"]
    del probe
    key = shape_key(desc, R, torch.cuda.get_device_name(dev), cus).text()
    cache = load_cache(cache_path)
    if key in cache:
        c = cache[key]
        return Choice(c["minibatch_rows"], c["comm_cus"], c["fwd_ms"], c.get("trials", []))

    y = torch.empty((desc.num_tokens, desc.hidden), dtype=torch.bfloat16, device=dev)
    timed: dict[tuple[int, int], float] = {}
    trials = []

    def time_one(M: int, comm: int) -> float:
        if (M, comm) in timed:
            return timed[(M, comm)]
        d = L.make_desc(desc.num_tokens, desc.hidden, desc.intermediate, desc.num_experts,
                        desc.top_k, e0=desc.expert_begin, E_loc=desc.num_local_experts, M=M,
                        S=desc.ring_slots, comm_cus=comm, precision=desc.precision)
        layer = MoKLayer(d, device=dev)
        stream = torch.cuda.current_stream(dev)
        for _ in range(warmup):
            layer.schedule(ids)
            layer.forward(x, ids, gates, wg, wu, wd, scales=scales, y=y)
        ms = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            layer.schedule(ids)
            layer.forward(x, ids, gates, wg, wu, wd, scales=scales, y=y)
            e1.record(stream)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        st = layer.status()
        del layer
        torch.cuda.empty_cache()
        if st != 0:
            raise RuntimeError(f"device status {st:#x} while tuning M={M} comm_cus={comm}")
        t = float(statistics.median(ms))
        timed[(M, comm)] = t
        trials.append({"minibatch_rows": M, "comm_cus": comm, "fwd_ms": round(t, 4)})
        return t

    comms = comm_grid or candidate_comm_cus(cus, desc.precision)
    M = desc.minibatch_rows
    comm = min(comms, key=lambda c: time_one(M, c))
    ms_grid = m_grid or candidate_minibatches(R, cus, comm, desc.intermediate)
    M = min(ms_grid, key=lambda m: time_one(m, comm))
    comm = min(comms, key=lambda c: time_one(M, c))
    best = min(timed, key=timed.get)
    choice = Choice(best[0], best[1], round(timed[best], 4), trials)
    if cache_path:
        cache[key] = choice.to_json()
        save_cache(cache_path, cache)
    return choice
