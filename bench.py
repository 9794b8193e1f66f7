"""Benchmark of the MoE layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--M 2048] [--S 4] [--comm-cus 32]
                    [--unfused] [--no-cpu-baseline]

A step is one pass of the layer over one batch: schedule + forward on one GPU's share of
an expert-parallel layer (hidden 7168, expert intermediate 2048, 64 experts with 8
local, top-8, a 16384-token pool: 2048 tokens from each of 8 sources), inputs resident
in HBM before the timed region.  Prints one JSON line.

`value` is algorithmic TFLOP/s of the step (6*D*I flops per routed row forward).
`roofline` reports the dominant kernel (the fused forward) against the bf16 dense
MFMA peak, timed with HIP events on the stream the kernels run on.
`cpu_baseline` times the float64 NumPy oracle on a bounded sample of the same workload
(its first 8192 tokens) on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--M", type=int, default=None)
    ap.add_argument("--S", type=int, default=None)
    ap.add_argument("--comm-cus", type=int, default=None)
    ap.add_argument("--unfused", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                          "(the layer shards by expert across GPUs, see the design notes)"}))
        sys.exit(2)
    import torch

    from mixture_experts_layer_mok_amd import _lib as L
    from mixture_experts_layer_mok_amd import gen
    from mixture_experts_layer_mok_amd.layer import MoKLayer, bf16_tensor

    L.load()
    cfg = gen.CONFIGS[args.config]
    over = {}
    if args.M:
        over["M"] = args.M
    if args.S:
        over["S"] = args.S
    if args.comm_cus:
        over["comm_cus"] = args.comm_cus
    cfg = cfg.replace(**over)
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    d = gen.make_inputs(cfg)
    dev = torch.device("cuda:0")
    x = bf16_tensor(d["x_bits"], dev)
    ids = torch.from_numpy(d["ids"]).to(dev)
    gates = torch.from_numpy(d["gates"]).to(dev)
    wg, wu, wd = (bf16_tensor(d[n], dev) for n in ("wg_bits", "wu_bits", "wd_bits"))
    flags = L.MOK_FLAG_UNFUSED if args.unfused else 0
    layer = MoKLayer(L.desc_from_config(cfg, flags=flags), device=dev)
    y = torch.empty((cfg.T, cfg.D), dtype=torch.bfloat16, device=dev)
    R = int(((d["ids"] >= cfg.e0) & (d["ids"] < cfg.e0 + cfg.n_local)).sum())
    flops_fwd = 6.0 * cfg.D * cfg.I * R

    stream = torch.cuda.current_stream()

    def step(ev=None):
        layer.schedule(ids)
        if ev is not None:
            ev[0].record(stream)
        layer.forward(x, ids, gates, wg, wu, wd, y=y)
        if ev is not None:
            ev[1].record(stream)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = layer.status()
    if st != 0:
        raise SystemExit(f"device status {st:#x} after warmup")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print("[bench] timed", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    st = layer.status()
    if st != 0:
        raise SystemExit(f"device status {st:#x} after timed steps")

    achieved = flops_fwd / (fwd_ms * 1e-3) / 1e12
    out = {
        "metric": "MoE layer forward TFLOPS (bf16)",
        "value": round(flops_fwd / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={cfg.T} D={cfg.D} I={cfg.I} E={cfg.E} "
                               f"local={cfg.n_local} k={cfg.k}",
                   "routed_rows": R, "minibatch_rows": cfg.M, "ring_slots": cfg.S,
                   "comm_cus": cfg.comm_cus, "mode": "unfused" if args.unfused else "fused"},
        "fwd_ms": round(fwd_ms, 4),
        "schedule_plus_fwd_ms": round(ms_step, 4),
        "routed_rows_per_s": round(R / (ms_step * 1e-3), 1),
        "roofline": {"bound": "mfma", "kernel": "k_fwd_fused" if not args.unfused else "unfused",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle as O
        Ts = min(args.cpu_tokens, cfg.T)
        sub = slice(0, Ts)
        Rs = int(((d["ids"][sub] >= cfg.e0) & (d["ids"][sub] < cfg.e0 + cfg.n_local)).sum())
        t0 = time.time()
        O.forward(d["x"][sub], d["ids"][sub], d["gates"][sub], d["wg"], d["wu"], d["wd"],
                  e0=cfg.e0, E=cfg.E, M=cfg.M)
        dt = time.time() - t0
        cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
        out["cpu_baseline"] = {"value": round(6.0 * cfg.D * cfg.I * Rs / dt / 1e12, 5),
                               "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                               "sample": f"float64 oracle forward on the first {Ts} tokens "
                                         f"({Rs} routed rows), {dt:.2f} s"}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
