"""Benchmark of the MoE layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5] [--M 2048] [--S 4]
                    [--comm-cus C] [--unfused] [--fwd-only] [--no-cpu-baseline] [--no-mx]
                    [--no-cold]
    python bench.py --sweep            # minibatch x comm-CU sweep of the forward, JSON lines
    python bench.py --copy-calibration # one plain device copy of known size (counter scale)
    python bench.py --autotune [--autotune-cache F]  # tune M and comm CUs first, then time
    python bench.py --trace [--config 4]  # in-kernel trace of the fused forward, decoded

A step is one pass of the layer over one batch of synthetic input on one GPU's share of
an expert-parallel layer (hidden 7168, expert intermediate 2048, 64 experts of which 8
are local, top-8, a 16384-token pool = 2048 tokens from each of 8 sources): schedule,
forward (persistent fused kernel) and backward, inputs resident in HBM before the timed
region.  Prints one JSON line.

`value` is the algorithmic TFLOP/s of the step: 6*D*I flops per routed row forward,
12*D*I backward (the GEMM1 replay of rows whose ring slot was recycled is not counted).
`kernels` gives each persistent kernel's rate against the bf16 dense MFMA peak (the
forward k_fwd_fused and the backward's k_bwd_main); their durations come from HIP events
recorded on the stream the kernels are launched on, around the forward and the backward
calls (each also holds a few-us helper launch).  `roofline` repeats the dominant one
(the one with the longer time, k_bwd_main on the default workload); its `traffic` is the
HBM byte count read from the committed FETCH_SIZE / WRITE_SIZE counter summary, scaled by
the copy calibration, and null when the kernel sources changed since the counters were
taken.  `phases_unfused` times the forward's four steps as separate launches with the
in-kernel phase clock: dispatch and combine against HBM bandwidth, GEMM1 and GEMM2
against the MFMA peak.  `mxfp8_fwd` does the same for the MXFP8 forward (config 4), and
`mxfp8_fwd_bwd` times forward + backward on that workload in MXFP8 and in bf16.
`mxfp8_permuted` times MXFP8 forward + backward on config 6 (the same skew with permuted
expert ranks: about 3.8k routed rows, the under-filled share).
`macrobatch` compares successive forwards run one after another with the same forwards
interleaved as macrobatches (MOK_FLAG_OVERLAP_NEXT, two workspaces and streams).
`ring_recycling` times the step again with 4 and 2 ring slots (fewer than the
minibatches): slots recycle inside the forward and the backward replays GEMM1.
`cpu_baseline` times the float64 NumPy oracle (forward + backward) on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 / MXFP8 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_bwd_main_c5_traffic.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "layer_c5_mfma_counters.txt")
CSRC = os.path.join(ROOT, "mixture_experts_layer_mok_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--M", type=int, default=None)
    ap.add_argument("--S", type=int, default=None)
    ap.add_argument("--comm-cus", type=int, default=None)
    ap.add_argument("--unfused", action="store_true")
    ap.add_argument("--fwd-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mx", action="store_true", help="skip the MXFP8 forward figure")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache steps")
    ap.add_argument("--no-ring", action="store_true",
                    help="skip the step timed with fewer ring slots than minibatches")
    ap.add_argument("--no-macrobatch", action="store_true",
                    help="skip the macrobatch interleave figure")
    ap.add_argument("--no-phases", action="store_true",
                    help="skip the per-phase rates of the forward as separate launches")
    ap.add_argument("--trace", action="store_true",
                    help="one traced fused forward: print where its time went (JSON)")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--autotune", action="store_true",
                    help="choose M and comm CUs for this shape on the device before timing")
    ap.add_argument("--autotune-cache", default=None, help="JSON cache of tuned choices")
    ap.add_argument("--copy-calibration", action="store_true")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of every kernel source: counter summaries taken on other sources are stale."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_traffic():
    """HBM bytes per launch of the backward's persistent kernel k_bwd_main from the
    committed counter summary, or None when it is absent or was taken on other kernel
    sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    m_hash = re.search(r"^source_hash:\s*(\w+)", text, re.M)
    m_bytes = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def read_mfma_counters():
    """Matrix-core busy fraction and shader clock of k_bwd_main from the committed counter
    summary (None when absent or taken on other kernel sources)."""
    try:
        with open(MFMA_FILE) as f:
            text = f.read()
    except OSError:
        return None
    m_hash = re.search(r"^source_hash:\s*(\w+)", text, re.M)
    m_busy = re.search(r"^k_bwd_main_mfma_busy:\s*([0-9.]+)", text, re.M)
    m_clk = re.search(r"^k_bwd_main_clock_ghz:\s*([0-9.]+)", text, re.M)
    if not (m_hash and m_busy and m_clk) or m_hash.group(1) != kernel_source_hash():
        return None
    return {"mfma_busy": float(m_busy.group(1)), "clock_ghz": float(m_clk.group(1))}


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, three times, for scaling the FETCH_SIZE and
    WRITE_SIZE counters: each launch moves exactly 1 GiB in and 1 GiB out."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def setup(cfg, unfused, save, device):
    import torch

    from mixture_experts_layer_mok_amd import _lib as L
    from mixture_experts_layer_mok_amd import gen
    from mixture_experts_layer_mok_amd.layer import MoKLayer, bf16_tensor

    log(f"generating {cfg.name} inputs")
    d = gen.make_inputs(cfg, with_dy=save)
    t = dict(x=bf16_tensor(d["x_bits"], device), ids=torch.from_numpy(d["ids"]).to(device),
             gates=torch.from_numpy(d["gates"]).to(device))
    for n in ("wg", "wu", "wd") + (("dy",) if save else ()):
        t[n] = bf16_tensor(d[n + "_bits"], device)
    flags = (L.MOK_FLAG_UNFUSED if unfused else 0) | (L.MOK_FLAG_SAVE_FOR_BWD if save else 0)
    layer = MoKLayer(L.desc_from_config(cfg, flags=flags), device=device)
    if cfg.precision == L.MOK_PREC_MXFP8:
        # weights are quantised once, before the layer (not part of a step): along each
        # forward GEMM's K, and for the backward transposed, along its GEMMs' K
        if save:
            t["wt"] = layer.quantize_weights_bwd(t["wg"], t["wu"], t["wd"])
        for n in ("wg", "wu", "wd"):
            t[n], t["s" + n[1]] = layer.quantize_weights(t[n])
        torch.cuda.synchronize()
    return d, t, layer


def time_layer(cfg, t, layer, steps, warmup, with_bwd):
    """Times `steps` steps after `warmup`; returns per-phase mean ms and total ms/step."""
    import torch
    stream = torch.cuda.current_stream()
    y = torch.empty((cfg.T, cfg.D), dtype=torch.bfloat16, device=t["x"].device)
    grads = {}

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        layer.schedule(t["ids"])
        if ev is not None:
            ev[1].record(stream)
        layer.forward(t["x"], t["ids"], t["gates"], t["wg"], t["wu"], t["wd"],
                      scales=(t.get("sg"), t.get("su"), t.get("sd")), y=y)
        if ev is not None:
            ev[2].record(stream)
        if with_bwd:
            if "wt" in t:
                grads.update(layer.backward_mx(t["dy"], t["x"], t["ids"], t["gates"], t["wt"]))
            else:
                grads.update(layer.backward(t["dy"], t["x"], t["ids"], t["gates"], t["wg"],
                                            t["wu"], t["wd"]))
            if ev is not None:
                ev[3].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    st = layer.status()
    if st != 0:
        raise SystemExit(f"device status {st:#x} after warmup")
    nev = 4 if with_bwd else 3
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    st = layer.status()
    if st != 0:
        raise SystemExit(f"device status {st:#x} after timed steps")
    res = {"ms_per_step": start.elapsed_time(end) / steps,
           "sched_ms": [e[0].elapsed_time(e[1]) for e in evs],
           "fwd_ms": [e[1].elapsed_time(e[2]) for e in evs]}
    if with_bwd:
        res["bwd_ms"] = [e[2].elapsed_time(e[3]) for e in evs]
    return res


def time_cold(cfg, t, layer, steps, with_bwd):
    """Per-phase times with the caches cold: before each step a 1 GiB buffer is written
    (outside the timed phases), which evicts the weights and rows from the 256 MB
    Infinity Cache and the L2s."""
    import torch
    stream = torch.cuda.current_stream()
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=t["x"].device)
    y = torch.empty((cfg.T, cfg.D), dtype=torch.bfloat16, device=t["x"].device)
    fwd, bwd = [], []
    # one untimed step first: with the scrub buffer taken, the gradient outputs may need
    # fresh device allocations, which must not fall inside a timed phase
    for i in range(-1, steps):
        scrub.fill_(i & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        layer.schedule(t["ids"])
        ev[0].record(stream)
        layer.forward(t["x"], t["ids"], t["gates"], t["wg"], t["wu"], t["wd"],
                      scales=(t.get("sg"), t.get("su"), t.get("sd")), y=y)
        ev[1].record(stream)
        if with_bwd:
            scrub.fill_((i + 128) & 0xFF)
            ev[2].record(stream)
            if "wt" in t:
                layer.backward_mx(t["dy"], t["x"], t["ids"], t["gates"], t["wt"])
            else:
                layer.backward(t["dy"], t["x"], t["ids"], t["gates"], t["wg"], t["wu"], t["wd"])
            ev.append(torch.cuda.Event(enable_timing=True))
            ev[3].record(stream)
        torch.cuda.synchronize()
        if i < 0:
            continue
        fwd.append(ev[0].elapsed_time(ev[1]))
        if with_bwd:
            bwd.append(ev[2].elapsed_time(ev[3]))
    if layer.status() != 0:
        raise SystemExit(f"device status {layer.status():#x} after the cold-cache steps")
    del scrub
    torch.cuda.empty_cache()
    out = {"fwd_ms": stats(fwd)}
    if with_bwd:
        out["bwd_ms"] = stats(bwd)
    return out


def stats(v):
    return {"mean": round(float(np.mean(v)), 4), "median": round(float(np.median(v)), 4),
            "min": round(float(np.min(v)), 4)}


def routed_rows(cfg, ids):
    return int(((ids >= cfg.e0) & (ids < cfg.e0 + cfg.n_local)).sum())


def sweep(args):
    """Forward time over minibatch sizes and comm-CU counts on the config-3 (bf16) or
    config-4 (MXFP8, Zipf routing) workload, against
    the two-waves lower bound for a 256 x 256 tile: each GEMM should see at least two full
    waves of tiles, 2 * C_compute * 256 * 256 / (2 I) rows for GEMM1."""
    import torch

    from mixture_experts_layer_mok_amd import _lib as L
    from mixture_experts_layer_mok_amd import gen
    L.load()
    dev = torch.device("cuda:0")
    base = gen.CONFIGS[args.config if args.config in (3, 4) else 3]
    d, t, _ = setup(base, False, False, dev)
    R = routed_rows(base, d["ids"])
    from mixture_experts_layer_mok_amd.layer import MoKLayer
    from mixture_experts_layer_mok_amd.tuning import layer_two_wave_min_rows
    cus = L.mok_device_cus()
    mx = base.precision == L.MOK_PREC_MXFP8
    comms = (24, 32, 40, 48, 64) if mx else (12, 16, 20, 24, 32, 48)
    Ms = (1024, 2048, 4096) if mx else (512, 1024, 1536, 2048, 2560, 3072, 3584, 4096,
                                              6144, 8192)
    for comm in comms:
        for M in Ms:
            cfg = base.replace(M=M, comm_cus=comm)
            layer = MoKLayer(L.desc_from_config(cfg), device=dev)
            r = time_layer(cfg, t, layer, args.steps, args.warmup, False)
            fwd = float(np.median(r["fwd_ms"]))
            m_min = layer_two_wave_min_rows(cus, comm, cfg.I)
            print(json.dumps({"sweep": "minibatch", "config": base.name, "M": M, "comm_cus": comm,
                              "fwd_ms_median": round(fwd, 4),
                              "fwd_tflops": round(6.0 * cfg.D * cfg.I * R / fwd / 1e9, 1),
                              "two_wave_min_rows": round(m_min), "above_two_waves": M >= m_min}),
                  flush=True)
            del layer
            torch.cuda.empty_cache()


def phase_rates(cfg, t, R, runs):
    """The same forward as separate launches (MOK_FLAG_UNFUSED) with the in-kernel phase
    clock (MOK_FLAG_TRACE): per launch, the median span from its first workgroup start to
    its last workgroup end over `runs` calls, and the rate that gives against the
    algorithmic work: dispatch D (2 + s_out) + 8 bytes per routed row (s_out = 2 for bf16,
    1 + 1/32 for MX codes and scales), combine 2 D per routed row + 2 D + 8 k per token,
    GEMM1 4 D I and GEMM2 2 D I flops per routed row."""
    import torch

    from mixture_experts_layer_mok_amd import _lib as L
    from mixture_experts_layer_mok_amd import trace as TR
    from mixture_experts_layer_mok_amd.layer import MoKLayer
    mx = cfg.precision == L.MOK_PREC_MXFP8
    layer = MoKLayer(L.desc_from_config(cfg, flags=L.MOK_FLAG_UNFUSED | L.MOK_FLAG_TRACE),
                     device=t["x"].device)
    y = torch.empty((cfg.T, cfg.D), dtype=torch.bfloat16, device=t["x"].device)
    sc = (t.get("sg"), t.get("su"), t.get("sd"))
    per = {n: [] for n in TR.PHASES}
    for i in range(runs + 2):
        layer.schedule(t["ids"])
        layer.forward(t["x"], t["ids"], t["gates"], t["wg"], t["wu"], t["wd"], scales=sc, y=y)
        ph = TR.read_phases(layer)
        if i >= 2:
            for n in TR.PHASES:
                per[n].append(ph[n])
    if layer.status() != 0:
        raise SystemExit(f"device status {layer.status():#x} after the unfused forwards")
    s_out = (1 + 1 / 32) if mx else 2
    peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    work = {"gather": ("hbm", R * (cfg.D * (2 + s_out) + 8)),
            "gemm1": ("mfma", 4.0 * cfg.D * cfg.I * R),
            "gemm2": ("mfma", 2.0 * cfg.D * cfg.I * R),
            "combine": ("hbm", R * 2 * cfg.D + cfg.T * (2 * cfg.D + 8 * cfg.k))}
    out = {}
    for n in TR.PHASES:
        us = float(np.median(per[n]))
        bound, w = work[n]
        if bound == "hbm":
            gbs = w / (us * 1e-6) / 1e9
            out[n] = {"us": round(us, 1), "bound": "hbm", "bytes": int(w),
                      "achieved_GBps": round(gbs, 1), "peak_GBps": PEAK_HBM_GBS,
                      "frac": round(gbs / PEAK_HBM_GBS, 4)}
        else:
            tf = w / (us * 1e-6) / 1e12
            out[n] = {"us": round(us, 1), "bound": "mfma", "flops": w,
                      "achieved_TFLOPs": round(tf, 1), "peak_TFLOPs": peak,
                      "frac": round(tf / peak, 4)}
    del layer
    torch.cuda.empty_cache()
    return out


def mx_forward_figure(args):
    """The MXFP8 forward on the Zipf-skewed config-4 workload (the pages' MXFP8 mode),
    timed like the main line; reported beside the bf16 step."""
    import torch

    from mixture_experts_layer_mok_amd import gen
    cfg = gen.CONFIGS[4]
    dev = torch.device("cuda:0")
    d, t, layer = setup(cfg, False, False, dev)
    R = routed_rows(cfg, d["ids"])
    log(f"timing the MXFP8 forward ({R} routed rows)")
    r = time_layer(cfg, t, layer, args.steps, args.warmup, False)
    fwd = float(np.mean(r["fwd_ms"]))
    tf = 6.0 * cfg.D * cfg.I * R / (fwd * 1e-3) / 1e12
    res = {"workload": f"{cfg.name}: Zipf(1.2) routing, {R} routed rows",
           "kernel": "k_fwd_fused<MX>",
           "schedule_ms": stats(r["sched_ms"]), "fwd_ms": stats(r["fwd_ms"]),
           "fwd_tflops": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "frac": round(tf / PEAK_FP8_TFLOPS, 4),
           "routed_rows_per_s": round(R / (r["ms_per_step"] * 1e-3), 1)}
    del layer
    torch.cuda.empty_cache()
    log("timing the MXFP8 forward's phases as separate launches")
    res["phases_unfused"] = phase_rates(cfg, t, R, 3)
    del t
    torch.cuda.empty_cache()
    return res


def mx_backward_figure(args):
    """Forward + backward in MXFP8 on the Zipf-skewed config-4 workload, beside the same
    workload in bf16: the backward's time in each precision (the pages compare MXFP8 and
    BF16 backward speedups).  The backward's rate counts 12 D I flops per routed row, of
    which the dH and dX GEMMs (6 D I) run on scaled e4m3 MFMA and the dW GEMMs in bf16."""
    import torch

    from mixture_experts_layer_mok_amd import _lib as L
    from mixture_experts_layer_mok_amd import gen
    dev = torch.device("cuda:0")
    out = {}
    for prec in (L.MOK_PREC_MXFP8, L.MOK_PREC_BF16):
        cfg = gen.CONFIGS[4].replace(precision=prec)
        d, t, layer = setup(cfg, False, True, dev)
        R = routed_rows(cfg, d["ids"])
        name = "mxfp8" if prec == L.MOK_PREC_MXFP8 else "bf16"
        log(f"timing the {name} forward + backward on {cfg.name} ({R} routed rows)")
        r = time_layer(cfg, t, layer, args.steps, args.warmup, True)
        bwd = float(np.mean(r["bwd_ms"]))
        out[name] = {"fwd_ms": stats(r["fwd_ms"]), "bwd_ms": stats(r["bwd_ms"]),
                     "bwd_tflops": round(12.0 * cfg.D * cfg.I * R / (bwd * 1e-3) / 1e12, 2)}
        del layer, t, d
        torch.cuda.empty_cache()
    out["workload"] = "c4 shape, Zipf(1.2) routing, forward saving for the backward"
    out["bwd_speedup_mxfp8_vs_bf16"] = round(out["bf16"]["bwd_ms"]["mean"] /
                                             out["mxfp8"]["bwd_ms"]["mean"], 3)
    return out


def mx_permuted_figure(args):
    """Forward + backward in MXFP8 on config 6: config 4's Zipf skew with the popularity
    ranks permuted, so this GPU's experts hold about 3.8k routed rows (two minibatches,
    experts of 35 to 2k rows): the under-filled share, beside config 4's overloaded one."""
    import torch

    from mixture_experts_layer_mok_amd import gen
    cfg = gen.CONFIGS[6]
    d, t, layer = setup(cfg, False, True, torch.device("cuda:0"))
    R = routed_rows(cfg, d["ids"])
    log(f"timing the MXFP8 forward + backward on {cfg.name} ({R} routed rows)")
    r = time_layer(cfg, t, layer, args.steps, args.warmup, True)
    fwd, bwd = float(np.mean(r["fwd_ms"])), float(np.mean(r["bwd_ms"]))
    out = {"workload": f"{cfg.name}: Zipf(1.2) routing with permuted ranks, {R} routed rows",
           "fwd_ms": stats(r["fwd_ms"]), "bwd_ms": stats(r["bwd_ms"]),
           "fwd_tflops": round(6.0 * cfg.D * cfg.I * R / (fwd * 1e-3) / 1e12, 2),
           "bwd_tflops": round(12.0 * cfg.D * cfg.I * R / (bwd * 1e-3) / 1e12, 2)}
    del layer, t, d
    torch.cuda.empty_cache()
    return out


def macrobatch_figure(args, n=4):
    """Macrobatch interleave on the config-3 workload (four ring slots, eight minibatches,
    so slots recycle): n forwards one after another on one stream and workspace, against
    the same n as interleaved macrobatches (two workspaces and two streams with
    MOK_FLAG_OVERLAP_NEXT, each combine overlapping the next dispatch).  Times are HIP
    events around each whole sequence; `overlap_us` comes from a traced pair of calls: how
    long the second call's workgroups ran before the first call's last workgroup ended."""
    import torch

    from mixture_experts_layer_mok_amd import _lib as L
    from mixture_experts_layer_mok_amd import gen
    from mixture_experts_layer_mok_amd.layer import MoKLayer, forward_macrobatches
    cfg = gen.CONFIGS[3]
    dev = torch.device("cuda:0")
    d, t, _ = setup(cfg, False, False, dev)
    batch = (t["x"], t["ids"], t["gates"], t["wg"], t["wu"], t["wd"])
    ys = [torch.empty((cfg.T, cfg.D), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    seq = MoKLayer(L.desc_from_config(cfg), device=dev)
    ilv = [MoKLayer(L.desc_from_config(cfg, flags=L.MOK_FLAG_OVERLAP_NEXT), device=dev)
           for _ in range(2)]

    def run_seq():
        for i in range(n):
            seq.schedule(t["ids"], stream=s0)
            seq.forward(*batch, y=ys[i], stream=s0)

    def run_ilv():
        forward_macrobatches(ilv, (s0, s1), [batch] * n, ys)

    def timed(fn, reps):
        out = []
        for r in range(reps + 2):
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            torch.cuda.synchronize()
            e0.record(s0)
            s1.wait_event(e0)
            fn()
            e1.record(s1)
            s0.wait_event(e1)
            e2.record(s0)
            torch.cuda.synchronize()
            if r >= 2:
                out.append(e0.elapsed_time(e2) / n)
        return out

    log(f"timing {n} macrobatches, sequential and interleaved")
    seq_ms = timed(run_seq, max(3, args.steps // 2))
    ilv_ms = timed(run_ilv, max(3, args.steps // 2))
    for lay in [seq] + ilv:
        if lay.status() != 0:
            raise SystemExit(f"device status {lay.status():#x} in the macrobatch runs")
    # one traced pair: when did the second call start against the first call's end
    tr = [MoKLayer(L.desc_from_config(cfg, flags=L.MOK_FLAG_OVERLAP_NEXT | L.MOK_FLAG_TRACE),
                   device=dev) for _ in range(2)]
    for _ in range(2):
        forward_macrobatches(tr, (s0, s1), [batch] * 2, ys[:2])
    torch.cuda.synchronize()
    cus = L.mok_device_cus()
    recs = []
    for lay in tr:
        off, words = L.mok_trace_layout(lay.desc)
        raw = lay.ws[off:off + words * 4].cpu().numpy().view(np.uint32)
        cap = (words - L.MOK_TRACE_MAX_WORKGROUPS * 8) // 8
        recs.append(raw[cap * 8:cap * 8 + cus * 8].reshape(cus, 8).astype(np.int64))
    base = int(recs[0][:, 0].min())
    rel = lambda v: (v - base) & 0xFFFFFFFF  # noqa: E731  (10 ns ticks)
    end0 = int(rel(recs[0][:, 3]).max())
    start1 = int(rel(recs[1][:, 0]).min())
    del seq, ilv, tr, t, d
    torch.cuda.empty_cache()
    return {"workload": f"{cfg.name}: {n} macrobatches of the same shape (M={cfg.M}, "
                        f"S={cfg.S}, comm_cus={cfg.comm_cus})",
            "sequential_ms_per_macrobatch": stats(seq_ms),
            "interleaved_ms_per_macrobatch": stats(ilv_ms),
            "speedup": round(float(np.median(seq_ms)) / float(np.median(ilv_ms)), 4),
            "overlap_us": round(max(0, end0 - start1) * 0.01, 1),
            "first_call_us": round(end0 * 0.01, 1)}


def ring_figure(args):
    """The config-5 step (forward + backward) with fewer ring slots than minibatches, so
    that the timed step recycles slots inside the forward and replays GEMM1 for the
    recycled minibatches in the backward (the headline keeps every minibatch resident).
    The replay's flops are not counted in the rate."""
    import torch

    from mixture_experts_layer_mok_amd import _lib as L
    from mixture_experts_layer_mok_amd import gen
    from mixture_experts_layer_mok_amd.layer import MoKLayer
    base = gen.CONFIGS[5]
    dev = torch.device("cuda:0")
    d, t, _ = setup(base, False, True, dev)
    R = routed_rows(base, d["ids"])
    n_mb = -(-R // base.M)
    out = {"workload": f"{base.name}, M={base.M}: {n_mb} minibatches", "slots": {}}
    for S in (base.S, 4, 2):
        cfg = base.replace(S=S)
        layer = MoKLayer(L.desc_from_config(cfg, flags=L.MOK_FLAG_SAVE_FOR_BWD), device=dev)
        log(f"timing the step with {S} ring slots")
        r = time_layer(cfg, t, layer, max(3, args.steps // 2), args.warmup, True)
        ms = r["ms_per_step"]
        out["slots"][str(S)] = {
            "replayed_minibatches": max(0, n_mb - S), "ms_per_step": round(ms, 4),
            "fwd_ms": stats(r["fwd_ms"]), "bwd_ms": stats(r["bwd_ms"]),
            "tflops": round(18.0 * cfg.D * cfg.I * R / (ms * 1e-3) / 1e12, 2),
            "workspace_GB": round(L.mok_workspace_size(layer.desc) / 1e9, 3)}
        del layer
        torch.cuda.empty_cache()
    del t, d
    torch.cuda.empty_cache()
    return out


def trace_forward(args):
    """Warm-up forwards, then one forward with MOK_FLAG_TRACE on the same workload, decoded
    into where the compute and data-mover workgroups spent the kernel's span."""
    import torch

    from mixture_experts_layer_mok_amd import _lib as L
    from mixture_experts_layer_mok_amd import gen
    from mixture_experts_layer_mok_amd import trace as TR
    from mixture_experts_layer_mok_amd.layer import MoKLayer
    cfg = gen.CONFIGS[args.config]
    over = {k: v for k, v in (("M", args.M), ("S", args.S), ("comm_cus", args.comm_cus)) if v}
    cfg = cfg.replace(**over)
    dev = torch.device("cuda:0")
    save = args.config == 5 or cfg.precision == L.MOK_PREC_MXFP8
    d, t, layer = setup(cfg, False, save, dev)
    flags = L.MOK_FLAG_TRACE | (L.MOK_FLAG_SAVE_FOR_BWD if save else 0)
    tl = MoKLayer(L.desc_from_config(cfg, flags=flags), device=dev)
    y = torch.empty((cfg.T, cfg.D), dtype=torch.bfloat16, device=dev)
    sc = (t.get("sg"), t.get("su"), t.get("sd"))
    for _ in range(args.warmup + 1):
        tl.schedule(t["ids"])
        tl.forward(t["x"], t["ids"], t["gates"], t["wg"], t["wu"], t["wd"], scales=sc, y=y)
    torch.cuda.synchronize()
    if tl.status() != 0:
        raise SystemExit(f"device status {tl.status():#x}")
    tab = tl.tables()
    d_ = tl.desc
    nN1 = (d_.intermediate + 127) // 128
    nN2 = (d_.hidden + 255) // 256
    tiles = tab["n_mtiles"] * (nN1 + nN2)
    recs, wgs = TR.read(tl, tiles, L.mok_device_cus())
    out = {"trace": TR.summarize(recs, wgs, cfg.comm_cus),
           "config": {"workload": cfg.name, "routed_rows": tab["R"], "minibatch_rows": cfg.M,
                      "ring_slots": cfg.S, "comm_cus": cfg.comm_cus, "tiles": int(tiles)}}
    if save:
        # the backward's persistent launch, traced on the same workspace (its records
        # replace the forward's)
        if "wt" in t:
            tl.backward_mx(t["dy"], t["x"], t["ids"], t["gates"], t["wt"])
        else:
            tl.backward(t["dy"], t["x"], t["ids"], t["gates"], t["wg"], t["wu"], t["wd"])
        torch.cuda.synchronize()
        if tl.status() != 0:
            raise SystemExit(f"device status {tl.status():#x} after the backward")
        n = TR.bwd_tickets(d_, tab["n_mtiles"])
        brecs, bwgs = TR.read(tl, n, L.mok_device_cus())
        out["trace_backward"] = TR.summarize_bwd(brecs, bwgs)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this layer runs on one GPU only; --gpus must be 1. "
                          "Across GPUs it shards by expert, one process per GPU."}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    from mixture_experts_layer_mok_amd import _lib as L
    from mixture_experts_layer_mok_amd import gen

    L.load()
    if args.sweep:
        sweep(args)
        return
    if args.trace:
        trace_forward(args)
        return
    cfg = gen.CONFIGS[args.config]
    over = {k: v for k, v in (("M", args.M), ("S", args.S), ("comm_cus", args.comm_cus)) if v}
    cfg = cfg.replace(**over)
    mx = cfg.precision == L.MOK_PREC_MXFP8
    with_bwd = not args.fwd_only
    dev = torch.device("cuda:0")
    d, t, layer = setup(cfg, args.unfused, with_bwd, dev)
    R = routed_rows(cfg, d["ids"])
    tuned = None
    if args.autotune:
        from mixture_experts_layer_mok_amd import autotune as A
        from mixture_experts_layer_mok_amd.layer import MoKLayer
        log("tuning the minibatch size and the comm-CU split for this shape")
        ch = A.tune(L.desc_from_config(cfg), t["x"], t["ids"], t["gates"], t["wg"], t["wu"],
                    t["wd"], scales=(t.get("sg"), t.get("su"), t.get("sd")),
                    cache_path=args.autotune_cache)
        tuned = {"minibatch_rows": ch.minibatch_rows, "comm_cus": ch.comm_cus,
                 "fwd_ms": ch.fwd_ms, "trials": len(ch.trials)}
        cfg = cfg.replace(M=ch.minibatch_rows, comm_cus=ch.comm_cus)
        flags = (L.MOK_FLAG_UNFUSED if args.unfused else 0) | (L.MOK_FLAG_SAVE_FOR_BWD if with_bwd else 0)
        del layer
        torch.cuda.empty_cache()
        layer = MoKLayer(L.desc_from_config(cfg, flags=flags), device=dev)
    flops_fwd = 6.0 * cfg.D * cfg.I * R
    flops_bwd = 12.0 * cfg.D * cfg.I * R if with_bwd else 0.0
    log(f"timing {args.steps} steps after {args.warmup} warmup")
    r = time_layer(cfg, t, layer, args.steps, args.warmup, with_bwd)
    ms = r["ms_per_step"]
    fwd_ms = float(np.mean(r["fwd_ms"]))
    achieved = flops_fwd / (fwd_ms * 1e-3) / 1e12
    mode = "unfused" if args.unfused else "fused"
    prec = "mxfp8" if mx else "bf16"
    peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    out = {
        "metric": f"MoE layer fwd+bwd TFLOPS ({prec})" if with_bwd else
                  f"MoE layer forward TFLOPS ({prec})",
        "value": round((flops_fwd + flops_bwd) / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3+e8m0 (fp32 accumulate)" if mx else "bf16",
        "data": "synthetic (seeded normal draws at the layer's real shape)",
        "config": {"workload": f"{cfg.name}: pool T={cfg.T} x D={cfg.D}, I={cfg.I}, "
                               f"E={cfg.E} (experts {cfg.e0}..{cfg.e0 + cfg.n_local - 1} local), "
                               f"top-{cfg.k}" + (", forward+backward" if with_bwd else
                                                 ", forward"),
                   "routed_rows": R, "minibatch_rows": cfg.M, "ring_slots": cfg.S,
                   "comm_cus": cfg.comm_cus, "mode": mode, **({"autotuned": tuned} if tuned else {})},
        "schedule_ms": stats(r["sched_ms"]),
        "fwd_ms": stats(r["fwd_ms"]),
        "fwd_tflops": round(achieved, 2),
        "routed_rows_per_s": round(R / (ms * 1e-3), 1),
        "schedule_share": round(float(np.mean(r["sched_ms"])) / ms, 4),
    }
    if with_bwd:
        bwd_ms = float(np.mean(r["bwd_ms"]))
        out["bwd_ms"] = stats(r["bwd_ms"])
        out["bwd_tflops"] = round(flops_bwd / (bwd_ms * 1e-3) / 1e12, 2)
    # per-kernel view: the persistent forward and the backward's persistent kernel, each
    # against the bf16 dense MFMA peak.  Both durations come from HIP events on the stream
    # the kernels run on, around the forward call (a counter-reset kernel of a few us, then
    # k_fwd_fused) and around the backward call (the row-offset kernel and the empty replay
    # launch, a few us, then k_bwd_main).
    kernels = {"k_fwd_fused" if not args.unfused else "forward (unfused launches)": {
        "ms": round(fwd_ms, 4), "flops": flops_fwd, "achieved_TFLOPs": round(achieved, 2),
        "peak_TFLOPs": peak, "frac": round(achieved / peak, 4)}}
    dominant = next(iter(kernels))
    dom = kernels[dominant]
    if with_bwd:
        bwd_tf = flops_bwd / (bwd_ms * 1e-3) / 1e12
        kernels["k_bwd_main"] = {"ms": round(bwd_ms, 4), "flops": flops_bwd,
                                 "achieved_TFLOPs": round(bwd_tf, 2), "peak_TFLOPs": peak,
                                 "frac": round(bwd_tf / peak, 4)}
        if bwd_ms > fwd_ms:
            dominant, dom = "k_bwd_main", kernels["k_bwd_main"]
    out["kernels"] = kernels
    # the committed counters were taken on the default command (config 5 as defined, fused,
    # forward saving a and b for the backward)
    c5 = gen.CONFIGS[5]
    default_cmd = (not args.unfused and with_bwd and args.config == 5
                   and (cfg.M, cfg.S, cfg.comm_cus) == (c5.M, c5.S, c5.comm_cus))
    traffic = read_traffic() if default_cmd and dominant == "k_bwd_main" else None
    out["roofline"] = {"bound": "mfma", "kernel": dominant, "achieved": dom["achieved_TFLOPs"],
                       "peak": peak, "unit": "TFLOP/s", "frac": dom["frac"], "traffic": traffic}
    mfma = read_mfma_counters() if default_cmd and dominant == "k_bwd_main" else None
    if mfma:
        # the counters' view: matrix cores busy per shader cycle, and the clock the card ran
        # at; peak_at_clock is the dense peak scaled to that clock
        out["roofline"].update(mfma_busy=mfma["mfma_busy"], clock_ghz=mfma["clock_ghz"],
                               peak_at_clock=round(peak * mfma["clock_ghz"] / 2.4, 1))
    if not args.no_phases:
        log("timing the forward's phases as separate launches (dispatch and combine rates)")
        out["phases_unfused"] = phase_rates(cfg, t, R, 3)
    if not args.no_cold:
        log("timing cold-cache steps (1 GiB scrub before each)")
        out["cold_cache"] = time_cold(cfg, t, layer, min(args.steps, 5), with_bwd)
    if not mx and not args.no_mx and args.config == 5:
        out["mxfp8_fwd"] = mx_forward_figure(args)
        out["mxfp8_fwd_bwd"] = mx_backward_figure(args)
        out["mxfp8_permuted"] = mx_permuted_figure(args)
    if not args.no_macrobatch and args.config == 5:
        out["macrobatch"] = macrobatch_figure(args)
    if not args.no_ring and args.config == 5:
        out["ring_recycling"] = ring_figure(args)
    if not args.no_cpu_baseline:
        import oracle as O
        log("timing the float64 oracle on the host")
        t0 = time.time()
        O.forward(d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"], e0=cfg.e0, E=cfg.E,
                  M=cfg.M)
        if with_bwd:
            O.backward(d["dy"], d["x"], d["ids"], d["gates"], d["wg"], d["wu"], d["wd"],
                       e0=cfg.e0, E=cfg.E, M=cfg.M)
        dt = time.time() - t0
        cores = len(os.sched_getaffinity(0))
        omp = os.environ.get("OMP_NUM_THREADS")
        if omp and omp.isdigit():
            cores = min(cores, int(omp))
        out["cpu_baseline"] = {
            "value": round((flops_fwd + flops_bwd) / dt / 1e12, 5), "unit": "TFLOP/s",
            "cores": cores, "cpu": cpu_model(), "kind": "oracle",
            "sample": f"the whole workload ({R} routed rows), "
                      f"{'forward+backward' if with_bwd else 'forward'} once in float64 "
                      f"NumPy: {dt:.1f} s"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
