"""Decoding of the fused forward's in-kernel trace (MOK_FLAG_TRACE).

The kernel writes, per tile ticket, the workgroup, the GEMM and minibatch, and four
timestamps (ticket taken, inputs ready, K loop done, signal done) plus the time its
epilogue's stores were all issued, and per
workgroup the start, the end of the minibatch-0 fill, the end of its role and of its
drain (record layout in include/mok.h, mok_trace_layout).  Timestamps are the low 32 bits
of the 100 MHz constant clock.  `summarize` turns one run's records into where the time of
the compute and data-mover workgroups went, as shares of the kernel's span.
"""
from __future__ import annotations

import numpy as np

TICK_US = 0.01  # 100 MHz


def read(layer, tiles: int, cus: int) -> tuple[np.ndarray, np.ndarray]:
    """Ticket records [tiles, 8] and workgroup records [cus, 8] (uint32) of the last traced
    launch on `layer` (a MoKLayer built with MOK_FLAG_TRACE); synchronises."""
    import torch

    from . import _lib as L
    off, words = L.mok_trace_layout(layer.desc)
    torch.cuda.synchronize(layer.device)
    raw = layer.ws[off:off + words * 4].cpu().numpy().view(np.uint32)
    tile_cap = (words - L.MOK_TRACE_MAX_WORKGROUPS * 8) // 8
    if tiles > tile_cap or cus > L.MOK_TRACE_MAX_WORKGROUPS:
        raise ValueError(f"{tiles} tickets / {cus} workgroups exceed the trace region")
    return raw[:tiles * 8].reshape(tiles, 8).copy(), \
        raw[tile_cap * 8:tile_cap * 8 + cus * 8].reshape(cus, 8).copy()


def summarize(tiles: np.ndarray, wgs: np.ndarray, comm_cus: int) -> dict:
    t0 = int(wgs[:, 0].min())

    def rel(x):
        return (x.astype(np.int64) - t0) & 0xFFFFFFFF  # ticks since the kernel start

    start, fill, role, drain = (rel(wgs[:, i]) for i in range(4))
    span = float(drain.max())
    comp = np.arange(len(wgs)) >= comm_cus
    wg = tiles[:, 0].astype(np.int64)
    g2 = (tiles[:, 1] & 1).astype(bool)
    t_tk, t_rd, t_k, t_end = (rel(tiles[:, i]) for i in range(2, 6))
    t_e = rel(tiles[:, 6])
    wait, kloop, epi = t_rd - t_tk, t_k - t_rd, t_end - t_k
    epi_issue, signal = t_e - t_k, t_end - t_e
    n_comp = int(comp.sum())
    tot = span * n_comp
    # per compute workgroup: time between its fill and its role end not inside a tile
    inside = np.zeros(len(wgs))
    np.add.at(inside, wg, (t_end - t_tk).astype(float))
    fill_c = float((fill[comp] - start[comp]).sum())
    role_c = float((role[comp] - fill[comp]).sum())
    between = role_c - float(inside[comp].sum())
    after = float((span - role[comp]).sum())  # drain and the idle end
    us = lambda v: round(float(v) * TICK_US, 2)  # noqa: E731
    out = {
        "span_us": us(span),
        "compute_cus": n_comp,
        "compute_share": {
            "k_loop": round(float(kloop.sum()) / tot, 4),
            "epilogue_and_signal": round(float(epi.sum()) / tot, 4),
            "wait_for_inputs": round(float(wait.sum()) / tot, 4),
            "between_tiles": round(between / tot, 4),
            "fill": round(fill_c / tot, 4),
            "after_role": round(after / tot, 4),
        },
        "tile_us": {
            name: {"n": int(m.sum()), "k_loop": us(kloop[m].mean()), "epilogue": us(epi[m].mean()),
                   "epilogue_issue": us(epi_issue[m].mean()),
                   "store_drain_and_signal": us(signal[m].mean()), "wait": us(wait[m].mean())}
            for name, m in (("gemm1", ~g2), ("gemm2", g2)) if m.any()},
        "first_tile_us": us(t_tk.min()),
        "last_tile_end_us": us(t_end.max()),
    }
    if comm_cus > 0:
        cm = ~comp
        out["comm"] = {"fill_us": us((fill[cm] - start[cm]).mean()),
                       "role_us": us((role[cm] - fill[cm]).mean()),
                       "drain_us": us((drain[cm] - role[cm]).mean()),
                       "drain_chunks": int(wgs[cm, 5].sum())}
    out["drain_chunks_compute"] = int(wgs[comp, 5].sum())
    return out


BWD_KINDS = ("dh", "dx", "dw", "row_sums", "mx_quant")


def bwd_tickets(desc, m_tiles: int) -> int:
    """Tickets of the backward's persistent launch: dH, dX, dW tiles and row-sum chunks,
    and in MXFP8 one quantisation ticket per m-tile."""
    from . import _lib as L
    nDt = (desc.hidden + 255) // 256
    nIt = (desc.intermediate + 255) // 256
    mx = 1 if desc.precision == L.MOK_PREC_MXFP8 else 0
    return m_tiles * (nIt + nDt + mx) + desc.num_local_experts * 3 * nDt * nIt + \
        (desc.num_tokens + 31) // 32


def summarize_bwd(recs: np.ndarray, wgs: np.ndarray) -> dict:
    """Backward launch: per ticket kind, the mean wait for inputs, K loop and epilogue
    (for the row sums: the sum itself) in microseconds, and each kind's share of the
    workgroups' time over the launch's span."""
    t0 = int(wgs[:, 0].min())

    def rel(x):
        return (x.astype(np.int64) - t0) & 0xFFFFFFFF

    span = float(rel(wgs[:, 2]).max())
    tot = span * len(wgs)
    kind = recs[:, 1]
    t_tk, t_rd, t_k, t_end = (rel(recs[:, i]) for i in range(2, 6))
    out = {"span_us": round(span * TICK_US, 2), "workgroups": int(len(wgs)), "kinds": {}}
    busy = 0.0
    for k, name in enumerate(BWD_KINDS):
        m = kind == k
        if not m.any():
            continue
        wait, body, epi = (t_rd - t_tk)[m], (t_k - t_rd)[m], (t_end - t_k)[m]
        busy += float((t_end - t_tk)[m].sum())
        out["kinds"][name] = {
            "n": int(m.sum()), "wait_us": round(float(wait.mean()) * TICK_US, 2),
            ("k_loop_us" if k < 3 else "sum_us" if k == 3 else "work_us"):
                round(float(body.mean()) * TICK_US, 2),
            "epilogue_us": round(float(epi.mean()) * TICK_US, 2),
            "share": round(float((t_end - t_tk)[m].sum()) / tot, 4)}
    out["outside_tickets_share"] = round(1.0 - busy / tot, 4)
    return out


PHASES = ("gather", "gemm1", "gemm2", "combine")


def read_phases(layer) -> dict:
    """Durations (us) of the gather, GEMM1, GEMM2 and combine launches of the last
    unfused forward run with MOK_FLAG_TRACE on `layer`: per launch, the latest workgroup
    end minus the earliest workgroup start; synchronises."""
    import torch

    from . import _lib as L
    off, words = L.mok_trace_layout(layer.desc)
    torch.cuda.synchronize(layer.device)
    raw = layer.ws[off:off + words * 4].cpu().numpy()
    grids = raw[:16].view(np.uint32)[:4].astype(np.int64)
    rec = raw[32:].view(np.uint64).astype(np.int64)
    out, w = {}, 0
    for name, g in zip(PHASES, grids):
        r = rec[w:w + 2 * g].reshape(g, 2)
        out[name] = float(r[:, 1].max() - r[:, 0].min()) * TICK_US
        w += 2 * g
    return out
