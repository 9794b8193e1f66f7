"""Torch-facing convenience over the C ABI: owns a workspace tensor for one descriptor
and calls the library entry points.  PyTorch provides device memory and streams only;
every step of the layer runs in libmok's kernels."""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 device tensor holding the given uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(t: torch.Tensor) -> np.ndarray:
    return (bf16_bits(t).astype(np.uint32) << 16).view(np.float32)


class MoKLayer:
    def __init__(self, desc: L.mok_desc_t, device="cuda"):
        self.desc = desc
        self.device = torch.device(device)
        self.ws_bytes = L.mok_workspace_size(desc)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)

    def schedule(self, ids: torch.Tensor, stream=None) -> None:
        L.mok_schedule(self.desc, ids, self.ws, self.ws_bytes, stream)

    def forward(self, x, ids, gates, wg, wu, wd, scales=(None, None, None), y=None, stream=None):
        if y is None:
            y = torch.empty((self.desc.num_tokens, self.desc.hidden), dtype=torch.bfloat16,
                            device=self.device)
        L.mok_moe_fwd(self.desc, x, ids, gates, wg, wu, wd, scales[0], scales[1], scales[2], y,
                      self.ws, self.ws_bytes, stream)
        return y

    def backward(self, dy, x, ids, gates, wg, wu, wd, stream=None):
        d = self.desc
        T, D, I, k, nl = d.num_tokens, d.hidden, d.intermediate, d.top_k, d.num_local_experts
        dx = torch.empty((T, D), dtype=torch.bfloat16, device=self.device)
        dg = torch.empty((T, k), dtype=torch.float32, device=self.device)
        dwg = torch.empty((nl, I, D), dtype=torch.float32, device=self.device)
        dwu = torch.empty((nl, I, D), dtype=torch.float32, device=self.device)
        dwd = torch.empty((nl, D, I), dtype=torch.float32, device=self.device)
        L.mok_moe_bwd(d, dy, x, ids, gates, wg, wu, wd, dx, dg, dwg, dwu, dwd, self.ws,
                      self.ws_bytes, stream)
        return dict(dx=dx, dg=dg, dwg=dwg, dwu=dwu, dwd=dwd)

    def backward_mx(self, dy, x, ids, gates, wt, stream=None):
        """MXFP8 backward; wt = (wd_t, wd_t_scales, wgu_t, wgu_t_scales) from
        quantize_weights_bwd."""
        d = self.desc
        T, D, I, k, nl = d.num_tokens, d.hidden, d.intermediate, d.top_k, d.num_local_experts
        dx = torch.empty((T, D), dtype=torch.bfloat16, device=self.device)
        dg = torch.empty((T, k), dtype=torch.float32, device=self.device)
        dwg = torch.empty((nl, I, D), dtype=torch.float32, device=self.device)
        dwu = torch.empty((nl, I, D), dtype=torch.float32, device=self.device)
        dwd = torch.empty((nl, D, I), dtype=torch.float32, device=self.device)
        L.mok_moe_bwd_mx(d, dy, x, ids, gates, *wt, dx, dg, dwg, dwu, dwd, self.ws,
                         self.ws_bytes, stream)
        return dict(dx=dx, dg=dg, dwg=dwg, dwu=dwu, dwd=dwd)

    def quantize_weights_bwd(self, wg, wu, wd, stream=None):
        """The MXFP8 backward's weight operands: W_down^T codes [E_loc, I, D] with scales
        [E_loc, I, D/32], and [W_gate; W_up]^T codes [E_loc, D, 2I] with scales
        [E_loc, D, 2I/32] (blocks of 32 along each GEMM's K)."""
        nl, I, D = wg.shape
        dev = self.device
        wdt = torch.empty((nl, I, D), dtype=torch.uint8, device=dev)
        wdts = torch.empty((nl, I, D // 32), dtype=torch.uint8, device=dev)
        wgut = torch.empty((nl, D, 2 * I), dtype=torch.uint8, device=dev)
        wguts = torch.empty((nl, D, 2 * I // 32), dtype=torch.uint8, device=dev)
        L.mok_quantize_mx_t(wd, nl, D, I, wdt, D, wdts, D // 32, stream)
        L.mok_quantize_mx_t(wg, nl, I, D, wgut, 2 * I, wguts, 2 * I // 32, stream)
        L.mok_quantize_mx_t(wu, nl, I, D, wgut.data_ptr() + I, 2 * I, wguts.data_ptr() + I // 32,
                            2 * I // 32, stream)
        return wdt, wdts, wgut, wguts

    def tables(self, stream=None) -> dict:
        d = self.desc
        TK = d.num_tokens * d.top_k
        nl = d.num_local_experts
        dev = self.device
        out = dict(counts=torch.empty(nl, dtype=torch.int32, device=dev),
                   offsets=torch.empty(nl + 1, dtype=torch.int32, device=dev),
                   perm=torch.empty(TK, dtype=torch.int32, device=dev),
                   pos=torch.empty(TK, dtype=torch.int32, device=dev),
                   hdr=torch.empty(4, dtype=torch.int32, device=dev))
        L.mok_schedule_tables(d, self.ws, out["counts"], out["offsets"], out["perm"], out["pos"],
                              out["hdr"], self.ws_bytes, stream)
        torch.cuda.synchronize(dev)
        res = {k: v.cpu().numpy() for k, v in out.items()}
        R = int(res["hdr"][0])
        res["perm"] = res["perm"][:R]
        res["R"], res["n_mb"], res["n_mtiles"], res["status"] = (int(v) for v in res["hdr"])
        return res

    def status(self, stream=None) -> int:
        return L.mok_read_device_status(self.ws, stream)

    def quantize_weights(self, w: torch.Tensor, stream=None):
        """MXFP8 codes and scales of a bf16 weight tensor, blocks along its last axis."""
        cols = w.shape[-1]
        rows = w.numel() // cols
        codes = torch.empty(w.shape, dtype=torch.uint8, device=self.device)
        scales = torch.empty(tuple(w.shape[:-1]) + (cols // 32,), dtype=torch.uint8,
                             device=self.device)
        L.mok_quantize_mx(w, rows, cols, codes, scales, stream)
        return codes, scales


def forward_macrobatches(layers, streams, batches, ys):
    """Forwards of successive macrobatches with the combine of each overlapping the
    dispatch of the next: macrobatch i runs on layers[i % 2] (their own workspaces, built
    with MOK_FLAG_OVERLAP_NEXT) and streams[i % 2], so a workspace is reused only by the
    next call on its own stream.  Each schedule is issued ahead of the previous
    macrobatch's forward, so it never waits behind it.  batches[i] = (x, ids, gates, wg,
    wu, wd[, scales]); ys[i] receives the output.  Returns without synchronising."""
    n = len(batches)

    def args(i):
        b = batches[i]
        return b[:6], (b[6] if len(b) > 6 else (None, None, None))

    if n == 0:
        return ys
    layers[0].schedule(batches[0][1], stream=streams[0])
    for i in range(n):
        if i + 1 < n:
            j = (i + 1) % 2
            layers[j].schedule(batches[i + 1][1], stream=streams[j])
        (x, ids, gates, wg, wu, wd), sc = args(i)
        layers[i % 2].forward(x, ids, gates, wg, wu, wd, scales=sc, y=ys[i],
                              stream=streams[i % 2])
    return ys
