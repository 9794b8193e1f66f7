"""Host decoding of the in-kernel trace (mixture_experts_layer_mok_amd/trace.py) on
hand-made records: shares of the compute workgroups' time and per-kind means."""
import numpy as np

from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import trace as TR


def _wg(start, fill, role, drain, comm, chunks):
    return [start, fill, role, drain, comm, chunks, 0, 0]


def test_forward_summary_shares():
    # one comm workgroup (0) and one compute workgroup (1); times in 10 ns ticks, with a
    # start near the 32-bit wrap to check the modular arithmetic
    base = 2**32 - 50
    wgs = np.array([_wg(base, base + 10, base + 60, base + 100, 1, 3),
                    _wg(base, base + 10, base + 90, base + 100, 0, 1)], dtype=np.uint64)
    wgs = (wgs % 2**32).astype(np.uint32)
    # two tiles on workgroup 1: [ticket, ready, K done, signal done, epilogue issued]
    tiles = np.array([[1, 0, base + 10, base + 12, base + 40, base + 45, base + 44, 0],
                      [1, 3, base + 46, base + 50, base + 80, base + 88, base + 86, 0]],
                     dtype=np.uint64)
    tiles = (tiles % 2**32).astype(np.uint32)
    s = TR.summarize(tiles, wgs, comm_cus=1)
    assert s["span_us"] == 1.0 and s["compute_cus"] == 1
    sh = s["compute_share"]
    assert abs(sh["k_loop"] - 0.58) < 1e-9          # (28 + 30) / 100
    assert abs(sh["epilogue_and_signal"] - 0.13) < 1e-9  # (5 + 8) / 100
    assert abs(sh["wait_for_inputs"] - 0.06) < 1e-9      # (2 + 4) / 100
    assert abs(sh["between_tiles"] - 0.03) < 1e-9        # 80 - 77 inside tiles
    assert abs(sh["fill"] - 0.10) < 1e-9 and abs(sh["after_role"] - 0.10) < 1e-9
    assert abs(sum(sh.values()) - 1.0) < 1e-9
    assert s["tile_us"]["gemm1"]["n"] == 1 and s["tile_us"]["gemm2"]["n"] == 1
    assert s["tile_us"]["gemm2"]["epilogue_issue"] == 0.06   # 86 - 80 ticks
    assert s["comm"]["drain_chunks"] == 3 and s["drain_chunks_compute"] == 1


def test_backward_summary():
    wgs = np.array([[0, 0, 200, 200, 0, 2, 0, 0], [0, 0, 200, 200, 0, 1, 0, 0]], dtype=np.uint32)
    recs = np.array([[0, 0, 0, 0, 80, 100, 0, 0],      # dH: K 80, epilogue 20
                     [1, 1, 0, 10, 150, 160, 0, 0],    # dX: wait 10, K 140, epilogue 10
                     [0, 3, 100, 100, 130, 130, 0, 0]],  # row sums: 30
                    dtype=np.uint32)
    s = TR.summarize_bwd(recs, wgs)
    assert s["span_us"] == 2.0 and s["workgroups"] == 2
    k = s["kinds"]
    assert k["dh"]["k_loop_us"] == 0.8 and k["dh"]["epilogue_us"] == 0.2
    assert k["dx"]["wait_us"] == 0.1 and k["dx"]["k_loop_us"] == 1.4
    assert k["row_sums"]["sum_us"] == 0.3 and "dw" not in k
    assert abs(s["outside_tickets_share"] - (1 - 290 / 400)) < 1e-4
    shape = dict(hidden=512, intermediate=256, num_local_experts=2, num_tokens=64)
    for prec, quant in ((L.MOK_PREC_BF16, 0), (L.MOK_PREC_MXFP8, 1)):
        desc = type("D", (), dict(shape, precision=prec))()
        assert TR.bwd_tickets(desc, 3) == 3 * (1 + 2 + quant) + 2 * 3 * 2 + 2
