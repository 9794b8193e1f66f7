"""Host-side sizing rules for the layer's launch parameters.

The two-waves rule (Leiphone article on MoK, section 02; news brief, section on the
three design decisions): a minibatch should give each grouped GEMM at least two full
waves of output tiles on the compute units.  For GEMM1, whose output is the 2I fused
gate/up columns of every row, a minibatch of M rows holds (M / tile_m) * (2I / tile_n)
tiles, so two waves need M >= 2 * compute_units * tile_m * tile_n / (2I).
"""
from __future__ import annotations


def two_wave_min_rows(compute_units: int, tile_m: int, tile_n: int, intermediate: int) -> float:
    """Smallest minibatch (rows) for which GEMM1 has two full waves of tiles."""
    if min(compute_units, tile_m, tile_n, intermediate) <= 0:
        raise ValueError("sizes must be positive")
    return 2.0 * compute_units * tile_m * tile_n / (2.0 * intermediate)


# This build's tile: 256 rows x 256 B rows (128 gate + 128 up columns) per workgroup.
TILE_M = 256
TILE_N = 256


def layer_two_wave_min_rows(total_cus: int, comm_cus: int, intermediate: int) -> float:
    return two_wave_min_rows(total_cus - comm_cus, TILE_M, TILE_N, intermediate)
