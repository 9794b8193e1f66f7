"""Host-side bounds check of the GEMM tile's load offsets (no GPU): compiles
csrc/tile_bounds_check.cpp with the host compiler and runs it for every shape the
tests and the benchmark use, plus ragged edge cases."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_mok_amd", "csrc")
EXE = os.path.join(ROOT, "_build", "tile_bounds_check")


@pytest.fixture(scope="module")
def checker():
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    subprocess.run(["g++", "-O2", "-std=c++17", "-o", EXE,
                    os.path.join(CSRC, "tile_bounds_check.cpp")], check=True)
    return EXE


@pytest.mark.parametrize("D,I", [(128, 64), (192, 192), (128, 128), (256, 320), (2048, 1024),
                                 (7168, 2048), (64, 64), (320, 448)])
def test_tile_offsets_in_bounds(checker, D, I):
    r = subprocess.run([checker, str(D), str(I)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
