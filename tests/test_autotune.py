"""Host logic of the per-shape tuner: candidate grids, shape keys and the JSON cache."""
import json

import pytest

from mixture_experts_layer_mok_amd import _lib as L
from mixture_experts_layer_mok_amd import autotune as A
from mixture_experts_layer_mok_amd.tuning import layer_two_wave_min_rows


def test_r_bucket():
    assert [A.r_bucket(r) for r in (0, 1, 2, 3, 16270, 16384, 16385)] == [1, 1, 2, 4, 16384,
                                                                           16384, 32768]


@pytest.mark.parametrize("R,comm,I", [(16270, 20, 2048), (86552, 32, 2048), (16384, 32, 1024),
                                      (256, 8, 64)])
def test_candidate_minibatches_bracket_two_waves(R, comm, I):
    ms = A.candidate_minibatches(R, 256, comm, I)
    assert ms == sorted(set(ms)) and ms
    assert all(m % 512 == 0 and 512 <= m <= 8192 for m in ms)
    hi = -(-R // 512) * 512
    assert all(m <= max(512, hi) for m in ms)
    two = layer_two_wave_min_rows(256, comm, I)
    if two <= min(8192, hi):  # the threshold itself is on the grid when it is reachable
        assert any(abs(m - two) <= 256 for m in ms)


@pytest.mark.parametrize("prec", [L.MOK_PREC_BF16, L.MOK_PREC_MXFP8])
def test_candidate_comm_cus(prec):
    cs = A.candidate_comm_cus(256, prec)
    assert cs == sorted(cs) and len(cs) >= 3
    assert all(c % 4 == 0 and 8 <= c <= 64 for c in cs)
    if prec == L.MOK_PREC_MXFP8:
        assert min(cs) >= 16


def test_shape_key_and_cache_roundtrip(tmp_path):
    d = L.make_desc(16384, 7168, 2048, 64, 8, e0=0, E_loc=8, M=2048, S=4, comm_cus=20)
    k1 = A.shape_key(d, 16270, "gpu", 256).text()
    assert k1 == A.shape_key(d, 16000, "gpu", 256).text()       # same bucket
    assert k1 != A.shape_key(d, 17000, "gpu", 256).text()       # next bucket
    d2 = L.make_desc(16384, 7168, 2048, 64, 8, e0=0, E_loc=8, M=2048, S=4, comm_cus=20,
                     precision=L.MOK_PREC_MXFP8)
    assert k1 != A.shape_key(d2, 16270, "gpu", 256).text()
    p = tmp_path / "tune.json"
    assert A.load_cache(str(p)) == {}
    c = A.Choice(2048, 20, 1.61, [{"minibatch_rows": 2048, "comm_cus": 20, "fwd_ms": 1.61}])
    A.save_cache(str(p), {k1: c.to_json()})
    back = A.load_cache(str(p))
    assert back[k1]["minibatch_rows"] == 2048 and back[k1]["comm_cus"] == 20
    json.loads(p.read_text())
