"""fo_plan_search (host C++) against the oracle's predictive search, candidate by candidate.

Both walk the candidates in cut-mask order; the predictions agree to rounding
(relative 1e-12) and the chosen composition has the oracle's best prediction.
Host-only plans: no GPU needed.
"""

import json
import os

import numpy as np
import pytest

from oracle.search import search, wave_bytes_of
from oracle.tiles import make_plan

fo = pytest.importorskip("gemm_tile_signaling_amd")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "search_toy.json")


def _curve(seed, n=6):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = np.cumsum(rng.uniform(1e4, 4e6, size=n))
    y = np.sort(rng.uniform(2e-6, 4e-4, size=n))
    return x, y


def _compare(m, N, BM, BN, S, W, gemm_s, curve, mode="tile", ranks=1, row_dest=None):
    o = make_plan(m, N, BM=BM, BN=BN, S=S, W=W, mode=mode, ranks=ranks, row_dest=row_dest)
    p = fo.Plan(m, N, 64, "bf16", BM=BM, BN=BN, swizzle=S, wave_size=W, mode=mode, ranks=ranks,
                row_dest=row_dest, host_only=True)
    assert p.T == o.T
    best, best_t, all_t = search(wave_bytes_of(o), gemm_s, list(curve[0]), list(curve[1]))
    comp, t, allg = p.search(gemm_s, curve[0], curve[1], with_all=True)
    np.testing.assert_allclose(allg, np.array(all_t), rtol=1e-12, atol=0)
    assert t == pytest.approx(best_t, rel=1e-12)
    assert sum(comp) == p.T
    assert allg[int(sum(1 << (sum(comp[:i + 1]) - 1) for i in range(len(comp) - 1)))] == t
    return comp, best


def test_hand_evaluated_toy_through_the_library():
    g = json.load(open(GOLDEN))
    p = fo.Plan(256, 64, 64, "bf16", BM=64, BN=64, swizzle=1, wave_size=1, host_only=True)  # 4 one-tile waves
    assert p.T == 4
    scale = 64 * 64 * 2                                      # bytes of one wave here
    for case in g["cases"]:
        cb = np.array(case["curve_bytes"]) * scale
        comp, t, allg = p.search(g["duration"], cb, case["curve_seconds"], with_all=True)
        assert list(comp) == case["best"]
        assert t == pytest.approx(min(case["predictions"].values()))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tile_mode_random_curves(seed):
    _compare([1000], 264, 128, 128, 3, 7, 1e-4 * seed, _curve(seed))


def test_profiled_and_prefill_shapes():
    _compare([2048], 8192, 256, 128, 4, 256, 250e-6, _curve(11))
    comp, best = _compare([4096], 8192, 256, 128, 4, 256, 220e-6, _curve(12))
    assert len(comp) >= 1


def test_moe_shape_seventeen_waves():
    from workloads import WORKLOADS, moe_routing
    w = WORKLOADS["moe_a2a"]
    m_per, tok = moe_routing(w)
    dest = tok // (w.tokens // w.ranks)
    _compare(m_per, w.N, 256, 128, 4, 256, 400e-6, _curve(13), mode="subtoken", ranks=8, row_dest=dest)


def test_search_errors():
    p = fo.Plan(256, 64, 64, "bf16", BM=64, BN=64, swizzle=1, wave_size=1, host_only=True)
    with pytest.raises(fo.FoError) as e:
        p.search(1.0, [2.0, 1.0], [1.0, 2.0])                # sizes not increasing
    assert e.value.code == fo.FO_ERR_INVALID
    with pytest.raises(fo.FoError) as e:
        p.search(-1.0, [1.0], [1.0])
    assert e.value.code == fo.FO_ERR_INVALID
    with pytest.raises(fo.FoError) as e:
        p.search(1.0, [1.0], [-1.0])
    assert e.value.code == fo.FO_ERR_INVALID
    big = fo.Plan(64 * 25, 64, 64, "bf16", BM=64, BN=64, swizzle=1, wave_size=1, host_only=True)   # T = 25
    with pytest.raises(fo.FoError) as e:
        big.search(1.0, [1.0], [1.0])
    assert e.value.code == fo.FO_ERR_UNSUPPORTED
    empty = fo.Plan(0, 64, 64, "bf16", BM=64, BN=64, swizzle=1, wave_size=4, composition=(), host_only=True)
    assert empty.search(1.0, [1.0], [1.0]) == ((), 0.0, None)
