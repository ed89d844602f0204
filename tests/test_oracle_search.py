"""Pins of the oracle's predictive partition search (deep-dive 四 › 在线阶段: 预测搜索算法).

The recurrence is pinned to values evaluated by hand (tests/golden/search_toy.json),
to closed forms (no communication cost; no computation), and the curve
interpolation to its sample points and segment midpoints.
"""

import json
import os

import pytest

import oracle
from oracle.search import group_bytes, curve_latency, predict, search, wave_bytes_of
from oracle.tiles import make_plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "search_toy.json")


def _comp(key):
    return tuple(int(x) for x in key.split(","))


def test_hand_evaluated_toy():
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        for key, want in case["predictions"].items():
            got = predict(_comp(key), g["wave_bytes"], g["duration"], case["curve_bytes"], case["curve_seconds"])
            assert got == pytest.approx(want, abs=1e-12), (case["note"], key)
        best, best_t, all_t = search(g["wave_bytes"], g["duration"], case["curve_bytes"], case["curve_seconds"])
        assert list(best) == case["best"]
        assert best_t == pytest.approx(min(case["predictions"].values()))
        assert len(all_t) == 2 ** (len(g["wave_bytes"]) - 1)


def test_interpolation_at_samples_midpoints_and_ends():
    cb, cs = [10.0, 20.0, 40.0], [1.0, 3.0, 4.0]
    for b, s in zip(cb, cs):
        assert curve_latency(cb, cs, b) == s
    assert curve_latency(cb, cs, 15.0) == pytest.approx(2.0)
    assert curve_latency(cb, cs, 30.0) == pytest.approx(3.5)
    assert curve_latency(cb, cs, 5.0) == 1.0             # below the first sample: its latency
    assert curve_latency(cb, cs, 80.0) == pytest.approx(8.0)   # beyond: the last sample's bandwidth
    assert curve_latency(cb, cs, 0.0) == 0.0
    with pytest.raises(ValueError):
        curve_latency([2.0, 2.0], [1.0, 1.0], 1.0)


def test_free_communication_gives_the_gemm_duration_for_every_candidate():
    wb = [3.0, 5.0, 7.0, 2.0, 1.0]
    best, best_t, all_t = search(wb, 10.0, [1.0, 2.0], [0.0, 0.0])
    assert all(t == pytest.approx(10.0) for t in all_t)
    assert best == (1, 1, 1, 1, 1)                        # ties: the candidate with most groups


def test_equal_predictions_go_to_the_partition_with_most_groups():
    """A flat per-call cost shorter than a wave (worked by hand): every group's call ends a quarter wave
    after its computation, before the next group's computation does, so every partition ends at
    4 + 0.25; the tie goes to the partition with the most groups."""
    wb = [1.0, 1.0, 1.0, 1.0]
    cb, cs = [1.0, 100.0], [0.25, 0.25]
    best, best_t, all_t = search(wb, 4.0, cb, cs)
    assert all_t == [4.25] * 8
    assert best == (1, 1, 1, 1) and best_t == 4.25


def test_no_computation_sums_the_calls():
    """With zero GEMM time, every call waits only for the previous one: the sum of the latencies."""
    wb = [4.0, 1.0, 2.0, 8.0]
    cb, cs = [1.0, 16.0], [3.0, 6.0]                       # per-call cost 3 at 1 byte, +0.2 per byte
    for comp in oracle.enumerate_compositions(4):
        want = sum(curve_latency(cb, cs, s) for s in group_bytes(comp, wb))
        assert predict(comp, wb, 0.0, cb, cs) == pytest.approx(want)
    best, _, _ = search(wb, 0.0, cb, cs)
    assert best == (4,)                                   # a fixed per-call cost favours one call


def test_single_wave_partition_waits_for_the_whole_gemm():
    """P = 1: nothing overlaps, the prediction is the GEMM plus one call on everything."""
    wb = [2.0, 2.0, 2.0]
    assert predict((3,), wb, 9.0, [1.0, 100.0], [1.0, 100.0]) == pytest.approx(9.0 + 6.0)


def test_wave_bytes_cover_the_output():
    p = make_plan([2048], 8192, BM=256, BN=128, S=4, W=256)
    wb = wave_bytes_of(p)
    assert wb == [16 * 2 ** 20, 16 * 2 ** 20]
    q = make_plan([250], 200, BM=64, BN=64, S=3, W=5)    # ragged edges, partial last wave
    assert sum(wave_bytes_of(q)) == 250 * 200 * 2
    assert len(wave_bytes_of(q)) == q.T
