"""Pins for the oracle's tile grid, dispatch order, waves, groups and counting table.

Each test pins the oracle to something other than itself: the pages' printed
worked examples (tests/golden/*.json, each with its citation), a brute-force
re-derivation, or a hand-computed case.
"""

import itertools
import json
import os

import pytest

import oracle
from oracle.tiles import make_plan, swizzle_order, counting_trajectory
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- counting table

def test_pages_counting_table_example():
    """Deep-dive 一 › 组级 Tile 计数: 8 tiles, 4 waves, groups {W1},{W2,W3},{W4}."""
    g = _golden("counting_table_example.json")
    W = g["tiles_per_wave"]
    comp = tuple(len(ws) for ws in g["group_waves"])
    # 8 tiles with the identity dispatch order (S = 1): any grid with 8 tiles
    plan = make_plan(2 * 4, 4 * 4, BM=4, BN=4, S=1, W=W, composition=comp)
    assert plan.NT == g["tiles"] and plan.T == g["waves"] and plan.P == g["table_size"]
    assert plan.group_tiles == g["thresholds"]
    for j, ids in enumerate(g["group_tile_ids"]):
        assert [plan.tile_of_b[b] for b in range(plan.NT) if plan.group_of_b[b] == j] == ids
    snaps, fire = counting_trajectory(plan)
    assert snaps == g["table_after_wave"]
    assert [w + 1 for w in fire] == g["group_fires_after_wave"]
    assert snaps[-1] == g["thresholds"]


def test_tiny_workload_hand_derived():
    """4x4 tile grid, S = 2, W = 4, groups (1, 2, 1): derived by hand.

    Bands of 2 tile rows; inside a band the order walks down each column:
    (0,0),(1,0),(0,1),(1,1),(0,2),(1,2),(0,3),(1,3), then rows 2-3 likewise.
    """
    plan = make_plan(256, 256, BM=64, BN=64, S=2, W=4, composition=(1, 2, 1))
    assert plan.tile_of_b == [0, 4, 1, 5, 2, 6, 3, 7, 8, 12, 9, 13, 10, 14, 11, 15]
    slot_of_tile, _ = oracle.mapping_table(plan)
    assert slot_of_tile == [0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15]
    waves = [sorted(plan.tile_of_b[b] for b in range(16) if plan.wave_of_b[b] == w) for w in range(4)]
    assert waves == [[0, 1, 4, 5], [2, 3, 6, 7], [8, 9, 12, 13], [10, 11, 14, 15]]
    snaps, fire = counting_trajectory(plan)
    assert snaps == [[4, 0, 0], [4, 4, 0], [4, 8, 0], [4, 8, 4]]
    assert fire == [0, 2, 3]


def _swizzle_brute(tm_n, tn_n, S):
    """Grouped-M order written as nested loops: band, then column, then row."""
    out = []
    for band_start in range(0, tm_n, S):
        rows = range(band_start, min(band_start + S, tm_n))
        for tn in range(tn_n):
            for tm in rows:
                out.append(tm * tn_n + tn)
    return out


@pytest.mark.parametrize("tm_n,tn_n,S", [(a, b, s) for a in range(1, 9) for b in range(1, 9) for s in range(1, 6)])
def test_swizzle_matches_nested_loops_and_is_bijection(tm_n, tn_n, S):
    order = swizzle_order(tm_n, tn_n, S)
    assert order == _swizzle_brute(tm_n, tn_n, S)
    assert sorted(order) == list(range(tm_n * tn_n))


def test_swizzle_width_one_is_row_major():
    assert swizzle_order(3, 5, 1) == list(range(15))


def test_waves_and_partial_last_wave():
    plan = make_plan(300, 200, BM=64, BN=64, S=3, W=7)     # 5 x 4 = 20 tiles, ragged edges
    assert plan.NT == 20 and plan.T == 3
    assert [plan.wave_of_b.count(w) for w in range(3)] == [7, 7, 6]
    snaps, fire = counting_trajectory(plan)
    assert snaps == [[7, 0, 0], [7, 7, 0], [7, 7, 6]]
    assert fire == [0, 1, 2]


def test_counting_fire_once_and_final_table_random_partitions():
    plan0 = make_plan(640, 384, BM=64, BN=64, S=4, W=9)
    T = plan0.T
    for comp in oracle.enumerate_compositions(T)[:: max(1, 2 ** (T - 1) // 40)]:
        plan = make_plan(640, 384, BM=64, BN=64, S=4, W=9, composition=comp)
        snaps, fire = counting_trajectory(plan)
        assert snaps[-1] == plan.group_tiles
        assert sum(plan.group_tiles) == plan.NT
        # group j fires at the last wave of its waves, and fires exactly once
        ends = list(itertools.accumulate(comp))
        assert fire == [e - 1 for e in ends]
        for j in range(plan.P):
            full = [w for w in range(T) if snaps[w][j] == plan.group_tiles[j]]
            assert full and full[0] == fire[j]
        # counts never decrease and never pass the threshold
        for a, b in zip(snaps, snaps[1:]):
            assert all(x <= y for x, y in zip(a, b))
        assert all(s[j] <= plan.group_tiles[j] for s in snaps for j in range(plan.P))


def test_grouped_problems_concatenate_and_swizzle_inside():
    plan = make_plan([130, 0, 64], 128, BM=64, BN=64, S=2, W=4)
    # problem 0: 3 x 2 tiles (ids 0..5), problem 1: none, problem 2: 1 x 2 (ids 6, 7)
    assert plan.NT == 8
    assert plan.tile_of_b == [0, 2, 1, 3, 4, 5, 6, 7]
    assert plan.tile_rows == [64, 64, 64, 64, 2, 2, 64, 64]
    assert plan.tile_row0 == [0, 0, 64, 64, 128, 128, 130, 130]
    assert plan.tile_problem == [0, 0, 0, 0, 0, 0, 2, 2]


def test_invalid_partitions_rejected():
    with pytest.raises(ValueError):
        make_plan(256, 256, BM=64, BN=64, S=2, W=4, composition=(1, 2))      # sums to 3, T = 4
    with pytest.raises(ValueError):
        make_plan(256, 256, BM=64, BN=64, S=2, W=4, composition=(0, 4))
    with pytest.raises(ValueError):
        make_plan(256, 256, BM=64, BN=64, S=2, W=4, mode="subtile", ranks=3)  # 64 % 3
    with pytest.raises(ValueError):
        make_plan(250, 256, BM=64, BN=64, S=2, W=4, mode="subtile", ranks=4)  # ragged M


def test_empty_problem():
    plan = make_plan(0, 128, BM=64, BN=64, S=2, W=4, composition=())
    assert plan.NT == 0 and plan.T == 0 and plan.P == 0
    assert counting_trajectory(plan) == ([], [])
