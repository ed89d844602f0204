"""Pins for the mapping table, the three reorder layouts and the reorders.

Pins: the pages' printed mapping example, bijection and round trips on
tiny shapes, group contiguity, and the ReduceScatter / All-to-All
invariants that the deep-dive states in 二 › 不同通信原语的重排模式.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.layout import element_offsets, consumer_units, group_spans, row_offsets
from oracle.tiles import make_plan
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_pages_mapping_example():
    g = _golden("mapping_table_example.json")
    order = g["execution_order"]
    plan = make_plan(2, 8, BM=1, BN=4, S=1, W=4, dispatch_order=order)   # 2 x 2 tiles
    slot_of_tile, tile_of_slot = oracle.mapping_table(plan)
    assert {str(t): slot_of_tile[t] for t in range(4)} == g["mapping_table"]
    assert {str(s): tile_of_slot[s] for s in range(4)} == g["inverse_mapping_table"]
    # the pre-reordered buffer holds tile 0, 3, 1, 2 in that order
    X = np.arange(16, dtype=np.int64).reshape(2, 8)
    off = element_offsets(plan)
    flat = oracle.pre_reorder(X, off)
    tiles = {0: X[0, 0:4], 1: X[0, 4:8], 2: X[1, 0:4], 3: X[1, 4:8]}
    assert flat.tolist() == np.concatenate([tiles[t] for t in order]).tolist()


def _random_row_dest(M, D, seed):
    return np.random.Generator(np.random.PCG64(seed)).integers(0, D, size=M)


CASES = [
    dict(m=[256], N=256, BM=64, BN=64, S=2, W=4, mode="tile"),
    dict(m=[250], N=200, BM=64, BN=64, S=3, W=5, mode="tile"),            # ragged rows and cols
    dict(m=[33], N=17, BM=16, BN=8, S=2, W=3, mode="tile"),
    dict(m=[256], N=256, BM=64, BN=64, S=2, W=4, mode="subtile", ranks=4),
    dict(m=[512], N=128, BM=32, BN=32, S=3, W=5, mode="subtile", ranks=2),
    dict(m=[70, 0, 130, 64], N=96, BM=32, BN=32, S=2, W=6, mode="subtoken", ranks=4),
    dict(m=[100, 60], N=40, BM=64, BN=16, S=1, W=3, mode="subtoken", ranks=3),  # ragged cols
]


def _plan(c, comp_index=None):
    base = make_plan(c["m"], c["N"], BM=c["BM"], BN=c["BN"], S=c["S"], W=c["W"],
                     mode=c["mode"], ranks=c.get("ranks", 1),
                     row_dest=_random_row_dest(sum(c["m"]), c.get("ranks", 1), 7) if c["mode"] == "subtoken" else None)
    comps = oracle.enumerate_compositions(base.T)
    comp = comps[(comp_index or 0) % len(comps)]
    return make_plan(c["m"], c["N"], BM=c["BM"], BN=c["BN"], S=c["S"], W=c["W"], composition=comp,
                     mode=c["mode"], ranks=c.get("ranks", 1), row_dest=base.row_dest)


@pytest.mark.parametrize("ci", range(len(CASES)))
@pytest.mark.parametrize("comp_index", [0, 1, 5])
def test_offsets_are_permutation_and_groups_contiguous(ci, comp_index):
    plan = _plan(CASES[ci], comp_index)
    off = element_offsets(plan)
    assert off.shape == (plan.M, plan.N)
    assert np.array_equal(np.sort(off.ravel()), np.arange(plan.M * plan.N))
    spans = group_spans(plan)
    # every element of a group's tiles lies inside that group's span
    for s in range(plan.NT):
        t = plan.tile_of_b[s]
        j = plan.group_of_b[s]
        r0, c0 = plan.tile_row0[t], plan.tile_col0[t]
        blk = off[r0:r0 + plan.tile_rows[t], c0:c0 + plan.tile_cols[t]]
        assert blk.min() >= spans[j] and blk.max() < spans[j + 1]
    # group slots form one consecutive run
    for j in range(plan.P):
        sl = [s for s in range(plan.NT) if plan.group_of_b[s] == j]
        assert sl == list(range(sl[0], sl[-1] + 1))


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_round_trips_bit_exact(ci):
    plan = _plan(CASES[ci], 3)
    off = element_offsets(plan)
    rng = np.random.Generator(np.random.PCG64(99))
    X = rng.integers(0, 1 << 16, size=(plan.M, plan.N)).astype(np.uint16)
    Y = rng.integers(0, 1 << 16, size=plan.M * plan.N).astype(np.uint16)
    assert np.array_equal(oracle.post_reorder(oracle.pre_reorder(X, off), off), X)
    assert np.array_equal(oracle.pre_reorder(oracle.post_reorder(Y, off), off), Y)


def test_tile_mode_full_tiles_base_is_slot_times_tile():
    plan = make_plan(512, 384, BM=64, BN=128, S=3, W=5)
    ro = row_offsets(plan)
    for s in range(plan.NT):
        assert ro[s][0] == s * 64 * 128
        assert np.array_equal(np.diff(ro[s]), np.full(63, 128))


def test_intra_tile_row_major():
    plan = make_plan(130, 70, BM=64, BN=32, S=2, W=3)
    off = element_offsets(plan)
    for s in range(plan.NT):
        t = plan.tile_of_b[s]
        r0, c0, rows, cols = plan.tile_row0[t], plan.tile_col0[t], plan.tile_rows[t], plan.tile_cols[t]
        blk = off[r0:r0 + rows, c0:c0 + cols]
        assert np.array_equal(blk - blk[0, 0], np.arange(rows * cols).reshape(rows, cols))


@pytest.mark.parametrize("R,BM", [(4, 64), (2, 32), (8, 64)])
def test_reduce_scatter_kth_segments_are_complete_rows(R, BM):
    """All k-th subtiles together are complete rows (deep-dive 二 › (2))."""
    M, N = 4 * BM, 3 * 32
    plan0 = make_plan(M, N, BM=BM, BN=32, S=2, W=5, mode="subtile", ranks=R)
    for comp in oracle.enumerate_compositions(plan0.T):
        plan = make_plan(M, N, BM=BM, BN=32, S=2, W=5, composition=comp, mode="subtile", ranks=R)
        off = element_offsets(plan)
        row_id = np.repeat(np.arange(M)[:, None], N, axis=1)
        col_id = np.repeat(np.arange(N)[None, :], M, axis=0)
        flat_r = oracle.pre_reorder(row_id, off)
        flat_c = oracle.pre_reorder(col_id, off)
        units = consumer_units(plan)
        band = BM // R
        for k in range(R):
            rows = np.concatenate([flat_r[u[k][0]:u[k][1]] for u in units])
            cols = np.concatenate([flat_c[u[k][0]:u[k][1]] for u in units])
            want_rows = [m for m in range(M) if (m % BM) // band == k]
            # segment k, over all groups, is exactly those rows, each with every column
            assert sorted(set(rows.tolist())) == want_rows
            pairs = set(zip(rows.tolist(), cols.tolist()))
            assert len(pairs) == len(rows) == len(want_rows) * N


def test_all_to_all_buckets_are_destination_rows():
    """Subtokens bound for one destination are contiguous (deep-dive 二 › (3))."""
    m = [70, 0, 130, 64]
    D = 4
    dest = _random_row_dest(sum(m), D, 11)
    plan0 = make_plan(m, 96, BM=32, BN=32, S=2, W=6, mode="subtoken", ranks=D, row_dest=dest)
    for comp in oracle.enumerate_compositions(plan0.T)[::3]:
        plan = make_plan(m, 96, BM=32, BN=32, S=2, W=6, composition=comp, mode="subtoken", ranks=D, row_dest=dest)
        off = element_offsets(plan)
        Mt = sum(m)
        row_id = np.repeat(np.arange(Mt)[:, None], 96, axis=1)
        flat_r = oracle.pre_reorder(row_id, off)
        units = consumer_units(plan)
        for d in range(D):
            seg_rows = np.concatenate([flat_r[u[d][0]:u[d][1]] for u in units])
            assert np.all(dest[seg_rows] == d)
            assert seg_rows.size == np.count_nonzero(dest == d) * 96     # routing histogram x N
        # inside each bucket of each group: slot order, then row order
        for j, u in enumerate(units):
            for d in range(D):
                r = flat_r[u[d][0]:u[d][1]][::32] if u[d][1] > u[d][0] else np.array([], dtype=np.int64)
                slots = [s for s in range(plan.NT) if plan.group_of_b[s] == j]
                want = []
                for s in slots:
                    t = plan.tile_of_b[s]
                    for rr in range(plan.tile_rows[t]):
                        if dest[plan.tile_row0[t] + rr] == d:
                            want.append(plan.tile_row0[t] + rr)
                assert r.tolist() == want


def test_units_cover_spans():
    for c in CASES:
        plan = _plan(c, 2)
        spans = group_spans(plan)
        for j, u in enumerate(consumer_units(plan)):
            assert u[0][0] == spans[j] and u[-1][1] == spans[j + 1]
            assert all(a[1] == b[0] for a, b in zip(u, u[1:]))
