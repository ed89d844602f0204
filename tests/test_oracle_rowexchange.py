"""Pins for the ReduceScatter shards and the row exchange after the AllGather.

Deep-dive 二、重排机制 › 不同通信原语的重排模式, (2) ReduceScatter + AllGather:
piece k of every tile ends on rank k, the k-th pieces form complete rows, and
a block-cyclic row exchange without a mapping table restores the row order.
Pins: hand-worked examples (tests/golden/row_exchange_example.json); each
rank segment of every group (the consumer's work units, one ReduceScatter
call's piece for rank k) lands in shard k and nowhere else; every shard
holds whole rows; the gathered position of a row is block-cyclic; shards
followed by the exchange equal the post-communication reorder, with and
without the element-wise epilogue.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.epilogue import post_epilogue, row_problems
from oracle.layout import consumer_units, element_offsets
from oracle.rowexchange import (gathered_offsets, gathered_rows, row_exchange, row_exchange_epilogue, row_owner,
                                shard_reorder)
from oracle.tiles import make_plan
from tests.conftest import GOLDEN
from workloads import draw, random_bits, to_bits

CASES = [
    dict(m=[256], N=256, BM=64, BN=64, S=2, W=4, R=4),
    dict(m=[512], N=128, BM=32, BN=32, S=3, W=5, R=2),
    dict(m=[128, 0, 64], N=96, BM=32, BN=32, S=2, W=3, R=8),
    dict(m=[96], N=48, BM=16, BN=16, S=1, W=7, R=16),
]


def _plans(c):
    base = make_plan(c["m"], c["N"], BM=c["BM"], BN=c["BN"], S=c["S"], W=c["W"], mode="subtile", ranks=c["R"])
    for comp in oracle.enumerate_compositions(base.T)[:6]:
        yield make_plan(c["m"], c["N"], BM=c["BM"], BN=c["BN"], S=c["S"], W=c["W"], composition=comp,
                        mode="subtile", ranks=c["R"])


def test_hand_worked_examples():
    with open(os.path.join(GOLDEN, "row_exchange_example.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        plan = make_plan(c["m_per_problem"], 4, BM=c["BM"], BN=4, S=1, W=1, mode="subtile", ranks=c["R"])
        assert row_owner(plan).tolist() == c["owner"]
        assert gathered_rows(plan).tolist() == c["gathered"]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_rank_segments_land_in_their_shard(ci):
    """The piece every ReduceScatter call delivers to rank k (segment k of each group's span) is part of
    rank k's shard, and the shards hold nothing else."""
    for plan in _plans(CASES[ci]):
        off = element_offsets(plan)
        recv = np.arange(plan.M * plan.N, dtype=np.int64)        # each element names its reordered offset
        gathered = shard_reorder(recv, off, plan)
        per = plan.M // plan.ranks * plan.N
        for k in range(plan.ranks):
            shard = np.sort(gathered[k * per:(k + 1) * per])
            want = np.sort(np.concatenate([np.arange(*units[k]) for units in consumer_units(plan)]))
            assert np.array_equal(shard, want), k


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_shards_hold_whole_rows_and_positions_are_block_cyclic(ci):
    c = CASES[ci]
    plan = next(_plans(c))
    G = gathered_rows(plan)
    assert np.array_equal(np.sort(G), np.arange(plan.M))          # a permutation of the rows
    goff = gathered_offsets(plan)
    assert np.array_equal(np.sort(goff.ravel()), np.arange(plan.M * plan.N))
    assert np.all(goff % plan.N == np.arange(plan.N)[None, :])     # whole rows move, columns in place
    band, shard = plan.BM // plan.ranks, plan.M // plan.ranks
    m = np.arange(plan.M)
    block_cyclic = ((m % plan.BM) // band) * shard + (m // plan.BM) * band + m % band
    assert np.array_equal(goff[:, 0] // plan.N, block_cyclic)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_shards_then_exchange_is_the_post_reorder(ci):
    for plan in _plans(CASES[ci]):
        off = element_offsets(plan)
        Y = random_bits(13, plan.M * plan.N, "bf16")
        assert np.array_equal(row_exchange(shard_reorder(Y, off, plan), plan), oracle.post_reorder(Y, off))


@pytest.mark.parametrize("act", ["none", "relu", "silu"])
def test_exchange_epilogue_matches_post_epilogue(act):
    plan = next(_plans(CASES[2]))
    off = element_offsets(plan)
    Y = to_bits(draw(21, (plan.M * plan.N,), ("normal", 2.0)), "bf16")
    bias = to_bits(draw(22, (len(plan.m_per_problem) * plan.N,), ("normal", 1.0)), "bf16")
    rp = row_problems(plan)
    for b in (None, bias):
        want = post_epilogue(Y, off, "bf16", act, b, rp)
        got = row_exchange_epilogue(shard_reorder(Y, off, plan), plan, "bf16", act, b, rp)
        assert np.array_equal(got, want)


def test_other_layouts_are_refused():
    plan = make_plan([64], 64, BM=32, BN=32, S=1, W=2)
    with pytest.raises(ValueError):
        gathered_rows(plan)
