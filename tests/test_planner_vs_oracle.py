"""The C++ planner's tables equal the oracle's, bit for bit (host-only plans, no GPU).

The planner is host code inside libfo; FO_PLAN_HOST_ONLY builds its tables
without touching a device.  ``fo_plan_offsets`` evaluates the same per-slot
records and row-offset function the kernels use, so equality with the
oracle's element offsets covers the layout the GPU writes.
"""

import numpy as np
import pytest

import oracle
from oracle.layout import consumer_units, element_offsets, group_spans
from oracle.tiles import make_plan

fo = pytest.importorskip("gemm_tile_signaling_amd")


def _both(m, N, K=64, dtype="bf16", BM=64, BN=64, S=2, W=4, comp=None, mode="tile", ranks=1, row_dest=None,
          dispatch_order=None):
    o = make_plan(m, N, BM=BM, BN=BN, S=S, W=W, composition=comp, mode=mode, ranks=ranks, row_dest=row_dest,
                  dispatch_order=dispatch_order)
    p = fo.Plan(m, N, K, dtype, BM=BM, BN=BN, swizzle=S, wave_size=W, composition=comp, mode=mode, ranks=ranks,
                row_dest=row_dest, dispatch_order=dispatch_order, host_only=True)
    return o, p


def _assert_same(o, p):
    assert (p.NT, p.T, p.P, p.M) == (o.NT, o.T, o.P, o.M)
    t = p.tables()
    slot_of_tile, tile_of_slot = oracle.mapping_table(o)
    assert t["tile_of_slot"].tolist() == tile_of_slot
    assert t["slot_of_tile"].tolist() == slot_of_tile
    assert t["group_of_slot"].tolist() == o.group_of_b
    assert t["group_tiles"].tolist() == o.group_tiles
    assert t["span_off"].tolist() == group_spans(o)
    uo, gu = p.units()
    units = consumer_units(o)
    flat = [u for g in units for u in g]
    assert uo.tolist() == [u[0] for u in flat] + [flat[-1][1] if flat else 0]
    assert gu.tolist() == [0] + list(np.cumsum([len(g) for g in units]))
    # each group's units tile its span back to back (the consumer streams the span in one pass)
    span = t["span_off"].tolist()
    assert np.all(np.diff(uo) >= 0)
    for g in range(p.P):
        assert uo[gu[g]] == span[g] and uo[gu[g + 1]] == span[g + 1]
    assert np.array_equal(p.offsets(), element_offsets(o))


def test_pages_worked_examples():
    # counting-table example: 8 tiles (2 x 4 grid, identity order), 2 tiles per wave, groups (1, 2, 1)
    o, p = _both(128, 256, BM=64, BN=64, S=1, W=2, comp=(1, 2, 1))
    _assert_same(o, p)
    assert p.tables()["group_tiles"].tolist() == [2, 4, 2]
    # mapping example: execution order [t0, t3, t1, t2] on a 2 x 2 grid
    o, p = _both(128, 128, BM=64, BN=64, S=1, W=4, dispatch_order=[0, 3, 1, 2])
    _assert_same(o, p)
    assert p.tables()["slot_of_tile"].tolist() == [0, 2, 3, 1]


def test_tiny_workload_tables():
    o, p = _both(256, 256, K=256, dtype="fp16", BM=64, BN=64, S=2, W=4, comp=(1, 2, 1))
    _assert_same(o, p)
    assert p.tables()["tile_of_slot"].tolist() == [0, 4, 1, 5, 2, 6, 3, 7, 8, 12, 9, 13, 10, 14, 11, 15]


@pytest.mark.parametrize("m,N,BM,BN,S,W", [
    (256, 256, 64, 64, 2, 4), (250, 200, 64, 64, 3, 5), (1000, 264, 128, 128, 3, 7), (513, 384, 256, 128, 4, 3),
    (64, 64, 64, 64, 1, 1), (2048, 8192, 256, 128, 4, 256), (128, 8192, 64, 64, 1, 256),
])
def test_tile_mode_all_partitions(m, N, BM, BN, S, W):
    base = make_plan(m, N, BM=BM, BN=BN, S=S, W=W)
    comps = oracle.enumerate_compositions(base.T)
    for comp in comps[:: max(1, len(comps) // 16)]:
        o, p = _both(m, N, BM=BM, BN=BN, S=S, W=W, comp=comp)
        _assert_same(o, p)


@pytest.mark.parametrize("R,BM", [(4, 256), (2, 128), (4, 64), (8, 64)])
def test_subtile_mode(R, BM):
    BN = 128 if BM >= 128 else 64
    m, N = 4 * BM, 3 * BN
    base = make_plan(m, N, BM=BM, BN=BN, S=3, W=5, mode="subtile", ranks=R)
    for comp in oracle.enumerate_compositions(base.T):
        o, p = _both(m, N, BM=BM, BN=BN, S=3, W=5, comp=comp, mode="subtile", ranks=R)
        _assert_same(o, p)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_subtoken_mode_ragged_experts(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    m = [int(x) for x in rng.integers(0, 300, size=5)]
    m[2] = 0
    D = 4
    dest = rng.integers(0, D, size=sum(m))
    base = make_plan(m, 192, BM=128, BN=128, S=2, W=3, mode="subtoken", ranks=D, row_dest=dest)
    comps = oracle.enumerate_compositions(base.T)
    for comp in comps[:: max(1, len(comps) // 8)]:
        o, p = _both(m, 192, BM=128, BN=128, S=2, W=3, comp=comp, mode="subtoken", ranks=D, row_dest=dest)
        _assert_same(o, p)


def test_moe_workload_tables():
    """Seeded top-2 routing of 4096 tokens over 8 experts, D = 8 destinations."""
    from workloads import WORKLOADS, moe_routing
    w = WORKLOADS["moe_a2a"]
    m_per, tok = moe_routing(w)
    dest = tok // (w.tokens // w.ranks)
    # full element-offset check on a narrower N (8 tile columns) so the oracle's map stays small
    base = make_plan(m_per, 1024, BM=256, BN=128, S=4, W=32)
    for comp in [None, (base.T,), (3,) * (base.T // 3) + ((base.T % 3,) if base.T % 3 else ())]:
        o, p = _both(m_per, 1024, K=w.K, BM=256, BN=128, S=4, W=32, comp=comp, mode="subtoken", ranks=8,
                     row_dest=dest)
        _assert_same(o, p)
    # the workload's own shape: tables only
    o, p = _both(m_per, w.N, K=w.K, BM=256, BN=128, S=4, W=256, comp=(4, 4, 4, 5), mode="subtoken", ranks=8,
                 row_dest=dest)
    assert p.NT == 4144 and p.T == 17
    t = p.tables()
    assert t["group_tiles"].tolist() == o.group_tiles
    assert t["span_off"].tolist() == group_spans(o)
    assert t["tile_of_slot"].tolist() == o.tile_of_b


def test_empty_problem():
    o, p = _both(0, 64, BM=64, BN=64, S=1, W=4, comp=())
    assert p.NT == 0 and p.T == 0 and p.P == 0
    assert p.offsets().shape == (0, 64)
