"""Properties over random plans (hypothesis): the oracle's layout invariants, and the C++ planner's tables
equal to the oracle's, on shapes drawn at random rather than picked by hand (host only, no GPU).

Deep-dive 二、重排机制 › 解决方案: 映射表重排 -- the mapping table places
every tile's elements in its group's contiguous span and the inverse mapping
puts them back; 一、信号机制 › 实现方法 -- a group's threshold is its tile
count.  For every drawn plan: the element offsets are a permutation of
0..M*N-1; post(pre(x)) == x and pre(post(y)) == y; every group's elements
fill exactly its span; the thresholds sum to the tile count; and the host
planner reproduces the oracle's tables and offsets bit for bit.
"""

import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from oracle.layout import element_offsets, group_spans, post_reorder, pre_reorder  # noqa: E402
from oracle.tiles import make_plan  # noqa: E402
from tests.test_planner_vs_oracle import _assert_same  # noqa: E402

fo = pytest.importorskip("gemm_tile_signaling_amd")

TILES = [(64, 64), (128, 128), (256, 128), (256, 256)]


@st.composite
def plans(draw):
    BM, BN = draw(st.sampled_from(TILES))
    mode = draw(st.sampled_from(["tile", "subtile", "subtoken"]))
    problems = draw(st.integers(1, 3)) if mode == "subtoken" else 1
    if mode == "subtile":        # the ReduceScatter layout takes whole tiles only
        m = [draw(st.integers(1, 4)) * BM]
        N = draw(st.integers(1, 4)) * BN
    else:
        m = [draw(st.integers(0 if problems > 1 else 1, 600)) for _ in range(problems)]
        if sum(m) == 0:
            m[0] = 1
        N = draw(st.integers(1, 700 // 8)) * 8
    S = draw(st.integers(1, 5))
    W = draw(st.integers(1, 12))
    ranks = 1
    row_dest = None
    if mode == "subtile":
        ranks = draw(st.sampled_from([2, 4, 8]))
    elif mode == "subtoken":
        ranks = draw(st.sampled_from([2, 4, 8]))
        seed = draw(st.integers(0, 2 ** 16))
        row_dest = np.random.Generator(np.random.PCG64(seed)).integers(0, ranks, size=sum(m)).astype(np.int32)
    base = make_plan(m, N, BM=BM, BN=BN, S=S, W=W, mode=mode, ranks=ranks, row_dest=row_dest)
    # a random composition of the T waves: a cut after wave i or not, for each of the T-1 boundaries
    cuts = draw(st.lists(st.booleans(), min_size=base.T - 1, max_size=base.T - 1))
    comp, run = [], 1
    for cut in cuts:
        if cut:
            comp.append(run)
            run = 0
        run += 1
    comp = tuple(comp + [run])
    return dict(m=m, N=N, BM=BM, BN=BN, S=S, W=W, comp=comp, mode=mode, ranks=ranks, row_dest=row_dest)


def _oracle_plan(c):
    return make_plan(c["m"], c["N"], BM=c["BM"], BN=c["BN"], S=c["S"], W=c["W"], composition=c["comp"],
                     mode=c["mode"], ranks=c["ranks"], row_dest=c["row_dest"])


@settings(max_examples=200, deadline=None, derandomize=True, database=None)
@given(plans())
def test_layout_invariants_on_random_plans(c):
    o = _oracle_plan(c)
    off = element_offsets(o)                                           # [M, N]
    mn = o.M * o.N
    assert np.array_equal(np.sort(off.ravel()), np.arange(mn))          # a bijection onto the buffer
    rng = np.random.Generator(np.random.PCG64(1))
    X = rng.integers(0, 1 << 16, size=(o.M, o.N), dtype=np.uint32).astype(np.uint16)
    y = rng.integers(0, 1 << 16, size=mn, dtype=np.uint32).astype(np.uint16)
    assert np.array_equal(post_reorder(pre_reorder(X, off), off), X)
    assert np.array_equal(pre_reorder(post_reorder(y, off), off), y)
    assert sum(o.group_tiles) == o.NT                                  # thresholds count every tile once
    spans = group_spans(o)
    grp = np.array(o.group_of_b)
    for j in range(o.P):                                               # a group's tiles fill its span
        elems = sum(o.tile_rows[o.tile_of_b[b]] * o.tile_cols[o.tile_of_b[b]] for b in np.flatnonzero(grp == j))
        assert spans[j + 1] - spans[j] == elems


@settings(max_examples=200, deadline=None, derandomize=True, database=None)
@given(plans())
def test_planner_equals_oracle_on_random_plans(c):
    o = _oracle_plan(c)
    p = fo.Plan(c["m"], c["N"], 64, "bf16", BM=c["BM"], BN=c["BN"], swizzle=c["S"], wave_size=c["W"],
                composition=c["comp"], mode=c["mode"], ranks=c["ranks"], row_dest=c["row_dest"], host_only=True)
    try:
        _assert_same(o, p)
    finally:
        p.close()
