"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

For every workload: two passes of the whole path; the counting table and
flags exact; the final output and the GEMM output at sampled elements
(random plus edge rows and columns) within 1e-2 * max(1, |oracle|), each
sampled element computed by the oracle as one fp64 dot product; the
signaling GEMM's reordered buffer, reordered back, bit-identical to the
plain GEMM; and both reorders bit-exact on seeded random patterns (full
offset maps where they fit, sampled offsets for the MoE shape).
"""

import numpy as np
import pytest

import oracle
from oracle.layout import element_offsets, row_offsets
from oracle.pipeline import offset_of
from oracle.tiles import make_plan
from tests.gpu_util import empty16, say, to_dev, to_host, tol_check, tol_check_out
from workloads import WORKLOADS, make_inputs, random_bits

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")
from gemm_tile_signaling_amd.pipeline import Pipeline  # noqa: E402

# (workload, partition, post-reorder group by group) -- the benchmark's schedules among them
CASES = [
    ("profiled", (2,), False), ("profiled", (1, 1), False), ("profiled", (1, 1), True),
    ("ar_prefill", (1, 1, 1, 1), True), ("ar_prefill", (2, 2), False), ("ar_prefill", (1, 3), False),
    ("ar_decode", (1,), False),
    ("rs", (1, 1, 1, 1), False), ("rs", (1, 2, 1), True),
    ("moe_a2a", (4, 4, 4, 5), True), ("moe_a2a", (1,) * 17, False),
]

_cache = {}


def _inputs(name):
    if name not in _cache:
        _cache.clear()
        w = WORKLOADS[name]
        _cache[name] = (w,) + make_inputs(w)
    return _cache[name]


def _samples(o, seed, n=3000):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = list(rng.integers(0, o.M, size=n))
    cols = list(rng.integers(0, o.N, size=n))
    # edge rows: the first and last row of every problem, against the first and last columns
    start = 0
    for m in o.m_per_problem:
        if m:
            for r in (start, start + m - 1):
                for c in (0, o.N - 1, o.N // 2):
                    rows.append(r)
                    cols.append(c)
        start += m
    return np.array(rows), np.array(cols)


@pytest.mark.parametrize("name,comp,per_group", CASES,
                         ids=[f"{n}-{'.'.join(map(str, c))}{'-pg' if g else ''}" for n, c, g in CASES])
def test_workload_full_size(name, comp, per_group):
    w, A, B, peer, m_per, row_dest = _inputs(name)
    o = make_plan(m_per, w.N, BM=w.BM, BN=w.BN, S=w.S, W=w.W, composition=comp, mode=w.mode, ranks=w.ranks,
                  row_dest=row_dest)
    p = fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W, composition=comp,
                mode=w.mode, ranks=w.ranks, row_dest=row_dest)
    assert (p.NT, p.T, p.P) == (o.NT, o.T, o.P)
    rows, cols = _samples(o, 1)
    s = oracle.sample_outputs(A, B, peer, o, w.dtype, rows, cols)
    say(f"workload {name} comp={comp} post per group={per_group} M={o.M} N={o.N} K={w.K} NT={o.NT} T={o.T}")
    dA, dB, dpeer = to_dev(A), to_dev(np.concatenate([b.reshape(-1) for b in B])), to_dev(peer)
    pipe = Pipeline(p, dA, dB, dpeer, post_per_group=per_group)
    pipe.step()
    pipe.step()
    pipe.join()
    torch.cuda.synchronize()
    assert int(pipe.status.item()) == 0
    sg = pipe.sig.cpu().numpy()
    assert sg[:p.P].tolist() == [2 * g for g in o.group_tiles]
    assert sg[p.flag_offset:p.flag_offset + p.P].tolist() == [2] * p.P
    out = to_host(pipe.out).reshape(o.M, o.N)
    want_out = oracle.decode_bits(s["out"], w.dtype)
    tol_check_out(out[rows, cols], want_out, s["C64"], w.dtype, "out (sampled)")
    # GEMM output: plain row-major GEMM, and the signaling GEMM's buffer reordered back
    C = empty16(o.M * o.N)
    back = empty16(o.M * o.N)
    p.gemm_plain(dA, dB, C)
    p.reorder_post(pipe.buf, back)
    torch.cuda.synchronize()
    Ch = to_host(C).reshape(o.M, o.N)
    ratio = tol_check(Ch[rows, cols], s["C64"], w.dtype, "C (sampled)")
    assert ratio < 0.05, ratio
    assert np.array_equal(to_host(back).reshape(o.M, o.N), Ch)


@pytest.mark.parametrize("name", ["profiled", "ar_prefill", "ar_decode", "rs", "moe_a2a"])
def test_workload_reorders_bit_exact(name):
    w = WORKLOADS[name]
    if w.experts:
        from workloads import moe_routing
        m_per, tok = moe_routing(w)
        row_dest = tok // (w.tokens // w.ranks)
    else:
        m_per, row_dest = [w.M], None
    o = make_plan(m_per, w.N, BM=w.BM, BN=w.BN, S=w.S, W=w.W, mode=w.mode, ranks=w.ranks, row_dest=row_dest)
    p = fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W, mode=w.mode,
                ranks=w.ranks, row_dest=row_dest)
    n = o.M * o.N
    X = random_bits(91, n, w.dtype)
    say(f"reorders {name} M={o.M} N={o.N}")
    dX = to_dev(X)
    pre, post = empty16(n), empty16(n)
    p.reorder_pre(dX, pre)
    p.reorder_post(dX, post)
    torch.cuda.synchronize()
    got_pre, got_post = to_host(pre), to_host(post)
    if n <= 64 * 2 ** 20:
        off = element_offsets(o)
        assert np.array_equal(got_pre, oracle.pre_reorder(X.reshape(o.M, o.N), off))
        assert np.array_equal(got_post, oracle.post_reorder(X, off).ravel())
    else:
        rows, cols = _samples(o, 2, n=20000)
        ro = row_offsets(o)
        slot_of_tile, _ = oracle.mapping_table(o)
        offs = np.array([offset_of(o, ro, slot_of_tile, int(m), int(c)) for m, c in zip(rows, cols)])
        assert np.array_equal(got_post.reshape(o.M, o.N)[rows, cols], X[offs])
        assert np.array_equal(got_pre[offs], X.reshape(o.M, o.N)[rows, cols])
        # every element moved: pre and post are inverse permutations
        assert np.array_equal(np.sort(got_pre), np.sort(X))
