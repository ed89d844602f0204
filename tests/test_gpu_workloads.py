"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

For every workload: two passes of the whole path; the counting table and
flags exact; the final output and the GEMM output at sampled elements within
1e-2 * max(1, |oracle|), each sampled element computed by the oracle as one
fp64 dot product.  The samples are stratified: at least 8 random elements
inside every tile, plus the first and last row of every problem.  For the
profiled and the prefill shapes the whole GEMM output is also checked
against the oracle's fp64 product.  The signaling GEMM's reordered buffer,
reordered back, is bit-identical to the plain GEMM; both reorders are
bit-exact on seeded random patterns (full offset maps where they fit,
sampled offsets for the MoE shape); on the ReduceScatter workload the rank
shards and the row exchange are bit-exact against the oracle applied to the
GPU's own consumer output.
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

# (workload, partition, post-reorder group by group, consumer) -- the benchmark's schedules among them
CASES = [
    ("profiled", (2,), False, "poll"), ("profiled", (1, 1), False, "gated"), ("profiled", (1, 1), True, "gated"),
    ("profiled", (1, 1), True, "poll"),
    ("ar_prefill", (1, 1, 1, 1), True, "gated"), ("ar_prefill", (1, 1, 1, 1), True, "poll"),
    ("ar_prefill", (2, 2), False, "poll"), ("ar_prefill", (1, 3), False, "gated"),
    ("ar_decode", (1,), False, "gated"), ("ar_decode", (1,), False, "poll"),
    ("rs", (1, 1, 1, 1), False, "poll"), ("rs", (1, 1, 1, 1), True, "poll"), ("rs", (1, 2, 1), True, "gated"),
    ("moe_a2a", (4, 4, 4, 5), True, "gated"), ("moe_a2a", (1,) * 17, False, "poll"),
    ("moe_a2a", (1,) * 17, True, "poll"),
]

_cache = {}


def _inputs(name):
    if name not in _cache:
        _cache.clear()
        w = WORKLOADS[name]
        _cache[name] = (w,) + make_inputs(w)
    return _cache[name]


def _samples(o, seed, per_tile=8):
    """At least `per_tile` random elements inside every tile, and the first and last row of every problem
    against the first, middle and last column."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows, cols = [], []
    for t in range(o.NT):
        rows.append(o.tile_row0[t] + rng.integers(0, o.tile_rows[t], size=per_tile))
        cols.append(o.tile_col0[t] + rng.integers(0, o.tile_cols[t], size=per_tile))
    rows, cols = list(np.concatenate(rows)), list(np.concatenate(cols))
    start = 0
    for m in o.m_per_problem:
        if m:
            for r in (start, start + m - 1):
                for c in (0, o.N - 1, o.N // 2):
                    rows.append(r)
                    cols.append(c)
        start += m
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


_full_c = {}


def _full_product(name, w, A, B):
    """The whole fp64 product for the workloads small enough to form it on the host."""
    if name not in _full_c:
        _full_c.clear()
        _full_c[name] = oracle.gemm_fp64(oracle.decode_bits(A, w.dtype), oracle.decode_bits(B[0], w.dtype).T)
    return _full_c[name]


@pytest.mark.parametrize("name,comp,per_group,consumer", CASES,
                         ids=[f"{n}-{'.'.join(map(str, c))}{'-pg' if g else ''}-{k}" for n, c, g, k in CASES])
def test_workload_full_size(name, comp, per_group, consumer):
    w, A, B, peer, m_per, row_dest = _inputs(name)
    o = make_plan(m_per, w.N, BM=w.BM, BN=w.BN, S=w.S, W=w.W, composition=comp, mode=w.mode, ranks=w.ranks,
                  row_dest=row_dest)
    p = fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W, composition=comp,
                mode=w.mode, ranks=w.ranks, row_dest=row_dest)
    assert (p.NT, p.T, p.P) == (o.NT, o.T, o.P)
    rows, cols = _samples(o, 1)
    s = oracle.sample_outputs(A, B, peer, o, w.dtype, rows, cols)
    say(f"workload {name} comp={comp} post per group={per_group} consumer={consumer} M={o.M} N={o.N} K={w.K} "
        f"NT={o.NT} T={o.T} samples={rows.size}")
    dA, dB, dpeer = to_dev(A), to_dev(np.concatenate([b.reshape(-1) for b in B])), to_dev(peer)
    pipe = Pipeline(p, dA, dB, dpeer, post_per_group=per_group, consumer=consumer)
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
    if name in ("profiled", "ar_prefill"):
        ratio = tol_check(Ch, _full_product(name, w, A, B), w.dtype, "C (every element)")
        assert ratio < 0.05, ratio
    if w.mode == "subtile":
        # ReduceScatter + AllGather: rank shards, then the block-cyclic row exchange (with and without an
        # epilogue), against the oracle applied to the GPU's own consumer output
        from oracle.epilogue import row_problems
        from oracle.rowexchange import row_exchange_epilogue, shard_reorder
        recv = to_host(pipe.recv)
        off = element_offsets(o)
        want_g = shard_reorder(recv, off, o)
        g, ex = empty16(o.M * o.N), empty16(o.M * o.N)
        p.reorder_shards(pipe.recv, g)
        p.row_exchange(g, ex)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(g), want_g)
        assert np.array_equal(to_host(ex).reshape(o.M, o.N), out)
        bias = random_bits(93, o.N, w.dtype)
        p.row_exchange(g, ex, bias=to_dev(bias), act="relu")
        torch.cuda.synchronize()
        assert np.array_equal(to_host(ex).reshape(o.M, o.N),
                              row_exchange_epilogue(want_g, o, w.dtype, "relu", bias, row_problems(o)))


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
        rows, cols = _samples(o, 2, per_tile=5)
        ro = row_offsets(o)
        slot_of_tile, _ = oracle.mapping_table(o)
        offs = np.array([offset_of(o, ro, slot_of_tile, int(m), int(c)) for m, c in zip(rows, cols)])
        assert np.array_equal(got_post.reshape(o.M, o.N)[rows, cols], X[offs])
        assert np.array_equal(got_pre[offs], X.reshape(o.M, o.N)[rows, cols])
        # every element moved: pre and post are inverse permutations
        assert np.array_equal(np.sort(got_pre), np.sort(X))
