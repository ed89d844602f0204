"""Pins for the oracle's end-to-end pipeline and its single-output sampler."""

import numpy as np
import pytest

import oracle
from oracle.numerics import decode_bits, round_to_dtype, encode_bits
from oracle.tiles import make_plan
from workloads import WORKLOADS, make_inputs, draw, to_bits


def _small_moe(seed=3):
    rng = np.random.Generator(np.random.PCG64(seed))
    m = [37, 0, 64, 90]
    M, N, K, D = sum(m), 48, 32, 3
    A = to_bits(draw(seed, (M, K), ("normal", 0.5)), "bf16")
    B = [to_bits(draw(seed + 10 + e, (N, K), ("normal", 0.5)), "bf16") for e in range(len(m))]
    peer = to_bits(draw(seed + 20, (M * N,), ("normal", 0.5)), "bf16")
    dest = rng.integers(0, D, size=M)
    return m, N, K, D, A, B, peer, dest


def test_tiny_workload_pipeline_definition():
    w = WORKLOADS["tiny"]
    A, B, peer, m_per, _ = make_inputs(w)
    plan = make_plan(m_per, w.N, BM=w.BM, BN=w.BN, S=w.S, W=w.W, composition=w.compositions[0])
    r = oracle.run_pipeline(A, B, peer, plan, w.dtype)
    # out[m, n] = round(round(C[m, n]) + peer[off(m, n)]) element by element
    C = decode_bits(r["C"], w.dtype)
    want = encode_bits(round_to_dtype(C + decode_bits(peer, w.dtype)[r["off"]], w.dtype), w.dtype)
    assert np.array_equal(r["out"], want)
    # C is A . B_stored^T: checked against the plain product of the decoded operands
    Cref = decode_bits(A, w.dtype) @ decode_bits(B[0], w.dtype).T
    assert np.array_equal(r["C64"], Cref)
    assert r["snapshots"] == [[4, 0, 0], [4, 4, 0], [4, 8, 0], [4, 8, 4]]
    assert r["fire_wave"] == [0, 2, 3]


def test_ternary_pipeline_is_exact_integers():
    w = WORKLOADS["tiny"]
    A, B, peer, m_per, _ = make_inputs(w, dist=("ternary",))
    plan = make_plan(m_per, w.N, BM=w.BM, BN=w.BN, S=w.S, W=w.W, composition=(1, 2, 1))
    r = oracle.run_pipeline(A, B, peer, plan, w.dtype)
    C = decode_bits(r["C"], w.dtype)
    assert np.array_equal(C, r["C64"])               # exact: |C| <= 256
    assert np.all(C == np.round(C))


@pytest.mark.parametrize("mode", ["tile", "subtile", "subtoken"])
def test_sampler_matches_full_pipeline(mode):
    if mode == "subtoken":
        m, N, K, D, A, B, peer, dest = _small_moe()
        plan = make_plan(m, N, BM=32, BN=16, S=2, W=5, mode=mode, ranks=D, row_dest=dest)
    else:
        M, N, K = 128, 96, 64
        A = to_bits(draw(1, (M, K), ("normal", 0.3)), "bf16")
        B = [to_bits(draw(2, (N, K), ("normal", 0.3)), "bf16")]
        peer = to_bits(draw(3, (M * N,), ("normal", 0.3)), "bf16")
        m = [M]
        plan = make_plan(m, N, BM=32, BN=32, S=3, W=5, mode=mode, ranks=4 if mode == "subtile" else 1)
    r = oracle.run_pipeline(A, B, peer, plan, "bf16")
    rng = np.random.Generator(np.random.PCG64(4))
    rows = rng.integers(0, plan.M, size=200)
    cols = rng.integers(0, plan.N, size=200)
    s = oracle.sample_outputs(A, B, peer, plan, "bf16", rows, cols)
    assert np.array_equal(s["off"], r["off"][rows, cols])
    assert np.array_equal(s["C"], r["C"][rows, cols])
    assert np.array_equal(s["out"], r["out"][rows, cols])
    assert np.allclose(s["C64"], r["C64"][rows, cols], rtol=0, atol=1e-12)


def test_moe_pipeline_grouped_product():
    m, N, K, D, A, B, peer, dest = _small_moe()
    plan = make_plan(m, N, BM=32, BN=16, S=2, W=5, mode="subtoken", ranks=D, row_dest=dest)
    r = oracle.run_pipeline(A, B, peer, plan, "bf16")
    Ad = decode_bits(A, "bf16")
    row = 0
    for e, me in enumerate(m):
        ref = Ad[row:row + me] @ decode_bits(B[e], "bf16").T
        assert np.array_equal(r["C64"][row:row + me], ref)
        row += me


def test_moe_workload_routing_shape():
    """Seeded top-2 routing: 8192 rows; with 256-row tiles the grid has 4144 tiles, 17 waves."""
    from workloads import moe_routing
    w = WORKLOADS["moe_a2a"]
    m_per, tok = moe_routing(w)
    assert sum(m_per) == w.tokens * w.topk
    assert np.all(np.bincount(tok, minlength=w.tokens) == w.topk)
    nt = sum(-(-x // 256) for x in m_per) * (w.N // 128)
    assert nt == 4144 and -(-nt // 256) == 17
