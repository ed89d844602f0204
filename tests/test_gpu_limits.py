"""Edge cases of size: an empty problem, and the largest output the plan accepts.

M * N = 2^30 elements (2 GiB per buffer) is the planner's limit: the consumer
and the reorders address each buffer with 32-bit byte offsets.  At that size
the oracle cannot build the whole offset map, so the checks are element by
element at sampled positions (the oracle's fp64 dot product and its reordered
offset of each sampled element), plus properties that hold at any size: the
final counting table, every flag raised, and post(pre(x)) == x.
"""

import numpy as np
import pytest

import oracle
from oracle.layout import row_offsets
from oracle.pipeline import offset_of
from oracle.tiles import make_plan
from tests.gpu_util import say, to_dev, tol_check, tol_check_out
from workloads import draw, to_bits

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")


def test_empty_problem_is_a_no_op():
    p = fo.Plan([0], 256, 64, "bf16", BM=256, BN=128, swizzle=4, wave_size=256)
    assert (p.NT, p.T, p.P, p.sig_words) == (0, 0, 0, 0)
    say("empty problem: every entry point returns without work")
    A = torch.zeros(64, dtype=torch.int16, device="cuda")
    B = torch.zeros(256 * 64, dtype=torch.int16, device="cuda")
    x = torch.full((16,), 7, dtype=torch.int16, device="cuda")
    sig = p.new_sig()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    p.gemm_signal(A, B, x, sig, 1)
    p.gemm_plain(A, B, x)
    p.consume_group(x, x, x, sig, 1, status)
    p.reorder_post(x, x)
    p.reorder_pre(x, x)
    p.reorder_post_ep(x, x, act="silu")
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert x.cpu().tolist() == [7] * 16
    assert p.search(1e-3, [1.0], [1e-6]) == ((), 0.0, None)


def test_largest_output_end_to_end():
    M, N, K = 2 ** 15, 2 ** 15, 64                          # M * N = 2^30
    dt = "bf16"
    o = make_plan([M], N, BM=256, BN=128, S=4, W=256)
    p = fo.Plan([M], N, K, dt, BM=256, BN=128, swizzle=4, wave_size=256)
    assert p.M * p.N == 2 ** 30 and (p.NT, p.T, p.P) == (o.NT, o.T, o.P) == (32768, 128, 128)
    A = to_bits(draw(71, (M, K), ("normal", 0.5)), dt)
    B = to_bits(draw(72, (N, K), ("normal", 0.5)), dt)
    rng = np.random.Generator(np.random.PCG64(73))
    rows = np.concatenate([rng.integers(0, M, 3000), [0, M - 1, M - 1, 0]])
    cols = np.concatenate([rng.integers(0, N, 3000), [0, N - 1, 0, N - 1]])
    ro = row_offsets(o)
    slot_of_tile, _ = oracle.mapping_table(o)
    offs = np.array([offset_of(o, ro, slot_of_tile, int(m), int(n)) for m, n in zip(rows, cols)])
    c64 = np.array([float(np.dot(oracle.decode_bits(A[m], dt), oracle.decode_bits(B[n], dt)))
                    for m, n in zip(rows, cols)])
    one = to_bits(np.array([1.0]), dt)[0]
    want_out = oracle.decode_bits(oracle.consume_add(oracle.encode_bits(oracle.round_to_dtype(c64, dt), dt),
                                                     np.full(c64.size, one, np.uint16), dt), dt)

    say(f"largest output: M={M} N={N} K={K} NT={p.NT} T={p.T} P={p.P} (2 GiB per buffer)")
    n = M * N
    dA, dB = to_dev(A).reshape(-1), to_dev(B).reshape(-1)
    buf = torch.empty(n, dtype=torch.int16, device="cuda")
    sig = p.new_sig()
    p.gemm_signal(dA, dB, buf, sig, 1)
    peer = torch.full((n,), int(np.uint16(one).view(np.int16)), dtype=torch.int16, device="cuda")
    recv = torch.empty_like(buf)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    p.consume_group(buf, peer, recv, sig, 1, status)
    del peer
    out = torch.empty_like(buf)
    p.reorder_post(recv, out)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    s = sig.cpu().numpy()
    assert s[:p.P].tolist() == o.group_tiles and s[p.flag_offset:p.flag_offset + p.P].tolist() == [1] * p.P

    ti = torch.from_numpy(offs).cuda()
    tr, tc = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    got_buf = buf[ti].cpu().numpy().view(np.uint16)
    got_out = out.view(M, N)[tr, tc].cpu().numpy().view(np.uint16)
    tol_check(got_buf, c64, dt, "reorder buffer at sampled offsets")
    tol_check_out(got_out, want_out, c64, dt, "out at sampled elements")

    say("largest output: round trip post(pre(x)) == x")
    pre = torch.empty_like(buf)
    p.reorder_pre(out, pre)
    torch.cuda.synchronize()
    assert torch.equal(pre, recv)
