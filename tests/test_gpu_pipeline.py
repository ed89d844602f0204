"""GPU parity of the whole path (signaling GEMM on stream A, consumer and
post-reorder on stream B) against the oracle's pipeline, small shapes.

Real-valued inputs: the final row-major output within 1e-2 * max(1, |oracle|).
Ternary inputs: bit-exact.  Several passes back to back with increasing epochs.
"""

import numpy as np
import pytest

import oracle
from oracle.tiles import make_plan
from tests.gpu_util import say, to_dev, to_host, tol_check_out
from tests.test_gpu_kernels import PLANS, _inputs, _plans, _stack

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")
from gemm_tile_signaling_amd.pipeline import Pipeline  # noqa: E402


@pytest.mark.parametrize("entry", PLANS, ids=[e[0] for e in PLANS])
@pytest.mark.parametrize("in_place", [False, True])
def test_pipeline_matches_oracle(entry, in_place):
    o, p = _plans(entry)
    dt = entry[4]
    A, B, peer = _inputs(entry, seed=500)
    r = oracle.run_pipeline(A, B, peer, o, dt)
    C = oracle.decode_bits(r["C"], dt)
    want_out = oracle.round_to_dtype(C + oracle.decode_bits(peer, dt)[r["off"]], dt)   # definition, row-major
    say(f"pipeline {entry[0]} in_place={in_place}")
    pipe = Pipeline(p, to_dev(A), to_dev(_stack(B)), to_dev(peer), in_place=in_place)
    for _ in range(3):
        pipe.step()
    pipe.join()
    torch.cuda.synchronize()
    assert int(pipe.status.item()) == 0
    s = pipe.sig.cpu().numpy()
    assert s[:p.P].tolist() == [3 * g for g in o.group_tiles]
    assert s[p.flag_offset:p.flag_offset + p.P].tolist() == [3] * p.P
    out = to_host(pipe.out).reshape(o.M, o.N)
    tol_check_out(out, want_out, r["C64"], dt, "out")
    # the oracle's own end-to-end result agrees with its definition
    assert np.array_equal(r["out"], oracle.encode_bits(want_out, dt))


@pytest.mark.parametrize("entry", [e for e in PLANS if e[3] <= 256], ids=[e[0] for e in PLANS if e[3] <= 256])
def test_pipeline_ternary_bit_exact(entry):
    o, p = _plans(entry)
    dt = entry[4]
    A, B, peer = _inputs(entry, dist=("ternary",), seed=600)
    r = oracle.run_pipeline(A, B, peer, o, dt)
    say(f"pipeline ternary {entry[0]}")
    pipe = Pipeline(p, to_dev(A), to_dev(_stack(B)), to_dev(peer))
    pipe.step()
    pipe.step()
    pipe.join()
    torch.cuda.synchronize()
    assert int(pipe.status.item()) == 0
    assert np.array_equal(to_host(pipe.recv), r["recv"])
    assert np.array_equal(to_host(pipe.out), r["out"].ravel())


@pytest.mark.parametrize("comp", [(1, 1, 1, 1), (1, 2, 1), (2, 2), (4,), (3, 1), (1, 3)])
def test_tiny_workload_every_partition_kind(comp):
    """The fp16 worked-example-sized GEMM under several wave-group partitions."""
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["tiny"]
    A, B, peer, m_per, _ = make_inputs(w)
    o = make_plan(m_per, w.N, BM=w.BM, BN=w.BN, S=w.S, W=w.W, composition=comp)
    p = fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W, composition=comp)
    r = oracle.run_pipeline(A, B, peer, o, w.dtype)
    say(f"tiny partition {comp}")
    pipe = Pipeline(p, to_dev(A), to_dev(B[0]), to_dev(peer))
    pipe.step()
    pipe.join()
    torch.cuda.synchronize()
    assert int(pipe.status.item()) == 0
    assert pipe.sig.cpu().numpy()[:p.P].tolist() == o.group_tiles
    want = oracle.round_to_dtype(oracle.decode_bits(r["C"], w.dtype) + oracle.decode_bits(peer, w.dtype)[r["off"]],
                                 w.dtype)
    tol_check_out(to_host(pipe.out).reshape(o.M, o.N), want, r["C64"], w.dtype, "out")


@pytest.mark.parametrize("entry", [e for e in PLANS if e[3] <= 256], ids=[e[0] for e in PLANS if e[3] <= 256])
def test_serial_passes_between_overlapped_ones(entry):
    """Passes without overlap (all three kernels on one queue) interleaved with
    overlapped ones: every pass is bit-exact against the oracle and the counting
    table keeps counting epochs."""
    o, p = _plans(entry)
    dt = entry[4]
    A, B, peer = _inputs(entry, dist=("ternary",), seed=610)
    r = oracle.run_pipeline(A, B, peer, o, dt)
    say(f"pipeline serial/overlapped {entry[0]}")
    pipe = Pipeline(p, to_dev(A), to_dev(_stack(B)), to_dev(peer))
    for serial in (True, False, True, True, False):
        pipe.step(serial=serial)
    pipe.join()
    torch.cuda.synchronize()
    assert int(pipe.status.item()) == 0
    s = pipe.sig.cpu().numpy()
    assert s[:p.P].tolist() == [5 * g for g in o.group_tiles]
    assert s[p.flag_offset:p.flag_offset + p.P].tolist() == [5] * p.P
    assert np.array_equal(to_host(pipe.out), r["out"].ravel())


@pytest.mark.parametrize("entry", [e for e in PLANS if e[0] in ("ragged_256", "subtile_r4", "tiny_fp16")],
                         ids=lambda e: e[0])
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("per_group", [False, True])
def test_back_to_back_passes_keep_recv_ordered(entry, in_place, per_group):
    """Consecutive passes alternate between two peer buffers and write separate
    outputs, so a consumer that rewrote recv before the previous pass's
    post-reorder had read it would leave the other peer's sums in an output.
    Every output is checked bit-exactly (ternary inputs) against the oracle,
    with the post-reorder over the whole output or group by group."""
    o, p = _plans(entry)
    dt = entry[4]
    A, B, peer0 = _inputs(entry, dist=("ternary",), seed=620)
    peer1 = _inputs(entry, dist=("ternary",), seed=640)[2]
    want = [oracle.run_pipeline(A, B, pr, o, dt)["out"].ravel() for pr in (peer0, peer1)]
    assert not np.array_equal(want[0], want[1])
    n = 40
    say(f"pipeline back-to-back {entry[0]}, {n} passes, in_place={in_place}, post per group={per_group}")
    peers = [to_dev(peer0), to_dev(peer1)]
    pipe = Pipeline(p, to_dev(A), to_dev(_stack(B)), peers[0], in_place=in_place, post_per_group=per_group)
    outs = [torch.empty(o.M * o.N, dtype=torch.int16, device="cuda") for _ in range(n)]
    for i in range(n):
        pipe.peer = peers[i % 2]
        pipe.out = outs[i]
        pipe.step()
    pipe.join()
    torch.cuda.synchronize()
    assert int(pipe.status.item()) == 0
    assert pipe.sig.cpu().numpy()[:p.P].tolist() == [n * g for g in o.group_tiles]
    for i in range(n):
        assert np.array_equal(to_host(outs[i]), want[i % 2]), f"pass {i}"
