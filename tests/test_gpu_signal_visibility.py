"""Can the consumer read a signalled span before this pass's tile stores are visible?  Tests built to see it.

Deep-dive 一、信号机制 › 动机: 数据依赖性 -- a group may be communicated only
once its tiles are computed; 五 › 专用监控内核 -- the consumer learns of
progress only through the counters and flags.  A consumer that read a span
too early would see the previous pass's data or whatever the buffer held.
So here every pass changes the GEMM's left operand (A and -A alternate: the
same magnitudes, the opposite sign, so every element of C changes), the
reorder buffer, recv and every pass's own output start as a NaN marker, and
every pass's output is checked element by element against the oracle.  The
plans carry epoch stamps (FO_PLAN_EPOCH_STAMPS), which the consumer checks
after each signal.  Both consumers run: the gated one (a stream wait on the
flag, then a kernel over the span) and the polling one (a persistent kernel
on the CUs).

The stale-read detector itself is exercised by forcing its condition from
the host: flags raised by hand, stamps left at an old epoch; the consumer must
report FO_ERR_STALE and still finish.
"""

import numpy as np
import pytest

import oracle
from oracle.layout import element_offsets
from oracle.tiles import make_plan
from tests.gpu_util import empty16, say, to_dev, to_host, tol_check_out, zeros_i32
from tests.test_gpu_kernels import PLANS, _inputs, _rng_dest, _stack
from workloads import WORKLOADS, make_inputs, random_bits

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")
from gemm_tile_signaling_amd.pipeline import Pipeline  # noqa: E402

MARKER = int(np.uint16(0x7FC0).view(np.int16))   # a NaN in bf16 (and in fp16)


def _negate(bits):
    """-x for 16-bit floating-point patterns: flip the sign bit (exact)."""
    return np.asarray(bits, dtype=np.uint16) ^ np.uint16(0x8000)


def _stamped_plans(entry):
    name, m, N, K, dt, BM, BN, S, W, comp, mode, R = entry
    dest = _rng_dest(sum(m), R, 5) if mode == "subtoken" else None
    o = make_plan(m, N, BM=BM, BN=BN, S=S, W=W, composition=comp, mode=mode, ranks=R, row_dest=dest)
    p = fo.Plan(m, N, K, dt, BM=BM, BN=BN, swizzle=S, wave_size=W, composition=comp, mode=mode, ranks=R,
                row_dest=dest, epoch_stamps=True)
    return o, p


def _run_alternating(p, o, dA, dA_neg, dB, dpeer, n, consumer, per_group):
    """n passes, A and -A alternating, each into its own marker-filled output; returns the outputs."""
    pipe = Pipeline(p, dA, dB, dpeer, post_per_group=per_group, consumer=consumer)
    pipe.buf.fill_(MARKER)
    pipe.recv.fill_(MARKER)
    outs = [torch.full((o.M * o.N,), MARKER, dtype=torch.int16, device="cuda") for _ in range(n)]
    for i in range(n):
        pipe.A = dA if i % 2 == 0 else dA_neg
        pipe.out = outs[i]
        pipe.step()
    pipe.join()
    torch.cuda.synchronize()
    status = int(pipe.status.item())
    sig = pipe.sig.cpu().numpy()
    pipe.close()
    return outs, status, sig


SMALL = [e for e in PLANS if e[0] in ("tiny_fp16", "ragged_256", "subtile_r4", "subtoken_d4", "ragged_64")]


@pytest.mark.parametrize("entry", SMALL, ids=[e[0] for e in SMALL])
@pytest.mark.parametrize("consumer", ["gated", "poll"])
@pytest.mark.parametrize("per_group", [False, True])
def test_every_pass_sees_its_own_tiles_small(entry, consumer, per_group):
    o, p = _stamped_plans(entry)
    dt = entry[4]
    A, B, peer = _inputs(entry, seed=700)
    An = _negate(A)
    want = []
    for a in (A, An):
        r = oracle.run_pipeline(a, B, peer, o, dt)
        want.append((r["out"], r["C64"]))
    assert not np.array_equal(want[0][0], want[1][0])
    n = 6
    say(f"alternating operands {entry[0]} consumer={consumer} post per group={per_group}, {n} passes")
    outs, status, sig = _run_alternating(p, o, to_dev(A), to_dev(An), to_dev(_stack(B)), to_dev(peer), n,
                                         consumer, per_group)
    assert status == 0, fo.status_string(status)
    assert sig[:p.P].tolist() == [n * g for g in o.group_tiles]
    assert sig[p.stamp_offset:p.stamp_offset + p.NT].tolist() == [n] * p.NT
    for i in range(n):
        w_out, c64 = want[i % 2]
        tol_check_out(to_host(outs[i]).reshape(o.M, o.N), oracle.decode_bits(w_out, dt), c64, dt, f"pass {i}")


FULL = [("profiled", (1, 1)), ("ar_prefill", (1, 1, 1, 1))]
_full_cache = {}


def _full_reference(name, comp):
    """Inputs, plan and the whole fp64 product of a full-size workload (one fp64 matmul on the host)."""
    key = (name, comp)
    if key not in _full_cache:
        _full_cache.clear()
        w = WORKLOADS[name]
        A, B, peer, m_per, _ = make_inputs(w)
        o = make_plan(m_per, w.N, BM=w.BM, BN=w.BN, S=w.S, W=w.W, composition=comp)
        C64 = oracle.gemm_fp64(oracle.decode_bits(A, w.dtype), oracle.decode_bits(B[0], w.dtype).T)
        peer_at = oracle.decode_bits(peer, w.dtype)[element_offsets(o)]
        _full_cache[key] = (w, A, B, peer, m_per, o, C64, peer_at)
    return _full_cache[key]


@pytest.mark.parametrize("consumer", ["gated", "poll"])
@pytest.mark.parametrize("per_group", [True, False])
@pytest.mark.parametrize("name,comp", FULL, ids=[f"{n}-{'.'.join(map(str, c))}" for n, c in FULL])
def test_every_pass_sees_its_own_tiles_full_size(name, comp, consumer, per_group):
    """At the benchmark's shapes and schedules: four passes, A / -A / A / -A, every output element checked."""
    w, A, B, peer, m_per, o, C64, peer_at = _full_reference(name, comp)
    p = fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W, composition=comp,
                epoch_stamps=True)
    n = 4
    say(f"alternating operands {name} comp={comp} consumer={consumer} post per group={per_group}, {n} passes")
    outs, status, sig = _run_alternating(p, o, to_dev(A), to_dev(_negate(A)), to_dev(B[0]), to_dev(peer), n,
                                         consumer, per_group)
    assert status == 0, fo.status_string(status)
    assert sig[p.stamp_offset:p.stamp_offset + p.NT].tolist() == [n] * p.NT
    Cr = oracle.round_to_dtype(C64, w.dtype)
    for i in range(n):
        sgn = 1.0 if i % 2 == 0 else -1.0
        want = oracle.round_to_dtype(sgn * Cr + peer_at, w.dtype)      # out = round(C + peer[off]), C rounded
        tol_check_out(to_host(outs[i]).reshape(o.M, o.N), want, sgn * C64, w.dtype, f"pass {i}")


@pytest.mark.parametrize("consumer", ["gated", "poll"])
def test_stale_detector_reports_an_old_stamp(consumer):
    """Flags raised by hand while the stamps still hold an older epoch: the consumer reports FO_ERR_STALE,
    finishes every group, and stays silent once the stamps are current."""
    entry = [e for e in PLANS if e[0] == "ragged_128"][0]
    o, p = _stamped_plans(entry)
    dt = entry[4]
    send = random_bits(51, o.M * o.N, dt)
    peer = random_bits(52, o.M * o.N, dt)
    want = oracle.consume_add(send, peer, dt)
    dsend, dpeer = to_dev(send), to_dev(peer)
    sig = p.new_sig()
    p.flag_of(sig).fill_(2)
    p.stamps_of(sig).fill_(2)
    p.stamps_of(sig)[p.NT // 2] = 1                 # one tile still carries the previous epoch
    for stamps_ok in (False, True):
        if stamps_ok:
            p.stamps_of(sig).fill_(2)
        status = zeros_i32(1)
        recv = empty16(o.M * o.N)
        say(f"stale detector consumer={consumer} stamps current={stamps_ok}")
        if consumer == "gated":
            p.consume_group_gated(dsend, dpeer, recv, sig, 2, status)
        else:
            p.consume_group(dsend, dpeer, recv, sig, 2, status, timeout_us=200000)
        torch.cuda.synchronize()
        assert int(status.item()) == (0 if stamps_ok else fo.FO_ERR_STALE)
        assert np.array_equal(to_host(recv), want)


def test_persistent_consumer_grid_is_capped_at_the_cu_count():
    entry = PLANS[0]
    o, p = _stamped_plans(entry)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = empty16(o.M * o.N)
    sig = p.new_sig()
    p.flag_of(sig).fill_(1)
    p.stamps_of(sig).fill_(1)
    status = zeros_i32(1)
    say(f"consumer grid cap: {cus} CUs")
    with pytest.raises(fo.FoError) as e:
        p.consume_group(buf, buf, buf, sig, 1, status, num_workgroups=cus + 1)
    assert e.value.code == fo.FO_ERR_INVALID
    p.consume_group(buf, buf, buf, sig, 1, status, num_workgroups=cus)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
