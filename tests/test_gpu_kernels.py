"""GPU parity of each kernel against the oracle, on seeded inputs spanning several tiles and ragged edges.

Bit-exact: both reorders, the consumer's add, the counting table, flags,
tickets and fire counts, and the GEMM on ternary inputs (exact integers).
Within |gpu - oracle| <= 1e-2 * max(1, |oracle|): the GEMM on real-valued
inputs.  All calls go through the C ABI (the ctypes binding).
"""

import numpy as np
import pytest

import oracle
from oracle.layout import element_offsets, group_spans
from oracle.tiles import make_plan
from oracle.epilogue import post_epilogue, row_problems
from tests.gpu_util import empty16, say, to_dev, to_host, tol_check, tol_check_out, ulp_distance, zeros_i32
from workloads import draw, random_bits, to_bits

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")


def _rng_dest(M, D, seed):
    return np.random.Generator(np.random.PCG64(seed)).integers(0, D, size=M)


# (name, m_per_problem, N, K, dtype, BM, BN, S, W, composition, mode, ranks)
PLANS = [
    ("tiny_fp16", [256], 256, 256, "fp16", 64, 64, 2, 4, (1, 2, 1), "tile", 1),
    ("ragged_64", [250], 200, 128, "bf16", 64, 64, 3, 5, None, "tile", 1),
    ("ragged_128", [1000], 264, 192, "bf16", 128, 128, 3, 7, None, "tile", 1),
    ("ragged_256", [513], 384, 320, "bf16", 256, 128, 4, 3, (1, 1, 1), "tile", 1),
    ("subtile_r4", [1024], 256, 128, "bf16", 256, 128, 2, 3, None, "subtile", 4),
    ("subtile_r2_fp16", [256], 192, 64, "fp16", 64, 64, 2, 4, (2, 1), "subtile", 2),
    ("subtoken_d4", [70, 0, 130, 64], 192, 128, "bf16", 128, 128, 2, 3, None, "subtoken", 4),
    ("subtoken_d8_256", [300, 257, 1], 256, 64, "bf16", 256, 128, 1, 2, None, "subtoken", 8),
    ("fp16_256x128", [300, 200], 256, 192, "fp16", 256, 128, 1, 3, (1, 1), "tile", 1),
    ("ragged_rows_cols_256x128", [300], 200, 128, "bf16", 256, 128, 2, 2, None, "tile", 1),
    # 256 x 128 tiles whose 64-row or 64-column wave bands lie wholly past the edge (1, 3 and 1 of 4 row
    # bands hold rows; the last column tile has one of its two column bands): those waves skip their MFMAs
    ("empty_bands_256x128", [40, 130, 300], 320, 192, "bf16", 256, 128, 2, 5, None, "tile", 1),
    # 256 x 256 tiles (K-slices of 32): ragged rows and columns, rank bands, fp16
    ("ragged_256x256", [600], 640, 192, "bf16", 256, 256, 2, 3, None, "tile", 1),
    ("subtile_r8_256x256", [512], 512, 128, "bf16", 256, 256, 1, 2, None, "subtile", 8),
    ("fp16_256x256", [256, 256], 512, 256, "fp16", 256, 256, 1, 3, (1, 1), "tile", 1),
    # 256 x 256 tiles with a 128-row or 64-column wave band wholly past the edge (rows 40 and 44; a last
    # column tile of 64 columns): those waves skip their MFMAs
    ("empty_bands_256x256", [40, 300], 320, 192, "bf16", 256, 256, 2, 3, None, "tile", 1),
]


def _plans(entry):
    name, m, N, K, dt, BM, BN, S, W, comp, mode, R = entry
    dest = _rng_dest(sum(m), R, 5) if mode == "subtoken" else None
    o = make_plan(m, N, BM=BM, BN=BN, S=S, W=W, composition=comp, mode=mode, ranks=R, row_dest=dest)
    p = fo.Plan(m, N, K, dt, BM=BM, BN=BN, swizzle=S, wave_size=W, composition=comp, mode=mode, ranks=R,
                row_dest=dest)
    return o, p


def _inputs(entry, dist=None, seed=100):
    name, m, N, K, dt, *_ = entry
    M = sum(m)
    if dist is None:
        dist = ("normal", 0.5) if dt == "bf16" else ("uniform", -1.0, 1.0)
    A = to_bits(draw(seed + 1, (M, K), dist), dt)
    B = [to_bits(draw(seed + 2 + e, (N, K), dist), dt) for e in range(len(m))]
    peer = to_bits(draw(seed + 50, (M * N,), dist), dt)
    return A, B, peer


def _stack(B):
    return np.concatenate([b.reshape(-1) for b in B])


# --------------------------------------------------------------------------- reorders

@pytest.mark.parametrize("entry", PLANS, ids=[e[0] for e in PLANS])
def test_reorder_pre_post_bit_exact(entry):
    o, p = _plans(entry)
    off = element_offsets(o)
    X = random_bits(7, o.M * o.N, entry[4])
    Y = random_bits(8, o.M * o.N, entry[4])
    want_pre = oracle.pre_reorder(X.reshape(o.M, o.N), off)
    want_post = oracle.post_reorder(Y, off).ravel()
    say(f"reorder {entry[0]} M={o.M} N={o.N} NT={o.NT}")
    dX, dY = to_dev(X), to_dev(Y)
    r1, r2 = empty16(o.M * o.N), empty16(o.M * o.N)
    p.reorder_pre(dX, r1)
    p.reorder_post(dY, r2)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(r1), want_pre)
    assert np.array_equal(to_host(r2), want_post)


@pytest.mark.parametrize("entry", PLANS, ids=[e[0] for e in PLANS])
def test_reorder_post_by_groups(entry):
    """fo_reorder_post_groups writes exactly the elements whose reordered offset lies in the
    groups' spans (oracle spans) and leaves the rest of out untouched; one call per group
    rebuilds the whole row-major output."""
    from oracle.layout import group_spans
    o, p = _plans(entry)
    off = element_offsets(o).ravel()
    spans = group_spans(o)
    Y = random_bits(9, o.M * o.N, entry[4])
    want = oracle.post_reorder(Y, off).ravel()
    marker = 0x7FC0
    dY = to_dev(Y)
    say(f"reorder_post by groups {entry[0]} P={p.P}")
    for g0, g1 in {(0, p.P), (0, 1), (p.P - 1, p.P), (p.P // 2, p.P // 2)}:
        out = empty16(o.M * o.N, marker)
        p.reorder_post(dY, out, groups=(g0, g1))
        torch.cuda.synchronize()
        inside = (off >= spans[g0]) & (off < spans[g1])
        got = to_host(out)
        assert np.array_equal(got[inside], want[inside]), (g0, g1)
        assert np.all(got[~inside] == marker), (g0, g1)
    out = empty16(o.M * o.N, marker)
    for g in range(p.P):
        p.reorder_post(dY, out, groups=(g, g + 1))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), want)
    with pytest.raises(fo.FoError):
        p.reorder_post(dY, out, groups=(0, p.P + 1))


# --------------------------------------------------------------------------- fused post-reorder epilogue

@pytest.mark.parametrize("act", ["none", "relu", "silu"])
@pytest.mark.parametrize("entry", PLANS, ids=[e[0] for e in PLANS])
def test_post_reorder_epilogue(entry, act):
    """none / relu: bit-exact (one fp32 add, one rounding on both sides); silu: within one
    unit in the last place (the kernel evaluates exp in fp32, the oracle in fp64)."""
    o, p = _plans(entry)
    dt = entry[4]
    off = element_offsets(o)
    Y = to_bits(draw(61, (o.M * o.N,), ("normal", 2.0)), dt)
    bias = to_bits(draw(62, (len(o.m_per_problem) * o.N,), ("normal", 1.0)), dt)
    dY = to_dev(Y)
    for b in (None, bias):
        want = post_epilogue(Y, off, dt, act, b, row_problems(o)).ravel()
        say(f"post epilogue {entry[0]} act={act} bias={b is not None}")
        out = empty16(o.M * o.N)
        p.reorder_post_ep(dY, out, bias=to_dev(b) if b is not None else None, act=act)
        torch.cuda.synchronize()
        got = to_host(out)
        if act == "silu":
            d = ulp_distance(got, want)
            assert d.max() <= 1, (int(d.max()), int((d > 0).sum()))
        else:
            assert np.array_equal(got, want)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_silu_epilogue_over_the_whole_input_range(dt):
    """SiLU through the fused post-reorder on values spread over every exponent, negative ones included down to
    where the logistic underflows fp32 (x < -87) and the result is a bf16 denormal or zero, plus both infinities
    and the extreme finite values: within one unit in the last place of the fp64 oracle everywhere, NaN where
    the oracle's formula gives NaN (x = -inf)."""
    o, p = _plans(PLANS[0][:4] + (dt,) + PLANS[0][5:])      # the tiny plan, in the dtype under test
    off = element_offsets(o)
    n = o.M * o.N
    special = np.array([-64.0, -63.99, -87.0, -88.7, -92.0, -96.0, -100.0, -103.0, -110.0, -130.0, -1e30, -3e38,
                        3e38, -np.inf, np.inf, 0.0, -0.0, 1e-30, -1e-30], np.float32)
    rng = np.random.Generator(np.random.PCG64(5))
    spread = (rng.choice([-1.0, 1.0], n) * np.exp2(rng.uniform(-130, 128, n))).astype(np.float32)
    grid = -np.linspace(0.0, 140.0, n // 4, dtype=np.float32)
    vals = np.concatenate([special, grid, spread])[:n]
    Y = to_bits(vals, dt)
    want = post_epilogue(Y, off, dt, "silu", None, row_problems(o)).ravel()
    say(f"silu over the whole range {dt}")
    out = empty16(n)
    p.reorder_post_ep(to_dev(Y), out, act="silu")
    torch.cuda.synchronize()
    got = to_host(out)
    nan = np.isnan(oracle.decode_bits(want, dt))          # -inf: x / (1 + e^-x) is -inf / inf on both sides
    assert np.array_equal(np.isnan(oracle.decode_bits(got, dt)), nan) and nan.any()
    d = ulp_distance(got[~nan], want[~nan])
    assert d.max() <= 1, (int(d.max()), int((d > 0).sum()))


# --------------------------------------------------------------------------- consumer

@pytest.mark.parametrize("entry", PLANS, ids=[e[0] for e in PLANS])
def test_consumer_all_groups_bit_exact(entry):
    o, p = _plans(entry)
    dt = entry[4]
    send = random_bits(11, o.M * o.N, dt)
    peer = random_bits(12, o.M * o.N, dt)
    want = oracle.consume_add(send, peer, dt)
    say(f"consumer {entry[0]} P={o.P} units={p.num_units}")
    sig = p.new_sig()
    p.flag_of(sig).fill_(3)            # every group already signalled at epoch 3
    status = zeros_i32(1)
    dsend, dpeer = to_dev(send), to_dev(peer)
    recv = empty16(o.M * o.N)
    p.consume_group(dsend, dpeer, recv, sig, 3, status, num_workgroups=7)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(to_host(recv), want)
    # in place: recv aliases send
    p.consume_group(dsend, dpeer, dsend, sig, 3, status)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(dsend), want)


def test_consumer_times_out_on_unsignalled_group_and_leaves_it_untouched():
    entry = PLANS[0]
    o, p = _plans(entry)
    dt = entry[4]
    send = random_bits(21, o.M * o.N, dt)
    peer = random_bits(22, o.M * o.N, dt)
    want = oracle.consume_add(send, peer, dt)
    spans = group_spans(o)
    say("consumer time-out: group 2 never signalled, 20 ms limit")
    sig = p.new_sig()
    p.flag_of(sig)[0:2] = 1            # group 2 stays at 0: the host never raises it
    status = zeros_i32(1)
    recv = empty16(o.M * o.N)
    p.consume_group(to_dev(send), to_dev(peer), recv, sig, 1, status, timeout_us=20000, num_workgroups=4)
    torch.cuda.synchronize()
    assert int(status.item()) == fo.FO_ERR_TIMEOUT
    got = to_host(recv)
    assert np.array_equal(got[:spans[2]], want[:spans[2]])
    assert np.all(got[spans[2]:] == 0x7FC0)


@pytest.mark.parametrize("tile,M,N", [((64, 64), 1024, 2048), ((128, 128), 2048, 4096), ((256, 128), 2048, 8192),
                                      ((256, 256), 4096, 8192)])
def test_polling_consumer_launched_first_stays_beside_the_gemm(tile, M, N):
    """Residency: the persistent consumer (one workgroup per CU) is launched before the GEMM on another
    queue and polls until the GEMM signals; a full wave of GEMM workgroups (W = the CU count, two waves)
    must still find room beside it on every CU, or the consumer times out (bounded at 0.5 s) before the
    GEMM can signal.  Every tile is checked; beside the 256 x 256 tile (two 232-register GEMM waves per
    SIMD) the consumer runs in its slim form."""
    K = 512
    BM, BN = tile
    p = fo.Plan([M], N, K, "bf16", BM=BM, BN=BN)     # W = the CU count, one group per wave
    if p.NT != 2 * p.W:
        p.close()
        pytest.skip(f"the shapes give two waves on 256 CUs; this device has W = {p.W}")
    say(f"polling consumer first, tile {BM}x{BN}, W={p.W}")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    A = (torch.randn(M * K, device="cuda", generator=g) * 0.1).to(torch.bfloat16).view(torch.int16)
    B = (torch.randn(N * K, device="cuda", generator=g) * 0.1).to(torch.bfloat16).view(torch.int16)
    peer = torch.zeros(M * N, dtype=torch.int16, device="cuda")
    buf = torch.empty(M * N, dtype=torch.int16, device="cuda")
    recv = torch.empty_like(buf)
    sig = p.new_sig()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sa, sb = fo.stream_create(), fo.stream_create()
    torch.cuda.synchronize()
    try:
        for e in (1, 2):
            recv.fill_(-1)
            p.consume_group(buf, peer, recv, sig, e, status, timeout_us=500000, stream=sb)
            p.gemm_signal(A, B, buf, sig, e, stream=sa)
            torch.cuda.synchronize()
            assert int(status.item()) == 0, fo.status_string(int(status.item()))
            # peer is zero: every element of recv is its element of the GEMM's reordered output
            assert torch.equal(recv, buf)
    finally:
        fo.stream_destroy(sa)
        fo.stream_destroy(sb)
        p.close()


def test_consumer_group_range():
    entry = PLANS[1]
    o, p = _plans(entry)
    send = random_bits(31, o.M * o.N, "bf16")
    peer = random_bits(32, o.M * o.N, "bf16")
    want = oracle.consume_add(send, peer, "bf16")
    spans = group_spans(o)
    say("consumer groups [1, 3)")
    sig = p.new_sig()
    p.flag_of(sig).fill_(1)
    status = zeros_i32(1)
    recv = empty16(o.M * o.N)
    p.consume_group(to_dev(send), to_dev(peer), recv, sig, 1, status, g_begin=1, g_end=3)
    torch.cuda.synchronize()
    got = to_host(recv)
    assert np.array_equal(got[spans[1]:spans[3]], want[spans[1]:spans[3]])
    assert np.all(got[:spans[1]] == 0x7FC0) and np.all(got[spans[3]:] == 0x7FC0)


# --------------------------------------------------------------------------- GEMM

@pytest.mark.parametrize("entry", PLANS, ids=[e[0] for e in PLANS])
def test_gemm_plain_within_tolerance(entry):
    o, p = _plans(entry)
    dt = entry[4]
    A, B, _ = _inputs(entry)
    r = oracle.run_pipeline(A, B, np.zeros(o.M * o.N, np.uint16), o, dt)
    say(f"gemm_plain {entry[0]} M={o.M} N={o.N} K={p.K} tile={p.BM}x{p.BN}")
    C = empty16(o.M * o.N)
    p.gemm_plain(to_dev(A), to_dev(_stack(B)), C)
    torch.cuda.synchronize()
    ratio = tol_check(to_host(C).reshape(o.M, o.N), r["C64"], dt, "C")
    assert ratio < 0.05, ratio           # diagnostic: a wrong k-slice or operand would be O(1)


# ternary products sum to integers of magnitude <= K, exact in 16 bits only for K <= 256
TERNARY = [e for e in PLANS if e[3] <= 256]


@pytest.mark.parametrize("entry", TERNARY, ids=[e[0] for e in TERNARY])
def test_gemm_ternary_bit_exact(entry):
    o, p = _plans(entry)
    dt = entry[4]
    A, B, _ = _inputs(entry, dist=("ternary",))
    r = oracle.run_pipeline(A, B, np.zeros(o.M * o.N, np.uint16), o, dt)
    say(f"gemm ternary {entry[0]}")
    C = empty16(o.M * o.N)
    buf = empty16(o.M * o.N)
    sig = p.new_sig()
    dA, dB = to_dev(A), to_dev(_stack(B))
    p.gemm_plain(dA, dB, C)
    p.gemm_signal(dA, dB, buf, sig, 1)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(C), r["C"].ravel())
    assert np.array_equal(to_host(buf), r["send"])


@pytest.mark.parametrize("entry", PLANS, ids=[e[0] for e in PLANS])
def test_gemm_signal_tables_and_layout(entry):
    o, p = _plans(entry)
    dt = entry[4]
    A, B, _ = _inputs(entry, seed=300)
    r = oracle.run_pipeline(A, B, np.zeros(o.M * o.N, np.uint16), o, dt)
    say(f"gemm_signal {entry[0]} P={o.P} thresholds={o.group_tiles}")
    dA, dB = to_dev(A), to_dev(_stack(B))
    C = empty16(o.M * o.N)
    buf = empty16(o.M * o.N)
    back = empty16(o.M * o.N)
    sig = p.new_sig()
    trace = torch.zeros(2 * p.NT + p.P, dtype=torch.int64, device="cuda")
    p.gemm_plain(dA, dB, C)
    for epoch in (1, 2, 3):
        trace.zero_()
        p.gemm_signal(dA, dB, buf, sig, epoch, trace=trace)
        torch.cuda.synchronize()
        s = sig.cpu().numpy()
        assert s[:p.P].tolist() == [epoch * g for g in o.group_tiles]          # counting table
        assert s[p.flag_offset:p.flag_offset + p.P].tolist() == [epoch] * p.P  # every group signalled
        assert not s[p.P:p.flag_offset].any()                                 # padding untouched
        tr = trace.cpu().numpy().view(np.uint64)
        tickets = (tr[1:2 * p.NT:2] & 0xFFFFFFFF).astype(np.int64)
        for j in range(p.P):
            got = np.sort(tickets[np.array(o.group_of_b) == j])
            assert got.tolist() == list(range((epoch - 1) * o.group_tiles[j], epoch * o.group_tiles[j]))
        assert tr[2 * p.NT:].tolist() == [1] * p.P                             # each group fired once
        wg = (tr[1:2 * p.NT:2] >> 32).astype(np.int64)
        assert np.all(wg < p.W)
    # reordered layout: within tolerance of the oracle's pre-reordered C ...
    tol_check(to_host(buf), oracle.pre_reorder(r["C64"], r["off"]), dt, "reorder_buf")
    # ... and bit-identical to the plain GEMM once reordered back
    p.reorder_post(buf, back)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(back), to_host(C))


@pytest.mark.parametrize("entry", PLANS, ids=[e[0] for e in PLANS])
def test_serialized_waves_reproduce_the_counting_trajectory(entry):
    """With a device-wide barrier after every wave the GPU's counting table after each wave is the
    oracle's trajectory (deep-dive 一 › 实现方法: the worked example's table after each wave), the
    flags rise exactly at each group's last wave, and the output is the normal launch's, bit for bit."""
    o, p = _plans(entry)
    A, B, _ = _inputs(entry, seed=500)
    snaps_want, fire = oracle.counting_trajectory(o)
    dA, dB = to_dev(A), to_dev(_stack(B))
    ref = empty16(o.M * o.N)
    p.gemm_signal(dA, dB, ref, p.new_sig(), 1)
    buf = empty16(o.M * o.N)
    sig = p.new_sig()
    for epoch in (1, 2):
        say(f"serialized waves {entry[0]} T={p.T} P={p.P} epoch={epoch}")
        snaps = torch.zeros(2 * p.T * p.P + 2, dtype=torch.int32, device="cuda")
        p.gemm_signal_serialized(dA, dB, buf, sig, epoch, snaps)
        torch.cuda.synchronize()
        s = snaps.cpu().numpy().astype(np.int64)
        assert s[-1] == 0, fo.status_string(int(s[-1]))
        assert s[-2] == 2 * p.T * p.W                              # every workgroup at every barrier
        for w in range(p.T):
            cnt = s[2 * w * p.P:2 * w * p.P + p.P]
            flg = s[2 * w * p.P + p.P:2 * (w + 1) * p.P]
            base = [(epoch - 1) * g for g in o.group_tiles]
            assert cnt.tolist() == [b + x for b, x in zip(base, snaps_want[w])], (w, cnt.tolist())
            assert flg.tolist() == [epoch if fire[j] <= w else epoch - 1 for j in range(p.P)], (w, flg.tolist())
    assert np.array_equal(to_host(buf), to_host(ref))


def test_gemm_each_workgroup_runs_its_wave_slot():
    """With W = 4 on the tiny shape, workgroup g runs dispatch indices g, g+4, g+8, g+12."""
    entry = PLANS[0]
    o, p = _plans(entry)
    A, B, _ = _inputs(entry)
    say("gemm_signal wave placement W=4")
    sig = p.new_sig()
    trace = torch.zeros(2 * p.NT + p.P, dtype=torch.int64, device="cuda")
    buf = empty16(o.M * o.N)
    p.gemm_signal(to_dev(A), to_dev(_stack(B)), buf, sig, 1, trace=trace)
    torch.cuda.synchronize()
    tr = trace.cpu().numpy().view(np.uint64)
    wg = (tr[1:2 * p.NT:2] >> 32).astype(np.int64)
    assert wg.tolist() == [b % 4 for b in range(p.NT)]
    # per workgroup, its tiles signal in dispatch order
    ts = tr[0:2 * p.NT:2].astype(np.int64)
    for g in range(4):
        t = ts[g::4]
        assert np.all(np.diff(t) >= 0)


# --------------------------------------------------------------------------- addressing

def _views_above_bit31(sizes16):
    """Views of one allocation, each 256-byte aligned at an address whose low 32-bit word has bit 31 set.

    The kernels build buffer resources from 64-bit addresses split into two
    32-bit halves; a half widened as a signed value would corrupt the base
    only for such addresses, which the allocator hands out or not by chance.
    """
    total = sum((n * 2 + 255) // 256 * 256 for n in sizes16)
    assert total < 2 ** 31
    big = torch.empty(2 ** 32 + total, dtype=torch.uint8, device="cuda")
    base = big.data_ptr()
    start = (2 ** 31 - (base & 0xFFFFFFFF)) % 2 ** 32   # next address whose low word is exactly 2^31
    views, off = [], start
    for n in sizes16:
        v = big[off:off + 2 * n].view(torch.int16)
        assert v.data_ptr() & 0x80000000 and v.data_ptr() % 256 == 0
        views.append(v)
        off += (n * 2 + 255) // 256 * 256
    return big, views


def test_every_kernel_with_buffers_above_bit31_of_the_low_word():
    entry = PLANS[2]                                   # ragged_128: several tiles, ragged edges
    o, p = _plans(entry)
    dt = entry[4]
    MN = o.M * o.N
    A, B, peer = _inputs(entry, seed=400)
    Bs = _stack(B)
    Xh = random_bits(41, MN, dt)
    r = oracle.run_pipeline(A, B, peer, o, dt)
    c_send = oracle.pre_reorder(r["C64"], r["off"])
    say(f"high addresses {entry[0]} M={o.M} N={o.N} K={p.K}")
    big, (dA, dB, dpeer, C, buf, recv, out, X, Y) = _views_above_bit31([A.size, Bs.size] + [MN] * 7)
    dA.copy_(to_dev(A).reshape(-1))
    dB.copy_(to_dev(Bs).reshape(-1))
    dpeer.copy_(to_dev(peer).reshape(-1))
    X.copy_(to_dev(Xh).reshape(-1))
    for v in (C, buf, recv, out, Y):
        v.fill_(0x7FC0)
    sig = p.new_sig()
    status = zeros_i32(1)
    p.gemm_plain(dA, dB, C)
    p.gemm_signal(dA, dB, buf, sig, 1)
    p.consume_group(buf, dpeer, recv, sig, 1, status)
    p.reorder_post(recv, out)
    p.reorder_pre(X, Y)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    tol_check(to_host(C).reshape(o.M, o.N), r["C64"], dt, "C")
    tol_check(to_host(buf), c_send, dt, "reorder_buf")
    tol_check_out(to_host(recv), oracle.decode_bits(r["recv"], dt), c_send, dt, "recv")
    tol_check_out(to_host(out).reshape(o.M, o.N), oracle.decode_bits(r["out"], dt), r["C64"], dt, "out")
    assert np.array_equal(to_host(Y), oracle.pre_reorder(Xh.reshape(o.M, o.N), r["off"]))
    del big


# --------------------------------------------------------------------------- gated consumer

@pytest.mark.parametrize("entry", PLANS, ids=[e[0] for e in PLANS])
def test_consumer_gated_bit_exact(entry):
    """The consumer gated by a stream wait on each flag: bit-exact against the oracle over all groups,
    and over a range of groups (the rest of recv untouched)."""
    o, p = _plans(entry)
    dt = entry[4]
    send = random_bits(15, o.M * o.N, dt)
    peer = random_bits(16, o.M * o.N, dt)
    want = oracle.consume_add(send, peer, dt)
    spans = group_spans(o)
    say(f"consumer gated {entry[0]} P={o.P}")
    sig = p.new_sig()
    p.flag_of(sig).fill_(4)            # every group already signalled at epoch 4
    status = zeros_i32(1)
    dsend, dpeer = to_dev(send), to_dev(peer)
    recv = empty16(o.M * o.N)
    p.consume_group_gated(dsend, dpeer, recv, sig, 4, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(to_host(recv), want)
    if o.P >= 2:
        recv = empty16(o.M * o.N)
        p.consume_group_gated(dsend, dpeer, recv, sig, 3, status, g_begin=1, g_end=o.P)   # flags >= 3 as well
        torch.cuda.synchronize()
        got = to_host(recv)
        assert np.array_equal(got[spans[1]:], want[spans[1]:])
        assert np.all(got[:spans[1]] == 0x7FC0)


# --------------------------------------------------------------------------- ReduceScatter shards, row exchange

SUBTILE = [e for e in PLANS if e[10] == "subtile"] + [
    ("subtile_r8_multi", [256, 512], 256, 64, "bf16", 256, 128, 2, 3, None, "subtile", 8),
    ("subtile_r16_64", [192], 128, 64, "fp16", 64, 64, 1, 5, None, "subtile", 16),
]


@pytest.mark.parametrize("entry", SUBTILE, ids=[e[0] for e in SUBTILE])
def test_reorder_shards_and_row_exchange_bit_exact(entry):
    from oracle.rowexchange import row_exchange, shard_reorder
    o, p = _plans(entry)
    dt = entry[4]
    off = element_offsets(o)
    Y = random_bits(17, o.M * o.N, dt)
    want_g = shard_reorder(Y, off, o)
    say(f"shards + row exchange {entry[0]} M={o.M} N={o.N} R={entry[11]}")
    dY = to_dev(Y)
    g, out = empty16(o.M * o.N), empty16(o.M * o.N)
    p.reorder_shards(dY, g)
    p.row_exchange(g, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(g), want_g)
    assert np.array_equal(to_host(out), row_exchange(want_g, o).ravel())
    assert np.array_equal(to_host(out), oracle.post_reorder(Y, off).ravel())


@pytest.mark.parametrize("act", ["none", "relu", "silu"])
@pytest.mark.parametrize("entry", SUBTILE, ids=[e[0] for e in SUBTILE])
def test_row_exchange_epilogue(entry, act):
    """none / relu: bit-exact; silu within one unit in the last place (exp in fp32 against fp64)."""
    from oracle.rowexchange import row_exchange_epilogue
    o, p = _plans(entry)
    dt = entry[4]
    G = to_bits(draw(63, (o.M * o.N,), ("normal", 2.0)), dt)
    bias = to_bits(draw(64, (len(o.m_per_problem) * o.N,), ("normal", 1.0)), dt)
    dG = to_dev(G)
    for b in (None, bias):
        want = row_exchange_epilogue(G, o, dt, act, b, row_problems(o)).ravel()
        say(f"row exchange epilogue {entry[0]} act={act} bias={b is not None}")
        out = empty16(o.M * o.N)
        p.row_exchange(dG, out, bias=to_dev(b) if b is not None else None, act=act)
        torch.cuda.synchronize()
        got = to_host(out)
        if act == "silu":
            assert ulp_distance(got, want).max() <= 1
        else:
            assert np.array_equal(got, want)


def test_shard_calls_refuse_other_layouts():
    entry = PLANS[1]
    o, p = _plans(entry)
    x = empty16(o.M * o.N)
    for call in (lambda: p.reorder_shards(x, x), lambda: p.row_exchange(x, x)):
        with pytest.raises(fo.FoError) as e:
            call()
        assert e.value.code == fo.FO_ERR_INVALID
