"""Every kernel of the path on random plans (hypothesis, deterministic draws), bit-exact against the oracle.

The hand-picked plans of test_gpu_kernels.py cover the code paths; here the
same checks run on plans drawn at random -- tiles 64x64 .. 256x256, the three
layouts, ragged and empty problems, swizzle and wave sizes, a random
composition of the waves, K of 64 .. 256, bf16 or fp16 -- so that an indexing
slip that only some shape exposes has many chances to show.  Inputs are
ternary, so every product and sum of the GEMM is an exact integer and its
16-bit output is exact: the plain GEMM's row-major C, the signaling GEMM's
reordered buffer, the consumer's recv (either form; a random peer, one fp32 add and one
rounding per element) and the post-reorder's output are all compared bit for
bit, the fused bias + activation epilogue too (SiLU within one unit in the
last place), and the counting table and flags checked.
"""

import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import oracle  # noqa: E402
from oracle.epilogue import post_epilogue, row_problems  # noqa: E402
from oracle.layout import element_offsets  # noqa: E402
from tests.gpu_util import empty16, say, to_dev, to_host, ulp_distance, zeros_i32  # noqa: E402
from tests.test_properties import _oracle_plan, plans  # noqa: E402
from workloads import draw, random_bits, to_bits  # noqa: E402

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")


@settings(max_examples=400, deadline=None, derandomize=True, database=None)
@given(plans(), st.sampled_from(["bf16", "fp16"]), st.integers(1, 4), st.integers(0, 2 ** 16),
       st.sampled_from(["gated", "poll"]), st.sampled_from(["none", "relu", "silu"]))
def test_kernels_on_random_plans(c, dtype, kq, seed, consumer, act):
    K = 64 * kq
    o = _oracle_plan(c)
    M, N = o.M, o.N
    A = to_bits(draw(seed + 1, (M, K), ("ternary",)), dtype)
    B = [to_bits(draw(seed + 2 + e, (N, K), ("ternary",)), dtype) for e in range(len(c["m"]))]
    peer = random_bits(seed + 3, M * N, dtype)
    r = oracle.run_pipeline(A, B, peer, o, dtype)
    p = fo.Plan(c["m"], N, K, dtype, BM=c["BM"], BN=c["BN"], swizzle=c["S"], wave_size=c["W"], composition=c["comp"],
                mode=c["mode"], ranks=c["ranks"], row_dest=c["row_dest"])
    try:
        say(f"random plan {c['mode']} m={c['m']} N={N} K={K} {c['BM']}x{c['BN']} S={c['S']} W={c['W']} "
            f"comp={c['comp']} {dtype} NT={p.NT} P={p.P} consumer={consumer} act={act}")
        dA, dB, dpeer = to_dev(A), to_dev(np.concatenate([b.reshape(-1) for b in B])), to_dev(peer)
        C, buf, recv, out, out_ep = (empty16(M * N) for _ in range(5))
        bias = to_bits(draw(seed + 4, (len(c["m"]) * N,), ("normal", 1.0)), dtype)
        sig = p.new_sig()
        status = zeros_i32(1)
        p.gemm_plain(dA, dB, C)
        p.gemm_signal(dA, dB, buf, sig, 1)
        if consumer == "gated":
            p.consume_group_gated(buf, dpeer, recv, sig, 1, status)
        else:
            p.consume_group(buf, dpeer, recv, sig, 1, status)
        p.reorder_post(recv, out)
        p.reorder_post_ep(recv, out_ep, bias=to_dev(bias), act=act)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert np.array_equal(to_host(C), r["C"].ravel())
        assert np.array_equal(to_host(buf), r["send"])
        assert np.array_equal(to_host(recv), r["recv"])
        assert np.array_equal(to_host(out), r["out"].ravel())
        # the fused epilogue: bias + activation in the post-reorder's pass (SiLU within one unit in the last place)
        want_ep = post_epilogue(r["recv"], element_offsets(o), dtype, act, bias, row_problems(o)).ravel()
        if act == "silu":
            assert ulp_distance(to_host(out_ep), want_ep).max() <= 1
        else:
            assert np.array_equal(to_host(out_ep), want_ep)
        s = sig.cpu().numpy()
        assert s[:p.P].tolist() == list(o.group_tiles)
        assert s[p.flag_offset:p.flag_offset + p.P].tolist() == [1] * p.P
    finally:
        p.close()
