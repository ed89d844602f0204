"""fo_gemm_signal_noalloc, the signaling GEMM for callers that cannot allocate, against fo_gemm_signal.

Two calls in a row, the second on a smaller problem with another layout of the
signal words (the first plan's counters end in the words where the second
keeps its flags): each call's reordered buffer equals fo_gemm_signal's on the
same inputs bit for bit; the consumer and the post-reorder, fed the library's
signal words and epoch, give the output the allocating entry point's pass
gives (and the oracle's, within the GEMM's tolerance); the library's counting
table and flags hold the call's thresholds and epoch; epochs increase.
Plans whose signal words exceed the library's array are refused.
"""

import ctypes

import numpy as np
import pytest

import oracle
from tests.gpu_util import empty16, say, to_dev, to_host, tol_check_out, zeros_i32
from tests.test_gpu_kernels import PLANS, _inputs, _plans, _stack

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")


def _read_words(addr, n):
    """n uint32 words at a device address (hipMemcpy to the host)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    out = np.zeros(n, np.uint32)
    assert hip.hipMemcpy(out.ctypes.data, addr, 4 * n, 2) == 0        # hipMemcpyDeviceToHost
    return out


# 72 tiles of 64 x 64 in 72 one-tile waves cut into 67 groups: the flags start at word 128, and groups
# 64..66 count to 3, 3 and 2 -- in the words where the second, smaller plan (3 groups) keeps its flags
MANY_GROUPS = ("many_groups", [576], 512, 64, "bf16", 64, 64, 1, 1, (1,) * 64 + (3, 3, 2), "tile", 1)


def test_noalloc_matches_the_allocating_entry_point():
    # the second problem is smaller than the first; the third runs the eight-wave 256 x 128 kernel
    cases = [(MANY_GROUPS, "gated"), (next(x for x in PLANS if x[0] == "tiny_fp16"), "poll"),
             (next(x for x in PLANS if x[0] == "ragged_256"), "gated")]
    epochs = []
    for entry, consumer in cases:
        o, p = _plans(entry)
        dt = entry[4]
        A, B, peer = _inputs(entry, seed=900)
        dA, dB, dpeer = to_dev(A), to_dev(_stack(B)), to_dev(peer)
        say(f"no-alloc GEMM {entry[0]} M={o.M} N={o.N} P={p.P} consumer={consumer}")
        # the existing entry point, caller-owned signal words
        sig = p.new_sig()
        buf_ref, recv_ref, out_ref = empty16(o.M * o.N), empty16(o.M * o.N), empty16(o.M * o.N)
        st_ref = zeros_i32(1)
        p.gemm_signal(dA, dB, buf_ref, sig, 1)
        p.consume_group(buf_ref, dpeer, recv_ref, sig, 1, st_ref)
        p.reorder_post(recv_ref, out_ref)
        # the allocation-free entry point, the library's signal words and epoch
        buf, recv, out = empty16(o.M * o.N), empty16(o.M * o.N), empty16(o.M * o.N)
        st = zeros_i32(1)
        addr, epoch = p.gemm_signal_noalloc(dA, dB, buf)
        if consumer == "gated":
            p.consume_group_gated(buf, dpeer, recv, addr, epoch, st)
        else:
            p.consume_group(buf, dpeer, recv, addr, epoch, st, timeout_us=500000)
        p.reorder_post(recv, out)
        torch.cuda.synchronize()
        assert int(st_ref.item()) == 0 and int(st.item()) == 0, (int(st_ref.item()), int(st.item()))
        assert addr != 0 and addr % 256 == 0
        assert np.array_equal(to_host(buf), to_host(buf_ref))
        assert np.array_equal(to_host(recv), to_host(recv_ref))
        assert np.array_equal(to_host(out), to_host(out_ref))
        words = _read_words(addr, p.sig_words)
        assert words[:p.P].tolist() == list(p.tables()["group_tiles"])      # this call's counting table
        assert words[p.flag_offset:p.flag_offset + p.P].tolist() == [epoch] * p.P
        r = oracle.run_pipeline(A, B, peer, o, dt)
        tol_check_out(to_host(out).reshape(o.M, o.N), oracle.decode_bits(r["out"], dt), r["C64"], dt, "out")
        epochs.append(epoch)
        p.close()
    assert epochs[0] >= 1 and all(b > a for a, b in zip(epochs, epochs[1:]))


def test_noalloc_refuses_plans_beyond_its_array():
    # one wave per group, 16400 groups: the signal words need more than the library's 16384
    p = fo.Plan(64 * 16400, 64, 64, "bf16", BM=64, BN=64, swizzle=1, wave_size=1)
    assert p.sig_words > 16384
    x = torch.zeros(64, dtype=torch.int16, device="cuda")
    say(f"no-alloc refuses sig_words={p.sig_words}")
    with pytest.raises(fo.FoError) as e:
        p.gemm_signal_noalloc(x.data_ptr(), x.data_ptr(), x.data_ptr())
    assert e.value.code == fo.FO_ERR_UNSUPPORTED
    p.close()
    host = fo.Plan(256, 256, 256, host_only=True)
    with pytest.raises(fo.FoError) as e:
        host.gemm_signal_noalloc(x.data_ptr(), x.data_ptr(), x.data_ptr())
    assert e.value.code == fo.FO_ERR_INVALID
