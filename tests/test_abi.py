"""The C-ABI library loads, exports every symbol include/fo.h declares, and
rejects bad arguments with the documented codes -- all without a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

fo = pytest.importorskip("gemm_tile_signaling_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "fo.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fo_[a-z_]+)\s*\(", src)))


def test_library_is_built_from_the_current_sources():
    """The library the tests load is at least as new as every source and header it is built from: a
    build that failed leaves the previous library in place, and every other test would then check
    that one instead."""
    if os.environ.get("FO_LIB"):
        pytest.skip("FO_LIB names another library")
    lib_t = os.path.getmtime(fo.LIB_PATH)
    pkg = os.path.join(ROOT, "gemm_tile_signaling_amd")
    srcs = [os.path.join(ROOT, "include", "fo.h"), os.path.join(pkg, "build.py")]
    for d, _, files in os.walk(os.path.join(pkg, "csrc")):
        srcs += [os.path.join(d, f) for f in files if f.endswith((".cpp", ".hip", ".h"))]
    stale = [os.path.relpath(f, ROOT) for f in srcs if os.path.getmtime(f) > lib_t]
    assert not stale, f"libfo.so is older than {stale}: rebuild (python -m gemm_tile_signaling_amd.build)"


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"fo_plan_groups", "fo_gemm_signal", "fo_consume_group", "fo_reorder_post"} <= set(names)
    L = ctypes.CDLL(fo.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert fo.status_string(0) == "ok"
    for c in (-1, -2, -3, -4, -5):
        assert fo.status_string(c) not in ("ok", "unknown status")
    assert fo.status_string(-99) == "unknown status"


def _code(fn):
    with pytest.raises(fo.FoError) as e:
        fn()
    return e.value.code


def test_plan_argument_errors():
    P = fo.Plan
    assert _code(lambda: P(256, 256, 256, composition=(1, 2), BM=64, BN=64, wave_size=4, host_only=True)) == -1
    assert _code(lambda: P(256, 256, 256, composition=(0, 4), BM=64, BN=64, wave_size=4, host_only=True)) == -1
    assert _code(lambda: P(256, 250, 256, host_only=True)) == -1                    # N % 8
    assert _code(lambda: P(256, 256, 200, host_only=True)) == -2                    # K % 64
    assert _code(lambda: P(256, 256, 256, BM=32, BN=32, host_only=True)) == -2      # tile shape
    assert _code(lambda: P(250, 256, 256, BM=64, BN=64, mode="subtile", ranks=4, host_only=True)) == -1
    assert _code(lambda: P(256, 256, 256, BM=64, BN=64, mode="subtile", ranks=3, host_only=True)) == -1
    assert _code(lambda: P(4, 64, 64, BM=64, BN=64, mode="subtoken", ranks=2, row_dest=[0, 1, 2, 0],
                           host_only=True)) == -1
    assert _code(lambda: P(128, 128, 64, BM=64, BN=64, dispatch_order=[0, 0, 1, 2], host_only=True)) == -1
    assert _code(lambda: P([-1], 64, 64, host_only=True)) == -1
    # buffers are addressed with 32-bit byte offsets: M * N may not exceed 2^30 elements
    assert _code(lambda: P(2 ** 15 + 1, 2 ** 15, 64, host_only=True)) == -2
    assert P(2 ** 15, 2 ** 15, 64, host_only=True).M == 2 ** 15


def test_enqueue_on_host_only_plan_is_rejected():
    p = fo.Plan(256, 256, 256, "fp16", BM=64, BN=64, swizzle=2, wave_size=4, composition=(1, 2, 1), host_only=True)
    # addresses are never dereferenced: the host-only plan is refused first
    assert _code(lambda: p.gemm_signal(16, 16, 16, 16, 1, stream=0)) == -1
    assert _code(lambda: p.gemm_plain(16, 16, 16, stream=0)) == -1
    assert _code(lambda: p.consume_group(16, 16, 16, 16, 1, 16, stream=0)) == -1
    assert _code(lambda: p.reorder_post(16, 16, stream=0)) == -1
    assert _code(lambda: p.reorder_post(16, 16, groups=(0, 1), stream=0)) == -1
    assert _code(lambda: p.reorder_pre(16, 16, stream=0)) == -1
    assert p.info["device"] == -1


def test_default_plan_parameters():
    p = fo.Plan(2048, 8192, 8192, host_only=True)
    assert (p.BM, p.BN, p.S, p.W) == (256, 128, 4, 256)
    assert p.NT == 512 and p.T == 2 and p.P == 2


def test_signal_buffer_layout():
    """cnt[P] from word 0, flag[P] from the next multiple of 64 words (a 256-byte boundary)."""
    P = fo.Plan
    p = P(256, 256, 64, "fp16", BM=64, BN=64, swizzle=2, wave_size=4, composition=(1, 2, 1), host_only=True)
    assert (p.P, p.flag_offset, p.sig_words) == (3, 64, 67)
    many = P(64 * 80, 64, 64, BM=64, BN=64, swizzle=1, wave_size=1, host_only=True)   # one wave per group
    assert (many.P, many.flag_offset, many.sig_words) == (80, 128, 208)
    edge = P(64 * 64, 64, 64, BM=64, BN=64, swizzle=1, wave_size=1, host_only=True)
    assert (edge.P, edge.flag_offset, edge.sig_words) == (64, 64, 128)
    empty = P(0, 64, 64, BM=64, BN=64, swizzle=1, wave_size=4, composition=(), host_only=True)
    assert (empty.P, empty.flag_offset, empty.sig_words) == (0, 0, 0)


def test_status_string_of_the_stale_read_code():
    assert fo.FO_ERR_STALE == -6
    assert "stamp" in fo.status_string(-6)


def test_layout_of_b_and_operand_limits():
    """Only B stored [N, K] is implemented; a tile's operand rows must fit 32-bit byte offsets."""
    P = fo.Plan
    assert _code(lambda: P(256, 256, 256, host_only=True, b_layout="kn")) == -2
    # max(BM, BN) * K * 2 must stay below 2^32: K = 2^23 is refused at BM = 256, accepted at BM = BN = 64
    assert _code(lambda: P(256, 128, 2 ** 23, host_only=True)) == -2
    assert P(256, 128, 2 ** 23 - 64, host_only=True).K == 2 ** 23 - 64
    assert P(64, 64, 2 ** 23, BM=64, BN=64, host_only=True).K == 2 ** 23
    assert _code(lambda: P(64, 64, 2 ** 25, BM=64, BN=64, host_only=True)) == -2


def test_unknown_plan_flags_are_refused():
    L = fo.lib()
    m = (ctypes.c_int64 * 1)(256)
    d = fo._Desc(num_problems=1, m_per_problem=ctypes.cast(m, ctypes.POINTER(ctypes.c_int64)), N=256, K=256,
                 flags=fo.FO_PLAN_HOST_ONLY | 0x100)
    h = ctypes.c_void_p()
    assert L.fo_plan_groups(ctypes.byref(d), ctypes.byref(h)) == -1
    d.flags = fo.FO_PLAN_HOST_ONLY
    d.b_layout = 7
    assert L.fo_plan_groups(ctypes.byref(d), ctypes.byref(h)) == -1


def test_architecture_check():
    """The kernels are gfx950 code: the name up to the first ':' must be exactly gfx950."""
    assert fo.arch_supported("gfx950")
    assert fo.arch_supported("gfx950:sramecc+:xnack-")
    for other in ("gfx942", "gfx942:sramecc+:xnack-", "gfx90a", "gfx9500", "gfx95", "", None):
        assert not fo.arch_supported(other), other


def test_epoch_stamp_layout():
    """With epoch stamps the signal buffer gains one word per slot after the flags, on a 64-word boundary."""
    P = fo.Plan
    p = P(256, 256, 64, "fp16", BM=64, BN=64, swizzle=2, wave_size=4, composition=(1, 2, 1), host_only=True,
          epoch_stamps=True)
    assert (p.P, p.flag_offset, p.stamp_offset, p.NT, p.sig_words) == (3, 64, 128, 16, 144)
    assert p.info["flags"] == fo.FO_PLAN_HOST_ONLY | fo.FO_PLAN_EPOCH_STAMPS
    many = P(64 * 80, 64, 64, BM=64, BN=64, swizzle=1, wave_size=1, host_only=True, epoch_stamps=True)
    assert (many.flag_offset, many.stamp_offset, many.sig_words) == (128, 256, 256 + 80)
    plain = P(256, 256, 64, "fp16", BM=64, BN=64, swizzle=2, wave_size=4, composition=(1, 2, 1), host_only=True)
    assert plain.stamp_offset == -1
    with pytest.raises(ValueError):
        plain.stamps_of(np.zeros(plain.sig_words, np.int32))


def test_new_enqueue_calls_reject_host_only_and_wrong_layouts():
    p = fo.Plan(256, 256, 256, "fp16", BM=64, BN=64, swizzle=2, wave_size=4, mode="subtile", ranks=4,
                host_only=True)
    assert _code(lambda: p.consume_group_gated(16, 16, 16, 16, 1, 16, stream=0)) == -1
    assert _code(lambda: p.consume_group_gated(16, 16, 16, 16, 1, 16, trace=20, stream=0)) == -1
    assert _code(lambda: p.reorder_shards(16, 16, stream=0)) == -1
    assert _code(lambda: p.row_exchange(16, 16, stream=0)) == -1


def test_mfma_rate_argument_errors():
    L = fo.lib()
    out = 256                       # a 4-aligned address; nothing is launched on a refused call
    assert L.fo_mfma_rate(2, 16, 16, 1, 1, out, None) == -1          # dtype
    assert L.fo_mfma_rate(0, 0, 16, 1, 1, out, None) == -1           # no operands
    assert L.fo_mfma_rate(0, 8, 16, 1, 1, out, None) == -1           # misaligned operands
    assert L.fo_mfma_rate(0, 16, 0, 1, 1, out, None) == -1           # empty
    assert L.fo_mfma_rate(0, 16, 24, 1, 1, out, None) == -1          # not whole vectors
    assert L.fo_mfma_rate(0, 16, 16, 0, 1, out, None) == -1          # no workgroups
    assert L.fo_mfma_rate(0, 16, 16, 65537, 1, out, None) == -1      # too many
    assert L.fo_mfma_rate(0, 16, 16, 1, -1, out, None) == -1         # negative rounds
    assert L.fo_mfma_rate(0, 16, 16, 1, 1, 0, None) == -1            # no output
    assert L.fo_mfma_rate(0, 16, 16, 1, 1, 258, None) == -1          # misaligned output
