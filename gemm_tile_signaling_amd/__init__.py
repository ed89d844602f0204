"""Python binding of libfo, the signaling GEMM with tile reordering for MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libfo.so`` (built by ``gemm_tile_signaling_amd/build.py``).  There is no
fallback: if the library is missing, importing the binding's entry points
raises.  PyTorch supplies device memory and streams; any object with
``data_ptr()`` (a torch tensor) or a plain integer address is accepted as a
buffer.

The names follow the C ABI in ``include/fo.h``: ``Plan`` wraps
``fo_plan_groups``; its methods ``gemm_signal``, ``gemm_plain``,
``consume_group``, ``consume_group_gated``, ``reorder_post``,
``reorder_post_ep``, ``reorder_pre``, ``reorder_shards`` and ``row_exchange``
wrap the enqueue calls of the same names, and ``search`` wraps
``fo_plan_search``.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

__all__ = ["Plan", "FoError", "lib", "LIB_PATH", "status_string", "stream_create", "stream_destroy",
           "arch_supported", "mfma_rate", "mfma_rate_flops", "FO_OK", "FO_ERR_INVALID", "FO_ERR_UNSUPPORTED", "FO_ERR_HIP", "FO_ERR_NOMEM",
           "FO_ERR_TIMEOUT", "FO_ERR_STALE"]

# FO_LIB names another build of the same library (the sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("FO_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfo.so")

FO_OK, FO_ERR_INVALID, FO_ERR_UNSUPPORTED, FO_ERR_HIP, FO_ERR_NOMEM, FO_ERR_TIMEOUT, FO_ERR_STALE = \
    0, -1, -2, -3, -4, -5, -6
_DTYPES = {"bf16": 0, "fp16": 1}
_MODES = {"tile": 0, "subtile": 1, "subtoken": 2}
_ACTS = {"none": 0, "relu": 1, "silu": 2}
_B_LAYOUTS = {"nk": 0, "kn": 1}
FO_PLAN_HOST_ONLY = 1
FO_PLAN_EPOCH_STAMPS = 2


class FoError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} ({code})")
        self.code = code


class _Desc(C.Structure):
    _fields_ = [
        ("num_problems", C.c_int32), ("m_per_problem", C.POINTER(C.c_int64)),
        ("N", C.c_int64), ("K", C.c_int64),
        ("dtype", C.c_int32), ("BM", C.c_int32), ("BN", C.c_int32), ("swizzle", C.c_int32),
        ("wave_size", C.c_int32), ("num_groups", C.c_int32), ("waves_per_group", C.POINTER(C.c_int32)),
        ("mode", C.c_int32), ("ranks", C.c_int32), ("row_dest", C.POINTER(C.c_int32)),
        ("dispatch_order", C.POINTER(C.c_int32)), ("flags", C.c_uint32), ("b_layout", C.c_int32),
    ]


class _Info(C.Structure):
    _fields_ = [("M", C.c_int64), ("N", C.c_int64), ("K", C.c_int64)] + [
        (n, C.c_int32) for n in ("BM", "BN", "swizzle", "wave_size", "NT", "T", "P", "num_units",
                                 "mode", "ranks", "dtype", "num_problems", "device", "clock_khz",
                                 "sig_words", "flag_offset", "stamp_offset", "flags")]


_lib = None


def lib() -> C.CDLL:
    """Load libfo.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run gemm_tile_signaling_amd/build.py "
                              "(or __graft_entry__.build()) first; there is no fallback path")
        L = C.CDLL(LIB_PATH)
        vp, i32, u32, i64, u64 = C.c_void_p, C.c_int32, C.c_uint32, C.c_int64, C.c_uint64
        sig = {
            "fo_plan_groups": [C.POINTER(_Desc), C.POINTER(vp)],
            "fo_plan_destroy": [vp],
            "fo_plan_info_get": [vp, C.POINTER(_Info)],
            "fo_plan_tables": [vp, vp, vp, vp, vp, vp],
            "fo_plan_units": [vp, vp, vp],
            "fo_plan_offsets": [vp, vp],
            "fo_plan_search": [vp, C.c_double, vp, vp, i32, vp, vp, vp, vp],
            "fo_gemm_signal": [vp, vp, vp, vp, vp, u32, vp, vp],
            "fo_gemm_plain": [vp, vp, vp, vp, vp],
            "fo_gemm_signal_serialized": [vp, vp, vp, vp, vp, u32, vp, vp],
            "fo_gemm_signal_noalloc": [vp, vp, vp, vp, vp, vp, vp],
            "fo_consume_group": [vp, vp, vp, vp, vp, u32, i32, i32, vp, u64, i32, vp, vp],
            "fo_consume_group_gated": [vp, vp, vp, vp, vp, u32, i32, i32, vp, vp, vp],
            "fo_reorder_shards": [vp, vp, vp, vp],
            "fo_row_exchange": [vp, vp, vp, vp, i32, vp],
            "fo_stream_create": [C.POINTER(vp)],
            "fo_stream_destroy": [vp],
            "fo_reorder_post": [vp, vp, vp, vp],
            "fo_reorder_post_groups": [vp, i32, i32, vp, vp, vp],
            "fo_reorder_pre": [vp, vp, vp, vp],
            "fo_reorder_post_ep": [vp, vp, vp, vp, i32, vp],
            "fo_mfma_rate": [i32, vp, i64, i32, i32, vp, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = C.c_int
        L.fo_status_string.argtypes = [C.c_int]
        L.fo_status_string.restype = C.c_char_p
        L.fo_arch_supported.argtypes = [C.c_char_p]
        L.fo_arch_supported.restype = C.c_int
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().fo_status_string(int(code)).decode()


def _check(code: int, what: str):
    if code != FO_OK:
        raise FoError(code, what)


def _arr(a, ctype):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a), dtype={C.c_int32: np.int32, C.c_int64: np.int64}[ctype])
    return arr, arr.ctypes.data_as(C.POINTER(ctype))


def _ptr(x, *, numel: Optional[int] = None, itemsize: Optional[int] = None, name: str = "buffer") -> int:
    """Device address of a buffer; checks size, element width and contiguity of torch tensors."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if hasattr(x, "is_contiguous") and not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if hasattr(x, "is_cuda") and not x.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if itemsize is not None and x.element_size() != itemsize:
            raise ValueError(f"{name}: element size {x.element_size()} != {itemsize}")
        if numel is not None and x.numel() < numel:
            raise ValueError(f"{name}: {x.numel()} elements < {numel} required")
        return int(x.data_ptr())
    raise TypeError(f"{name}: expected a tensor or an address")


def _stream(s) -> int:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def arch_supported(arch: Optional[str]) -> bool:
    """``fo_arch_supported``: can a device with this gcnArchName run the kernels (gfx950)."""
    return bool(lib().fo_arch_supported(None if arch is None else arch.encode()))


def stream_create():
    """A HIP stream with a hardware queue of its own (``fo_stream_create``), as a torch stream."""
    import torch
    h = C.c_void_p()
    _check(lib().fo_stream_create(C.byref(h)), "fo_stream_create")
    return torch.cuda.ExternalStream(h.value)


def stream_destroy(s):
    _check(lib().fo_stream_destroy(int(s.cuda_stream)), "fo_stream_destroy")


def mfma_rate(ops, out, workgroups: int, iters: int, dtype: str = "bf16", stream=None):
    """``fo_mfma_rate``: MFMAs only, on operand values read from ``ops`` (a measurement aid for the GEMM's
    roofline).  ``out``: float32 device tensor of ``workgroups * 512`` elements."""
    nbytes = ops.numel() * ops.element_size() if hasattr(ops, "numel") else None
    if nbytes is None:
        raise TypeError("ops: expected a device tensor")
    _check(lib().fo_mfma_rate(_DTYPES[dtype], _ptr(ops, name="ops"), nbytes, int(workgroups), int(iters),
                              _ptr(out, numel=int(workgroups) * 512, itemsize=4, name="out"), _stream(stream)),
           "fo_mfma_rate")


def mfma_rate_flops(workgroups: int, iters: int) -> float:
    """FLOP of one ``mfma_rate`` launch: 8 waves x ``iters`` rounds x 32 MFMAs of 16x16x32 per workgroup."""
    return float(workgroups) * 8 * iters * 32 * 2 * 16 * 16 * 32


class Plan:
    """A wave-group plan (``fo_plan_groups``): tables built once, uploaded once.

    ``m_per_problem``: rows of each problem (an int for a plain GEMM).
    ``composition``: waves per group (a partition of T); None = one wave per group.
    ``host_only``: build the tables without a GPU (the enqueue calls then refuse it).
    ``epoch_stamps``: the stale-read detector (``FO_PLAN_EPOCH_STAMPS``): one stamp word per slot in
    the signal buffer, written by the signaling GEMM and checked by the consumer.
    ``b_layout``: "nk" (B stored [N, K], the only one implemented) or "kn" (refused).
    """

    def __init__(self, m_per_problem, N: int, K: int, dtype: str = "bf16", *, BM: int = 0, BN: int = 0,
                 swizzle: int = 0, wave_size: int = 0, composition: Optional[Sequence[int]] = None,
                 mode: str = "tile", ranks: int = 1, row_dest=None, dispatch_order=None, host_only: bool = False,
                 epoch_stamps: bool = False, b_layout: str = "nk"):
        L = lib()
        if isinstance(m_per_problem, (int, np.integer)):
            m_per_problem = [int(m_per_problem)]
        self._m, mp = _arr(list(m_per_problem), C.c_int64)
        self._comp, cp = _arr(list(composition) if composition is not None else None, C.c_int32)
        self._rd, rp = _arr(row_dest, C.c_int32)
        self._do, dp = _arr(dispatch_order, C.c_int32)
        d = _Desc(num_problems=len(self._m), m_per_problem=mp, N=int(N), K=int(K), dtype=_DTYPES[dtype],
                  BM=int(BM), BN=int(BN), swizzle=int(swizzle), wave_size=int(wave_size),
                  num_groups=len(self._comp) if self._comp is not None else 0, waves_per_group=cp,
                  mode=_MODES[mode], ranks=int(ranks), row_dest=rp, dispatch_order=dp,
                  flags=(FO_PLAN_HOST_ONLY if host_only else 0) | (FO_PLAN_EPOCH_STAMPS if epoch_stamps else 0),
                  b_layout=_B_LAYOUTS[b_layout])
        h = C.c_void_p()
        _check(L.fo_plan_groups(C.byref(d), C.byref(h)), "fo_plan_groups")
        self._h = h
        info = _Info()
        _check(L.fo_plan_info_get(h, C.byref(info)), "fo_plan_info_get")
        self.info = {n: getattr(info, n) for n, _ in _Info._fields_}
        self.dtype = dtype
        self.mode = mode
        for k in ("M", "N", "K", "BM", "BN", "NT", "T", "P", "num_units", "sig_words", "flag_offset",
                  "stamp_offset"):
            setattr(self, k, self.info[k])
        self.W = self.info["wave_size"]
        self.S = self.info["swizzle"]
        self.num_problems = self.info["num_problems"]

    # ------------------------------------------------------------------ host-side tables
    def tables(self) -> dict:
        NT, P = self.NT, self.P
        t_of_s = np.zeros(NT, np.int32)
        s_of_t = np.zeros(NT, np.int32)
        g_of_s = np.zeros(NT, np.int32)
        g_tiles = np.zeros(P, np.int32)
        span = np.zeros(P + 1, np.int64)
        _check(lib().fo_plan_tables(self._h, t_of_s.ctypes.data, s_of_t.ctypes.data, g_of_s.ctypes.data,
                                    g_tiles.ctypes.data, span.ctypes.data), "fo_plan_tables")
        return dict(tile_of_slot=t_of_s, slot_of_tile=s_of_t, group_of_slot=g_of_s, group_tiles=g_tiles,
                    span_off=span)

    def units(self):
        uo = np.zeros(self.num_units + 1, np.int64)
        gu = np.zeros(self.P + 1, np.int32)
        _check(lib().fo_plan_units(self._h, uo.ctypes.data, gu.ctypes.data), "fo_plan_units")
        return uo, gu

    def offsets(self) -> np.ndarray:
        off = np.full((self.M, self.N), -1, np.int64)
        _check(lib().fo_plan_offsets(self._h, off.ctypes.data if off.size else None), "fo_plan_offsets")
        return off

    def search(self, gemm_seconds: float, curve_bytes, curve_seconds, with_all: bool = False):
        """Predictive partition search (``fo_plan_search``): returns (composition, predicted
        seconds, every candidate's prediction in cut-mask order or None)."""
        cb = np.ascontiguousarray(curve_bytes, dtype=np.float64)
        cs = np.ascontiguousarray(curve_seconds, dtype=np.float64)
        if cb.shape != cs.shape or cb.ndim != 1:
            raise ValueError("curve_bytes and curve_seconds must be 1-D and of one length")
        best = np.zeros(max(1, self.T), np.int32)
        ng = C.c_int32()
        bt = C.c_double()
        allt = np.zeros(1 << (self.T - 1), np.float64) if with_all and 0 < self.T <= 24 else None
        _check(lib().fo_plan_search(self._h, float(gemm_seconds), cb.ctypes.data, cs.ctypes.data, int(cb.size),
                                    best.ctypes.data, C.byref(ng), C.byref(bt),
                                    allt.ctypes.data if allt is not None else None), "fo_plan_search")
        return tuple(int(x) for x in best[:ng.value]), bt.value, allt

    # ------------------------------------------------------------------ enqueue calls
    @property
    def mn(self) -> int:
        return self.M * self.N

    def new_sig(self, device="cuda"):
        """A zeroed signal buffer, int32[sig_words] (at least one word): cnt[P] from word 0 and
        flag[P] from word flag_offset.  torch's allocations are 256-byte aligned, which keeps the
        flags on cache lines apart from the counters."""
        import torch
        return torch.zeros(max(1, self.sig_words), dtype=torch.int32, device=device)

    def cnt_of(self, sig):
        """The counting-table words cnt[P] of a signal buffer (a view)."""
        return sig[:self.P]

    def flag_of(self, sig):
        """The flag words flag[P] of a signal buffer (a view)."""
        return sig[self.flag_offset:self.flag_offset + self.P]

    def stamps_of(self, sig):
        """The epoch stamps, one per slot, of a signal buffer (a view); plans with epoch_stamps only."""
        if self.stamp_offset < 0:
            raise ValueError("the plan has no epoch stamps")
        return sig[self.stamp_offset:self.stamp_offset + self.NT]

    def gemm_signal(self, A, B, reorder_buf, sig, epoch: int, trace=None, stream=None):
        _check(lib().fo_gemm_signal(
            self._h, _ptr(A, numel=self.M * self.K, itemsize=2, name="A"),
            _ptr(B, numel=self.num_problems * self.N * self.K, itemsize=2, name="B"),
            _ptr(reorder_buf, numel=self.mn, itemsize=2, name="reorder_buf"),
            _ptr(sig, numel=self.sig_words, itemsize=4, name="sig"), int(epoch),
            _ptr(trace, numel=2 * self.NT + self.P, itemsize=8, name="trace"), _stream(stream)), "fo_gemm_signal")

    def gemm_signal_noalloc(self, A, B, reorder_buf, stream=None):
        """``fo_gemm_signal_noalloc``: the signal words live in the library's own device array.
        Returns (device address of the signal words, epoch) for the consumer of this launch."""
        sig = C.c_void_p()
        epoch = C.c_uint32()
        _check(lib().fo_gemm_signal_noalloc(
            self._h, _ptr(A, numel=self.M * self.K, itemsize=2, name="A"),
            _ptr(B, numel=self.num_problems * self.N * self.K, itemsize=2, name="B"),
            _ptr(reorder_buf, numel=self.mn, itemsize=2, name="reorder_buf"), C.byref(sig), C.byref(epoch),
            _stream(stream)), "fo_gemm_signal_noalloc")
        return int(sig.value or 0), int(epoch.value)

    def gemm_signal_serialized(self, A, B, reorder_buf, sig, epoch: int, snapshots, stream=None):
        """Debug form with a device-wide barrier after every wave (``fo_gemm_signal_serialized``);
        ``snapshots`` is int32[T*2P + 2], zeroed: row w holds cnt[P] then flag[P] after wave w."""
        _check(lib().fo_gemm_signal_serialized(
            self._h, _ptr(A, numel=self.M * self.K, itemsize=2, name="A"),
            _ptr(B, numel=self.num_problems * self.N * self.K, itemsize=2, name="B"),
            _ptr(reorder_buf, numel=self.mn, itemsize=2, name="reorder_buf"),
            _ptr(sig, numel=self.sig_words, itemsize=4, name="sig"), int(epoch),
            _ptr(snapshots, numel=2 * self.T * self.P + 2, itemsize=4, name="snapshots"), _stream(stream)),
            "fo_gemm_signal_serialized")

    def gemm_plain(self, A, B, Cout, stream=None):
        _check(lib().fo_gemm_plain(
            self._h, _ptr(A, numel=self.M * self.K, itemsize=2, name="A"),
            _ptr(B, numel=self.num_problems * self.N * self.K, itemsize=2, name="B"),
            _ptr(Cout, numel=self.mn, itemsize=2, name="C"), _stream(stream)), "fo_gemm_plain")

    def consume_group(self, send, peer, recv, sig, epoch: int, status, g_begin: int = 0, g_end: Optional[int] = None,
                      timeout_us: int = 0, num_workgroups: int = 0, trace=None, stream=None):
        g_end = self.P if g_end is None else g_end
        _check(lib().fo_consume_group(
            self._h, _ptr(send, numel=self.mn, itemsize=2, name="send"),
            _ptr(peer, numel=self.mn, itemsize=2, name="peer"), _ptr(recv, numel=self.mn, itemsize=2, name="recv"),
            _ptr(sig, numel=self.sig_words, itemsize=4, name="sig"), int(epoch), int(g_begin), int(g_end),
            _ptr(status, numel=1, itemsize=4, name="status"), int(timeout_us), int(num_workgroups),
            _ptr(trace, numel=self.P, itemsize=8, name="trace"), _stream(stream)), "fo_consume_group")

    def consume_group_gated(self, send, peer, recv, sig, epoch: int, status, g_begin: int = 0,
                            g_end: Optional[int] = None, trace=None, stream=None):
        """Consumer gated by a stream wait on each group's flag (``fo_consume_group_gated``)."""
        g_end = self.P if g_end is None else g_end
        _check(lib().fo_consume_group_gated(
            self._h, _ptr(send, numel=self.mn, itemsize=2, name="send"),
            _ptr(peer, numel=self.mn, itemsize=2, name="peer"), _ptr(recv, numel=self.mn, itemsize=2, name="recv"),
            _ptr(sig, numel=self.sig_words, itemsize=4, name="sig"), int(epoch), int(g_begin), int(g_end),
            _ptr(status, numel=1, itemsize=4, name="status"), _ptr(trace, numel=self.P, itemsize=8, name="trace"),
            _stream(stream)), "fo_consume_group_gated")

    def reorder_shards(self, reordered, gathered, stream=None):
        """ReduceScatter plans: every rank's row shard, back to back (``fo_reorder_shards``)."""
        _check(lib().fo_reorder_shards(self._h, _ptr(reordered, numel=self.mn, itemsize=2, name="reordered"),
                                       _ptr(gathered, numel=self.mn, itemsize=2, name="gathered"),
                                       _stream(stream)), "fo_reorder_shards")

    def row_exchange(self, gathered, out, bias=None, act: str = "none", stream=None):
        """Block-cyclic row exchange of the gathered shards into row-major ``out``, fused with bias and
        activation (``fo_row_exchange``)."""
        _check(lib().fo_row_exchange(self._h, _ptr(gathered, numel=self.mn, itemsize=2, name="gathered"),
                                     _ptr(out, numel=self.mn, itemsize=2, name="out"),
                                     _ptr(bias, numel=self.num_problems * self.N, itemsize=2, name="bias"),
                                     _ACTS[act], _stream(stream)), "fo_row_exchange")

    def reorder_post(self, reordered, out, stream=None, groups: Optional[tuple] = None):
        """Inverse mapping into row-major ``out``; ``groups=(g_begin, g_end)`` restricts it to the
        tiles of those groups (``fo_reorder_post_groups``)."""
        src = _ptr(reordered, numel=self.mn, itemsize=2, name="reordered")
        dst = _ptr(out, numel=self.mn, itemsize=2, name="out")
        if groups is None:
            _check(lib().fo_reorder_post(self._h, src, dst, _stream(stream)), "fo_reorder_post")
        else:
            _check(lib().fo_reorder_post_groups(self._h, int(groups[0]), int(groups[1]), src, dst, _stream(stream)),
                   "fo_reorder_post_groups")

    def reorder_post_ep(self, reordered, out, bias=None, act: str = "none", stream=None):
        """Post-communication reorder fused with bias + activation (``fo_reorder_post_ep``)."""
        _check(lib().fo_reorder_post_ep(self._h, _ptr(reordered, numel=self.mn, itemsize=2, name="reordered"),
                                        _ptr(out, numel=self.mn, itemsize=2, name="out"),
                                        _ptr(bias, numel=self.num_problems * self.N, itemsize=2, name="bias"),
                                        _ACTS[act], _stream(stream)), "fo_reorder_post_ep")

    def reorder_pre(self, rowmajor, reordered, stream=None):
        _check(lib().fo_reorder_pre(self._h, _ptr(rowmajor, numel=self.mn, itemsize=2, name="in"),
                                    _ptr(reordered, numel=self.mn, itemsize=2, name="reordered"), _stream(stream)),
               "fo_reorder_pre")

    # ------------------------------------------------------------------ lifetime
    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            lib().fo_plan_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()
