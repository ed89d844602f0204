"""Helpers for the GPU tests: device buffers from seeded host arrays, tolerance checks.

Inputs come from ``workloads`` (seeded, synthetic); expected values come from
``oracle`` applied to the same host arrays.  Nothing here computes any part of
the method.
"""

from __future__ import annotations

import sys

import numpy as np

import oracle


def say(msg: str):
    """Name the case before a GPU step, flushed, so a failure can be located."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).to("cuda")


def to_host(t) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def empty16(n: int, fill: int = 0x7FC0):
    """A device buffer of n 16-bit elements pre-filled with a marker pattern (a NaN)."""
    import torch
    return torch.full((n,), np.int16(np.uint16(fill).view(np.int16)), dtype=torch.int16, device="cuda")


def zeros_i32(n: int):
    import torch
    return torch.zeros(n, dtype=torch.int32, device="cuda")


def tol_check(gpu_bits, ref_f64, dtype: str, what: str):
    """|gpu - oracle| <= 1e-2 * max(1, |oracle|) element by element; returns the diagnostic ratio."""
    g = oracle.decode_bits(gpu_bits, dtype)
    r = np.asarray(ref_f64, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values in the GPU result"
    err = np.abs(g - r)
    bound = 1e-2 * np.maximum(1.0, np.abs(r))
    bad = err > bound
    if bad.any():
        i = int(np.argmax(bad.ravel()))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at flat index {i}: "
                             f"gpu {g.ravel()[i]!r} oracle {r.ravel()[i]!r}")
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    return float(err.max() / rms) if rms > 0 and err.size else 0.0


def tol_check_out(gpu_bits, want_out, c_ref, dtype: str, what: str):
    """Tolerance for out = round(C + peer), derived from the GEMM's.

    The GEMM output C may differ from the oracle by up to
    tol_C = 1e-2 * max(1, |C|); the consumer adds peer exactly and rounds
    once on each side, so |out_gpu - out_oracle| <= tol_C + 2^(1-p) * (|out| + tol_C)
    with p the significand bits of the type.  Cancellation in C + peer is why
    the bound follows |C| and not |out|.
    """
    p = oracle.DTYPES[dtype]["p"]
    g = oracle.decode_bits(gpu_bits, dtype)
    r = np.asarray(want_out, dtype=np.float64)
    c = np.asarray(c_ref, dtype=np.float64)
    assert g.shape == r.shape == c.shape, (what, g.shape, r.shape, c.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values in the GPU result"
    tol_c = 1e-2 * np.maximum(1.0, np.abs(c))
    bound = tol_c + 2.0 ** (1 - p) * (np.abs(r) + tol_c)
    bad = np.abs(g - r) > bound
    if bad.any():
        i = int(np.argmax(bad.ravel()))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the derived bound; first at {i}: "
                             f"gpu {g.ravel()[i]!r} oracle {r.ravel()[i]!r} C {c.ravel()[i]!r}")


def ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Distance in units of the last place between two arrays of bf16/fp16 patterns.

    Both types order their finite values by the sign-magnitude integer of the
    pattern, so adjacent values differ by one; +0 and -0 are the same point.
    """
    def key(x):
        x = np.asarray(x, dtype=np.uint16).astype(np.int64)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(key(a_bits) - key(b_bits))
