"""Floating-point steps of the path, in fp64, for the oracle (test infrastructure only).

The pages fix no precision for the GEMM or for the data that the collective
moves.  Readings:

* the GEMM's inputs and output are in the model's 16-bit type (bf16 or fp16)
  and the product is accumulated in high precision; the oracle accumulates in
  fp64 and rounds once to the 16-bit type, round-to-nearest-even;
* the one-GPU stand-in for a group's collective adds a second buffer of the
  same type element by element and rounds the exact sum once,
  round-to-nearest-even.  (The sum of two 16-bit values rounded once is what
  an fp32 add followed by a rounding to 16 bits gives as well; the tests pin
  this.)

Rounding is written from the IEEE-754 definition: scale the value onto the
integer grid of its binade, round half to even, scale back, and send values
past the largest finite number to infinity.
"""

from __future__ import annotations

import numpy as np

# significand bits including the hidden one, smallest normal exponent, largest
# finite value.  IEEE-754 binary16 and the bfloat16 truncation of binary32.
DTYPES = {
    "bf16": dict(p=8, emin=-126, emax=127),
    "fp16": dict(p=11, emin=-14, emax=15),
}


def _max_finite(dtype: str) -> float:
    d = DTYPES[dtype]
    return float(np.ldexp(2.0 - 2.0 ** (1 - d["p"]), d["emax"]))


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round fp64 values to the nearest ``dtype`` value, ties to even.

    Returns fp64 values that are exactly representable in ``dtype``; zeros,
    infinities and NaNs pass through, and finite values whose rounding leaves
    the finite range become infinities of their sign.
    """
    d = DTYPES[dtype]
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)                      # |xf| in [2**(e-1), 2**e)
    # exponent of one unit in the last place: normal numbers carry p bits;
    # below the normal range the grid spacing stays at the subnormal spacing.
    ulp_e = np.maximum(e, d["emin"] + 1) - d["p"]
    y = np.ldexp(np.rint(np.ldexp(xf, -ulp_e)), ulp_e)   # rint: half to even
    big = np.abs(y) > _max_finite(dtype)
    y[big] = np.copysign(np.inf, y[big])
    out[fin] = y
    return out


def decode_bits(bits, dtype: str) -> np.ndarray:
    """16-bit patterns (uint16) -> fp64 values, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        if dtype == "bf16":
            return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        if dtype == "fp16":
            return b.view(np.float16).astype(np.float64)
    raise ValueError(dtype)


def encode_bits(values, dtype: str) -> np.ndarray:
    """fp64 values already representable in ``dtype`` -> uint16 patterns."""
    v = np.asarray(values, dtype=np.float64)
    if dtype == "bf16":
        f = v.astype(np.float32)              # exact: bf16 values are fp32 values
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    if dtype == "fp16":
        return v.astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


def gemm_fp64(A, B) -> np.ndarray:
    """C = A . B with A [M, K] and the logical B [K, N], accumulated in fp64.

    The GEMM itself is the untouched core of the method: the deep-dive's
    compute side (核心设计 › 计算侧) keeps it one kernel whose arithmetic the
    signaling does not change.  Reading: A is row-major [M, K]; B is the
    logical [K, N] operand (how the GPU stores it is the GPU's business).
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch {A.shape} x {B.shape}")
    return A @ B


def consume_add(send_bits, peer_bits, dtype: str) -> np.ndarray:
    """One-GPU stand-in for a group's collective: round(send + peer) per element.

    The deep-dive's communication side (核心设计 › 通信侧, 二 › (1) AllReduce)
    hands each group's contiguous span to an all-reduce; on one GPU the span
    is reduced with a second buffer of the same layout.  Inputs and output are
    16-bit patterns.
    """
    s = decode_bits(send_bits, dtype)
    p = decode_bits(peer_bits, dtype)
    return encode_bits(round_to_dtype(s + p, dtype), dtype)
