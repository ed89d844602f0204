"""Post-communication reordering fused with the element-wise epilogue (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Method: deep-dive 五、CUTLASS 扩展实现 › Epilogue 集成 -- the element-wise
operations that normally follow a GEMM (bias addition, ReLU, SiLU) are
applied in the same pass as the post-communication reorder, so the output
is written once, row-major, already activated.

Definition (readings: the bias is one row of N values per problem, the row's
problem selecting it; the activation acts on the biased value; one rounding
to the element type at the end):

    out[m, n] = round( act( recv[off[m, n]] + bias[problem(m), n] ) )

with act(x) = x, max(x, 0) or x / (1 + exp(-x)) (SiLU), evaluated in fp64.
"""

from __future__ import annotations

import numpy as np

from .layout import post_reorder
from .numerics import decode_bits, encode_bits, round_to_dtype

ACTS = ("none", "relu", "silu")


def activation(x, act: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if act == "none":
        return x
    if act == "relu":
        return np.where(x > 0, x, 0.0)
    if act == "silu":
        with np.errstate(over="ignore"):
            return x / (1.0 + np.exp(-x))
    raise ValueError(act)


def post_epilogue(recv_bits, off, dtype: str, act: str = "none", bias_bits=None, row_problem=None) -> np.ndarray:
    """16-bit patterns of the row-major, biased and activated output, [M, N]."""
    off = np.asarray(off)
    M, N = off.shape
    x = decode_bits(post_reorder(np.asarray(recv_bits, dtype=np.uint16), off), dtype)
    if bias_bits is not None:
        b = decode_bits(np.asarray(bias_bits, dtype=np.uint16), dtype).reshape(-1, N)
        rp = np.zeros(M, dtype=np.int64) if row_problem is None else np.asarray(row_problem, dtype=np.int64)
        x = x + b[rp]                                  # exact: a sum of two 16-bit values fits fp64
    return encode_bits(round_to_dtype(activation(x, act), dtype), dtype)


def row_problems(plan) -> np.ndarray:
    """Problem index of every output row (problems stack their rows in order)."""
    return np.repeat(np.arange(len(plan.m_per_problem)), plan.m_per_problem)
