"""Seeded synthetic inputs for the signaling-GEMM workloads.

This module only draws random numbers and rounds them to the 16-bit input
type.  It holds none of the method's arithmetic (no tiling, no swizzle, no
offsets, no GEMM), so both the CPU oracle's tests and the HIP path's tests
and benchmark may take their inputs from it.

Generator: numpy ``Generator(PCG64(seed))``; fp32 draws, rounded to bf16 or
fp16 round-to-nearest-even by torch's dtype conversion.  Seeds are
``10 * workload + {1: A, 2: B, 3: peer, 4: routing}`` (the decode slice of the
all-reduce workload uses 35, 36, 37).

The workloads stand in for the GEMM shapes that the pages profile (the
deep-dive's 背景与动机 › GEMM + 通信模式分析 and the wave-pattern profile of
一 › 关键洞察); no model weights or traces are used, only the shapes.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "draw", "to_bits", "random_bits", "moe_routing", "make_inputs"]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int                       # rows of the (stacked) output
    N: int
    K: int
    dtype: str                   # "bf16" or "fp16"
    dist: Tuple                  # ("uniform", lo, hi) | ("normal", std)
    seed_base: int               # seeds seed_base + 1 (A), + 2 (B), + 3 (peer), + 4 (routing)
    BM: int = 256
    BN: int = 128
    S: int = 4                   # swizzle width
    W: int = 256                 # wave size (tiles resident at once)
    compositions: Tuple = ()     # wave-group partitions to run; () = all
    mode: str = "tile"
    ranks: int = 1
    experts: int = 0             # > 0: grouped GEMM over experts (MoE)
    tokens: int = 0
    topk: int = 0


WORKLOADS = {
    # the pages' worked example, scaled up to a real GEMM
    "tiny": Workload("tiny", 256, 256, 256, "fp16", ("uniform", -1.0, 1.0), 10,
                     BM=64, BN=64, S=2, W=4, compositions=((1, 2, 1),)),
    # the profiled shape of the wave-pattern figure
    "profiled": Workload("profiled", 2048, 8192, 8192, "bf16", ("normal", 1.0 / math.sqrt(8192)), 20,
                         compositions=((2,), (1, 1))),
    # tensor-parallel all-reduce share: Llama3-70B down projection, TP=8
    "ar_prefill": Workload("ar_prefill", 4096, 8192, 3584, "bf16", ("normal", 0.02), 30),
    # S = 2: the two tile rows of a B column are neighbours in dispatch order and so share an XCD,
    # whose L2 then reads that column of B once (with S = 1 they would sit on different XCDs: twice
    # the HBM traffic, 8-10% slower)
    "ar_decode": Workload("ar_decode", 128, 8192, 3584, "bf16", ("normal", 0.02), 34,
                          BM=64, BN=64, S=2),
    # reduce-scatter layout: Llama2-7B TP=4, R = 4 rank segments
    "rs": Workload("rs", 8192, 4096, 2752, "bf16", ("normal", 0.02), 40, mode="subtile", ranks=4),
    # MoE all-to-all: 8 experts, 4096 tokens, top-2, D = 8 destinations
    "moe_a2a": Workload("moe_a2a", 8192, 14336, 4096, "bf16", ("normal", 0.02), 50,
                        mode="subtoken", ranks=8, experts=8, tokens=4096, topk=2,
                        compositions=((1,) * 17, (2,) * 8 + (1,), (4, 4, 4, 5), (8, 9), (17,))),
}


def draw(seed: int, shape, dist) -> np.ndarray:
    """fp32 draws from the workload's distribution."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if dist[0] == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape).astype(np.float32)
    if dist[0] == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
        x *= np.float32(dist[1])
        return x
    if dist[0] == "ternary":
        return rng.integers(-1, 2, size=shape).astype(np.float32)
    raise ValueError(dist)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> uint16 patterns of bf16/fp16 (round to nearest even, via torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    td = torch.bfloat16 if dtype == "bf16" else torch.float16
    return t.to(td).view(torch.int16).numpy().view(np.uint16)


def random_bits(seed: int, n: int, dtype: str) -> np.ndarray:
    """Random finite 16-bit patterns (all exponents), for layout-only checks."""
    rng = np.random.Generator(np.random.PCG64(seed))
    b = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    exp_mask = 0x7F80 if dtype == "bf16" else 0x7C00
    b[(b & exp_mask) == exp_mask] &= np.uint16(0xBFFF)   # clear the top exponent bit: no inf/NaN
    return b


def moe_routing(w: Workload) -> Tuple[List[int], np.ndarray]:
    """Top-k routing of tokens to experts, uniform random scores.

    Scores ``rng.random((tokens, experts))`` from seed ``seed_base + 4``; each
    token goes to its k highest-scoring (distinct) experts.  Output rows are
    sorted by expert, then by ascending token id.  Returns (rows per expert,
    token id of every output row).
    """
    rng = np.random.Generator(np.random.PCG64(w.seed_base + 4))
    scores = rng.random((w.tokens, w.experts))
    top = np.argsort(-scores, axis=1, kind="stable")[:, : w.topk]
    m_per, toks = [], []
    for e in range(w.experts):
        t = np.nonzero((top == e).any(axis=1))[0]
        m_per.append(int(t.size))
        toks.append(t)
    return m_per, np.concatenate(toks).astype(np.int64)


def make_inputs(w: Workload, *, dist=None, M: Optional[int] = None):
    """(A_bits [M, K], list of B_bits [N, K] per problem, peer_bits [M*N], m_per_problem, row_dest).

    ``dist`` overrides the value distribution (e.g. ternary inputs for exact
    checks); ``M`` overrides the row count of a plain GEMM.
    """
    dist = dist or w.dist
    if w.experts:
        m_per, tok = moe_routing(w)
        Mtot = sum(m_per)
        row_dest = (tok // (w.tokens // w.ranks)).astype(np.int64)
        nprob = w.experts
    else:
        Mtot = M if M is not None else w.M
        m_per, row_dest, nprob = [Mtot], None, 1
    A = to_bits(draw(w.seed_base + 1, (Mtot, w.K), dist), w.dtype)
    Ball = to_bits(draw(w.seed_base + 2, (nprob * w.N, w.K), dist), w.dtype)
    B = [Ball[e * w.N:(e + 1) * w.N] for e in range(nprob)]
    peer = to_bits(draw(w.seed_base + 3, (Mtot * w.N,), dist), w.dtype)
    return A, B, peer, m_per, row_dest
