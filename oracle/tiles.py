"""Tile grid, dispatch order, waves, wave groups, design space, counting table.

Oracle, test infrastructure only.  Written from the deep-dive page
"FlashOverlap: 信号驱动计算通信重叠论文详解":

* 一、信号机制 › 关键洞察 (waves: tiles that finish together, as many as the
  GPU runs at once; the wave count is tiles / processors);
* 一 › Block Swizzling 的影响 (tiles are handed to processors in an
  interleaved order, so one wave's tiles are scattered in memory);
* 一 › Wave Group 设计 (a group is one or more consecutive waves);
* 一 › 实现方法: 组级 Tile 计数 (a counting table of P entries, one atomic
  increment per finished tile, group j starts communicating when its entry
  reaches |G_j|; the worked example with 8 tiles in 4 waves);
* 三、Wave Group 划分设计空间 › 设计空间大小 (after every wave but the last
  one may communicate or not: 2^(T-1) partitions).

Readings where the pages are silent:

* swizzle: grouped-M order of width S (bands of S tile rows, walked column
  by column inside a band); S = 1 is row-major order;
* a wave is W consecutive dispatch indices, W the number of tiles resident at
  once; T = ceil(NT / W), so only the last wave may be partial;
* partitions are counted in waves, thresholds |G_j| in tiles;
* a grouped (MoE) GEMM is several problems sharing N and K; their tile grids
  are concatenated in problem order and the swizzle runs inside each grid.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np


def swizzle_order(tm_n: int, tn_n: int, S: int) -> List[int]:
    """Dispatch index b -> row-major tile index, grouped-M swizzle of width S.

    Tile rows are cut into bands of S rows (the last band may be shorter,
    height h).  Inside a band the dispatch walks down a column of h tiles,
    then moves to the next column.
    """
    if S < 1:
        raise ValueError("swizzle width must be >= 1")
    order = []
    for b in range(tm_n * tn_n):
        band, loc = divmod(b, S * tn_n)
        h = min(S, tm_n - band * S)
        tm = band * S + loc % h
        tn = loc // h
        order.append(tm * tn_n + tn)
    return order


def enumerate_compositions(T: int) -> List[tuple]:
    """All wave-group partitions of T waves: one per subset of the T-1 cut points.

    Deep-dive 三 › 设计空间大小: after each of the first T-1 waves the choice is
    to communicate or not; the last wave always communicates.
    """
    if T < 1:
        raise ValueError("T must be >= 1")
    out = []
    for mask in range(1 << (T - 1)):
        out.append(mask_to_composition(mask, T))
    return out


def mask_to_composition(mask: int, T: int) -> tuple:
    """Bit i of ``mask`` set = communicate after wave i+1 (waves counted from 1)."""
    sizes, run = [], 0
    for w in range(T):
        run += 1
        last = w == T - 1
        if last or (mask >> w) & 1:
            sizes.append(run)
            run = 0
    return tuple(sizes)


def composition_to_mask(comp: Sequence[int]) -> int:
    mask, pos = 0, 0
    for c in comp[:-1]:
        pos += c
        mask |= 1 << (pos - 1)
    return mask


@dataclass
class Plan:
    """Everything the oracle derives from a problem description.

    Shapes: ``m_per_problem`` rows per problem (one entry for a plain GEMM),
    shared N; tiles BM x BN; swizzle width S; wave size W; composition of the
    T waves into P groups; reorder ``mode`` in {"tile", "subtile",
    "subtoken"} with ``ranks`` (R or D) and, for "subtoken", the destination
    of every output row.
    """

    m_per_problem: List[int]
    N: int
    BM: int
    BN: int
    S: int
    W: int
    composition: tuple
    mode: str = "tile"
    ranks: int = 1
    row_dest: Optional[np.ndarray] = None
    # derived
    M: int = 0
    NT: int = 0
    T: int = 0
    P: int = 0
    tile_of_b: List[int] = field(default_factory=list)
    tile_rows: List[int] = field(default_factory=list)    # valid rows of tile t
    tile_cols: List[int] = field(default_factory=list)
    tile_row0: List[int] = field(default_factory=list)    # first output row
    tile_col0: List[int] = field(default_factory=list)
    tile_problem: List[int] = field(default_factory=list)
    wave_of_b: List[int] = field(default_factory=list)
    group_of_b: List[int] = field(default_factory=list)
    group_of_wave: List[int] = field(default_factory=list)
    group_tiles: List[int] = field(default_factory=list)  # |G_j| in tiles


def make_plan(m_per_problem, N, BM, BN, S, W, composition=None, mode="tile",
              ranks=1, row_dest=None, dispatch_order=None) -> Plan:
    """Build the tile grid, dispatch order, waves and groups.

    ``composition`` None means one wave per group (the finest partition).
    ``dispatch_order`` overrides the swizzle with an explicit b -> tile list
    (used to replay the pages' mapping example).
    """
    if isinstance(m_per_problem, int):
        m_per_problem = [m_per_problem]
    m_per_problem = [int(m) for m in m_per_problem]
    if N <= 0 or BM <= 0 or BN <= 0 or W <= 0 or any(m < 0 for m in m_per_problem):
        raise ValueError("bad sizes")
    tn_n = -(-N // BN)
    tile_rows, tile_cols, tile_row0, tile_col0, tile_problem = [], [], [], [], []
    tile_of_b = []
    row_base = 0
    for e, m in enumerate(m_per_problem):
        tm_n = -(-m // BM)
        first = len(tile_rows)
        for tm in range(tm_n):
            for tn in range(tn_n):
                tile_rows.append(min(BM, m - tm * BM))
                tile_cols.append(min(BN, N - tn * BN))
                tile_row0.append(row_base + tm * BM)
                tile_col0.append(tn * BN)
                tile_problem.append(e)
        tile_of_b += [first + t for t in swizzle_order(tm_n, tn_n, S)] if tm_n else []
        row_base += m
    NT = len(tile_rows)
    if dispatch_order is not None:
        if sorted(dispatch_order) != list(range(NT)):
            raise ValueError("dispatch_order must be a permutation of the tiles")
        tile_of_b = list(dispatch_order)
    T = -(-NT // W) if NT else 0
    if composition is None:
        composition = tuple([1] * T)
    composition = tuple(int(c) for c in composition)
    if any(c < 1 for c in composition) or sum(composition) != T:
        raise ValueError(f"composition {composition} is not a partition of T={T} waves")
    group_of_wave = []
    for j, c in enumerate(composition):
        group_of_wave += [j] * c
    wave_of_b = [b // W for b in range(NT)]
    group_of_b = [group_of_wave[w] for w in wave_of_b]
    P = len(composition)
    group_tiles = [group_of_b.count(j) for j in range(P)]
    if mode not in ("tile", "subtile", "subtoken"):
        raise ValueError(mode)
    M = sum(m_per_problem)
    if mode == "subtile":
        if BM % ranks or any(m % BM for m in m_per_problem) or N % BN:
            raise ValueError("subtile mode needs full tiles and BM divisible by R")
    if mode == "subtoken":
        if row_dest is None or len(row_dest) != M:
            raise ValueError("subtoken mode needs one destination per output row")
        row_dest = np.asarray(row_dest, dtype=np.int64)
        if row_dest.size and (row_dest.min() < 0 or row_dest.max() >= ranks):
            raise ValueError("row destination out of range")
    return Plan(m_per_problem=m_per_problem, N=N, BM=BM, BN=BN, S=S, W=W,
                composition=composition, mode=mode, ranks=ranks, row_dest=row_dest,
                M=M, NT=NT, T=T, P=P, tile_of_b=tile_of_b, tile_rows=tile_rows,
                tile_cols=tile_cols, tile_row0=tile_row0, tile_col0=tile_col0,
                tile_problem=tile_problem, wave_of_b=wave_of_b, group_of_b=group_of_b,
                group_of_wave=group_of_wave, group_tiles=group_tiles)


def counting_trajectory(plan: Plan):
    """Counting table after each wave, and the wave at which each group fires.

    Idealised schedule: every tile of wave w finishes before any tile of wave
    w+1.  Each finished tile adds one to its group's entry; group j fires the
    first time its entry equals |G_j| (deep-dive 一 › 组级 Tile 计数).
    Returns (snapshots: list of P-lists, one per wave; fire_wave: list of P).
    """
    cnt = [0] * plan.P
    snaps, fire = [], [None] * plan.P
    for w in range(plan.T):
        for b in range(plan.NT):
            if plan.wave_of_b[b] == w:
                cnt[plan.group_of_b[b]] += 1
        snaps.append(list(cnt))
        for j in range(plan.P):
            if fire[j] is None and cnt[j] == plan.group_tiles[j]:
                fire[j] = w
    return snaps, fire
