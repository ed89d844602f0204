"""Mapping table, reorder offsets and the two reorders (oracle, test infrastructure only).

Written from the deep-dive page "FlashOverlap: 信号驱动计算通信重叠论文详解",
二、重排机制:

* 解决方案: 映射表重排 -- a mapping table sends the scattered tile indices of
  a finished group to consecutive reorder indices; pre-communication
  reordering writes through it, post-communication reordering applies the
  inverse;
* 不同通信原语的重排模式 (and Figure 6) -- (1) AllReduce reorders whole
  tiles; (2) ReduceScatter cuts each tile along rows into one piece per
  rank, and piece k always goes to rank k, so all k-th pieces together are
  complete rows; (3) All-to-All cuts each tile's output by destination rank
  and makes the pieces for one rank contiguous;
* the code box under 二 shows the execution order [t0, t3, t1, t2] sent to
  reorder indices 0, 1, 2, 3 and back.

Readings:

* reorder indices ("slots") follow dispatch order, so each group occupies a
  consecutive run of slots;
* inside a tile, data is row-major with the tile's own row length; edge
  tiles are packed (only their valid rows and columns), so the reordered
  buffer has exactly M x N elements;
* ReduceScatter pieces are bands of BM/R rows; a group's span is laid out
  rank-major: rank k's segment holds the k-th band of every tile of the
  group, in slot order;
* All-to-All pieces are single tile rows ("subtokens"); a group's span is
  laid out destination-major; inside destination d the order is slot order,
  then row order inside the tile.
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np

from .tiles import Plan


def mapping_table(plan: Plan) -> Tuple[List[int], List[int]]:
    """(slot_of_tile, tile_of_slot): the mapping table and its inverse.

    Slot s holds the tile dispatched at index b = s.
    """
    tile_of_slot = list(plan.tile_of_b)
    slot_of_tile = [0] * plan.NT
    for s, t in enumerate(tile_of_slot):
        slot_of_tile[t] = s
    return slot_of_tile, tile_of_slot


def _group_slots(plan: Plan) -> List[List[int]]:
    slots = [[] for _ in range(plan.P)]
    for s in range(plan.NT):
        slots[plan.group_of_b[s]].append(s)
    return slots


def _tile_size(plan: Plan, t: int) -> int:
    return plan.tile_rows[t] * plan.tile_cols[t]


def group_spans(plan: Plan) -> List[int]:
    """P+1 element offsets: group j's contiguous span is [span[j], span[j+1])."""
    spans = [0]
    for j, slots in enumerate(_group_slots(plan)):
        spans.append(spans[-1] + sum(_tile_size(plan, plan.tile_of_b[s]) for s in slots))
    return spans


def row_offsets(plan: Plan) -> List[np.ndarray]:
    """For every slot s, the reordered offset of the first element of each tile row.

    Element (r, c) of the tile at slot s lands at ``row_offsets(plan)[s][r] + c``.
    """
    _, tile_of_slot = mapping_table(plan)
    spans = group_spans(plan)
    out: List[np.ndarray] = [None] * plan.NT
    for j, slots in enumerate(_group_slots(plan)):
        if plan.mode == "tile":
            pos = spans[j]
            for s in slots:
                t = tile_of_slot[s]
                rows, cols = plan.tile_rows[t], plan.tile_cols[t]
                out[s] = pos + cols * np.arange(rows, dtype=np.int64)
                pos += rows * cols
        elif plan.mode == "subtile":
            R, BM, BN = plan.ranks, plan.BM, plan.BN
            band = BM // R
            q = band * BN
            n_j = len(slots)
            for i, s in enumerate(slots):
                r = np.arange(BM, dtype=np.int64)
                k, rr = r // band, r % band
                out[s] = spans[j] + k * n_j * q + i * q + rr * BN
        else:  # subtoken
            D = plan.ranks
            per = {s: np.zeros(plan.tile_rows[tile_of_slot[s]], dtype=np.int64) for s in slots}
            pos = spans[j]
            for d in range(D):
                for s in slots:
                    t = tile_of_slot[s]
                    cols = plan.tile_cols[t]
                    r0 = plan.tile_row0[t]
                    dest = plan.row_dest[r0:r0 + plan.tile_rows[t]]
                    rows_d = np.nonzero(dest == d)[0]          # ascending row order
                    per[s][rows_d] = pos + cols * np.arange(len(rows_d), dtype=np.int64)
                    pos += cols * len(rows_d)
            for s in slots:
                out[s] = per[s]
            assert pos == spans[j + 1]
    return out


def element_offsets(plan: Plan) -> np.ndarray:
    """off[m, n]: where output element (m, n) sits in the reordered buffer."""
    off = np.full((plan.M, plan.N), -1, dtype=np.int64)
    _, tile_of_slot = mapping_table(plan)
    for s, ro in enumerate(row_offsets(plan)):
        t = tile_of_slot[s]
        r0, c0, cols = plan.tile_row0[t], plan.tile_col0[t], plan.tile_cols[t]
        off[r0:r0 + len(ro), c0:c0 + cols] = ro[:, None] + np.arange(cols, dtype=np.int64)[None, :]
    return off


def consumer_units(plan: Plan) -> List[List[Tuple[int, int]]]:
    """Per group, the [lo, hi) element ranges handed to one collective call each.

    AllReduce: the whole group span.  ReduceScatter: R rank segments of
    n_j * (BM/R) * BN elements.  All-to-All: D destination segments (some may
    be empty).
    """
    spans = group_spans(plan)
    units = []
    for j, slots in enumerate(_group_slots(plan)):
        lo, hi = spans[j], spans[j + 1]
        if plan.mode == "tile":
            units.append([(lo, hi)])
        elif plan.mode == "subtile":
            seg = len(slots) * (plan.BM // plan.ranks) * plan.BN
            units.append([(lo + k * seg, lo + (k + 1) * seg) for k in range(plan.ranks)])
        else:
            sizes = [0] * plan.ranks
            for s in slots:
                t = plan.tile_of_b[s]
                r0 = plan.tile_row0[t]
                dest = plan.row_dest[r0:r0 + plan.tile_rows[t]]
                for d in range(plan.ranks):
                    sizes[d] += plan.tile_cols[t] * int(np.count_nonzero(dest == d))
            segs, pos = [], lo
            for d in range(plan.ranks):
                segs.append((pos, pos + sizes[d]))
                pos += sizes[d]
            assert pos == hi
            units.append(segs)
    return units


def pre_reorder(X, off) -> np.ndarray:
    """Pre-communication reordering: flat[off[m, n]] = X[m, n]."""
    X = np.asarray(X)
    flat = np.empty(X.size, dtype=X.dtype)
    flat[off.ravel()] = X.ravel()
    return flat


def post_reorder(flat, off) -> np.ndarray:
    """Post-communication reordering: X[m, n] = flat[off[m, n]]."""
    return np.asarray(flat)[off]
