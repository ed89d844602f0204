"""The whole path on the CPU, and single outputs for full-size checks (oracle, test only).

Order of the steps follows the system overview of the deep-dive page
"FlashOverlap: 信号驱动计算通信重叠论文详解" (核心设计 › 系统总览) and Figure 5
of the summary page: the GEMM runs as one computation; when a group of tiles
is done its tiles are reordered into a contiguous span and the group is
signalled; the span is communicated; afterwards the tiles are reordered back.

Operands.  ``A_bits`` is the [M, K] row-major left operand (all problems'
rows stacked for a grouped GEMM).  ``B_bits`` is a list with one stored
right operand per problem, each [N, K] (K contiguous, the layout of a
linear layer's weight); the logical operand of the product is its
transpose, so C = A . B_stored^T.  ``peer_bits`` is the second buffer of
the consumer, flat M*N, in the reordered layout (it stands in for a peer's
identically reordered span).  All bit arrays are uint16 patterns of
``dtype``.
"""

from __future__ import annotations

import time
from typing import Dict, List, Optional

import numpy as np

from .layout import consumer_units, element_offsets, mapping_table, pre_reorder, post_reorder, row_offsets
from .numerics import consume_add, decode_bits, encode_bits, gemm_fp64, round_to_dtype
from .tiles import Plan, counting_trajectory


def _problem_rows(plan: Plan) -> List[int]:
    starts, pos = [], 0
    for m in plan.m_per_problem:
        starts.append(pos)
        pos += m
    return starts


def run_pipeline(A_bits, B_bits: List[np.ndarray], peer_bits, plan: Plan, dtype: str,
                 stage_seconds: Optional[Dict[str, float]] = None) -> Dict:
    """Every intermediate of the path for one batch.

    Returns C64 (fp64 product), C (rounded bits, row-major), off (element
    offsets), send (pre-reordered C), recv (consumer result, flat), out
    (post-reordered recv, row-major), the counting-table trajectory and the
    fire waves, the mapping tables and the consumer units.  ``stage_seconds``,
    if given, receives the wall time of each stage (gemm, offsets, pre_reorder,
    consume, post_reorder, tables); it changes nothing else.
    """
    clock = [time.perf_counter()]

    def lap(name):
        now = time.perf_counter()
        if stage_seconds is not None:
            stage_seconds[name] = stage_seconds.get(name, 0.0) + now - clock[0]
        clock[0] = now

    A = decode_bits(A_bits, dtype)
    if len(B_bits) != len(plan.m_per_problem):
        raise ValueError("one B per problem")
    C64 = np.zeros((plan.M, plan.N))
    for e, r0 in enumerate(_problem_rows(plan)):
        m = plan.m_per_problem[e]
        Be = decode_bits(B_bits[e], dtype)          # stored [N, K]
        C64[r0:r0 + m] = gemm_fp64(A[r0:r0 + m], Be.T)
    C = encode_bits(round_to_dtype(C64, dtype), dtype)
    lap("gemm")
    off = element_offsets(plan)
    lap("offsets")
    send = pre_reorder(C, off)
    lap("pre_reorder")
    recv = send.copy()
    units = consumer_units(plan)
    peer = np.asarray(peer_bits, dtype=np.uint16).ravel()
    for group in units:                       # groups in firing order
        for lo, hi in group:
            recv[lo:hi] = consume_add(send[lo:hi], peer[lo:hi], dtype)
    lap("consume")
    out = post_reorder(recv, off)
    lap("post_reorder")
    snaps, fire = counting_trajectory(plan)
    slot_of_tile, tile_of_slot = mapping_table(plan)
    lap("tables")
    return dict(C64=C64, C=C, off=off, send=send, recv=recv, out=out,
                snapshots=snaps, fire_wave=fire, slot_of_tile=slot_of_tile,
                tile_of_slot=tile_of_slot, units=units)


def offset_of(plan: Plan, ro: List[np.ndarray], slot_of_tile: List[int], m: int, n: int) -> int:
    """Reordered offset of output element (m, n), found by locating its tile."""
    starts = _problem_rows(plan)
    e = max(i for i, s in enumerate(starts) if s <= m and plan.m_per_problem[i] > 0 and m < s + plan.m_per_problem[i])
    tn_n = -(-plan.N // plan.BN)
    first = sum(-(-mm // plan.BM) * tn_n for mm in plan.m_per_problem[:e])
    tm, r = divmod(m - starts[e], plan.BM)
    tn, c = divmod(n, plan.BN)
    t = first + tm * tn_n + tn
    return int(ro[slot_of_tile[t]][r] + c)


def sample_outputs(A_bits, B_bits: List[np.ndarray], peer_bits, plan: Plan, dtype: str,
                   rows, cols) -> Dict:
    """C64, C and out at the sampled elements (rows[i], cols[i]), one by one.

    For full-size shapes where the whole product is too slow on the CPU:
    each sampled element is one fp64 dot product of an A row with a B row.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    starts = _problem_rows(plan)
    ro = row_offsets(plan)
    slot_of_tile, _ = mapping_table(plan)
    peer = np.asarray(peer_bits, dtype=np.uint16).ravel()
    c64 = np.empty(rows.size)
    offs = np.empty(rows.size, dtype=np.int64)
    for i, (m, n) in enumerate(zip(rows.tolist(), cols.tolist())):
        e = max(k for k, s in enumerate(starts) if s <= m and m < s + plan.m_per_problem[k])
        a = decode_bits(A_bits[m], dtype)
        b = decode_bits(B_bits[e][n], dtype)
        c64[i] = float(np.dot(a, b))
        offs[i] = offset_of(plan, ro, slot_of_tile, m, n)
    C = encode_bits(round_to_dtype(c64, dtype), dtype)
    out = consume_add(C, peer[offs], dtype)
    return dict(C64=c64, C=C, off=offs, out=out)
