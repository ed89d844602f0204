"""ReduceScatter + AllGather: rank shards and the row exchange (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Method: deep-dive 二、重排机制 › 不同通信原语的重排模式, (2) ReduceScatter +
AllGather.  Every tile is cut along its rows into as many equal pieces as
there are ranks; whatever rank computed a tile, piece k of it ends up on
rank k, so the k-th pieces of all tiles are whole output rows.  An AllGather
then collects every rank's rows, and a local row exchange -- a block-cyclic
permutation, with no mapping table, which can run in the same pass as the
element-wise operations -- brings the rows back into their order.

Readings (the pages give no formula):

* rank k owns the rows whose piece inside their tile is k: a row with index
  r inside its tile (problems start at multiples of BM in this mode) belongs
  to rank floor(r / (BM/R));
* after the ReduceScatter rank k keeps its rows as one row-major shard in
  increasing row order -- its "complete rows";
* the AllGather concatenates the shards in rank order;
* the row exchange is the permutation that returns the gathered rows to row
  order; the element-wise epilogue is the post-communication one
  (``oracle.epilogue``), applied after the exchange.
"""

from __future__ import annotations

import numpy as np

from .epilogue import post_epilogue
from .layout import post_reorder
from .tiles import Plan


def _require_subtile(plan: Plan):
    if plan.mode != "subtile":
        raise ValueError("the row exchange belongs to the ReduceScatter layout")


def row_owner(plan: Plan) -> np.ndarray:
    """Rank that holds each output row after the ReduceScatter (length M)."""
    _require_subtile(plan)
    band = plan.BM // plan.ranks
    owner = np.empty(plan.M, dtype=np.int64)
    start = 0
    for m in plan.m_per_problem:
        r = np.arange(m, dtype=np.int64) % plan.BM        # row inside its tile
        owner[start:start + m] = r // band
        start += m
    return owner


def gathered_rows(plan: Plan) -> np.ndarray:
    """G[g] = the output row at position g of the gathered buffer: rank 0's rows
    in increasing order, then rank 1's, and so on."""
    owner = row_owner(plan)
    return np.concatenate([np.nonzero(owner == k)[0] for k in range(plan.ranks)]).astype(np.int64)


def gathered_offsets(plan: Plan) -> np.ndarray:
    """goff[m, n]: where output element (m, n) sits in the gathered buffer."""
    G = gathered_rows(plan)
    pos = np.empty(plan.M, dtype=np.int64)
    pos[G] = np.arange(plan.M, dtype=np.int64)
    return pos[:, None] * plan.N + np.arange(plan.N, dtype=np.int64)[None, :]


def shard_reorder(recv_bits, off, plan: Plan) -> np.ndarray:
    """The gathered buffer (flat M*N) built from the consumer's result in the
    reordered layout: every rank's shard rows, taken through the mapping
    table's element offsets ``off``, shards back to back."""
    G = gathered_rows(plan)
    recv = np.asarray(recv_bits).ravel()
    return recv[np.asarray(off)[G]].ravel()


def row_exchange(gathered_bits, plan: Plan) -> np.ndarray:
    """Row-major [M, N] output from the gathered buffer."""
    return post_reorder(np.asarray(gathered_bits).ravel(), gathered_offsets(plan))


def row_exchange_epilogue(gathered_bits, plan: Plan, dtype: str, act: str = "none", bias_bits=None,
                          row_problem=None) -> np.ndarray:
    """The row exchange with bias and activation, one rounding: 16-bit patterns, [M, N]."""
    return post_epilogue(gathered_bits, gathered_offsets(plan), dtype, act, bias_bits, row_problem)
