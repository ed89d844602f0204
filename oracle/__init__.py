"""CPU oracle for the signaling GEMM with tile reordering (FlashOverlap hot path).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no tables, helpers, headers or constants) and imports nothing from it.

Sources.  Two web pages describe the method; they are cited by title and
section:

* the deep-dive page "FlashOverlap: 信号驱动计算通信重叠论文详解"
  (cited as *deep-dive*, with its section headings: 一、信号机制,
  二、重排机制, 三、Wave Group 划分设计空间, 四、实时调优, 五、CUTLASS 扩展实现);
* the summary page "Efficient and Adaptable Overlapping for Computation and
  Communication via Signaling and Reordering" (cited as *summary*: its
  abstract and figure captions).

Where the pages leave a step open, the oracle takes one plain reading; each
reading is named in the docstring of the function that takes it.

Modules
-------
``numerics``  rounding to bf16/fp16, the fp64 GEMM, the consumer's add.
``tiles``     tile grid, swizzled dispatch order, waves, wave groups, the
              partition design space and the counting-table trajectory.
``layout``    mapping table and its inverse, element offsets for the three
              reorder patterns, pre- and post-communication reordering.
``pipeline``  the whole path end to end, and single-output sampling for
              full-size checks.
``rowexchange`` the ReduceScatter + AllGather pattern: every rank's row shard
              and the block-cyclic row exchange after the AllGather.
``search``    the predictive wave-group partition search.
``epilogue``  the post-communication reorder with bias and activation.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against the pages' worked examples, closed forms, invariants or brute force.
"""

from .numerics import (
    DTYPES,
    round_to_dtype,
    decode_bits,
    encode_bits,
    gemm_fp64,
    consume_add,
)
from .tiles import (
    Plan,
    make_plan,
    swizzle_order,
    enumerate_compositions,
    composition_to_mask,
    mask_to_composition,
    counting_trajectory,
)
from .layout import (
    mapping_table,
    element_offsets,
    row_offsets,
    pre_reorder,
    post_reorder,
    consumer_units,
)
from .pipeline import run_pipeline, sample_outputs

__all__ = [
    "DTYPES", "round_to_dtype", "decode_bits", "encode_bits", "gemm_fp64",
    "consume_add", "Plan", "make_plan", "swizzle_order",
    "enumerate_compositions", "composition_to_mask", "mask_to_composition",
    "counting_trajectory", "mapping_table", "element_offsets", "row_offsets",
    "pre_reorder", "post_reorder", "consumer_units", "run_pipeline",
    "sample_outputs",
]
