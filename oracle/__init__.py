"""CPU oracle for paged-KV decode attention: TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy restatement of what the paged-attention hot path
computes, written from the pages (not from the GPU code).  It shares no code
with the HIP library or its Python binding, and neither side imports the
other.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package;
the product path never falls back to it.

Sources, cited by page title and section:

* "19.2 KV Cache 系统化管理" (paper.xwysyy.cn, llm-fullstack-book 19_2),
  §19.2.2 (blocks, block table, reference counts, copy-on-write) and §19.2.3
  (the simplified implementation: ``PhysicalBlockPool``, ``BlockTable``,
  ``paged_attention`` with an online softmax, and the check against standard
  attention).
* "LLM 推理引擎的内存管理与调度" (zhouzhq2021.github.io, "LLM serving as an
  operating system"), §3 (block-table address computation), §4 (sharing,
  reference counts, copy-on-write of a shared tail block) and §8 (chunked
  prefill).

Modules:

* :mod:`oracle.allocator` -- block pool mirror: LIFO free list, reference
  counts, fork, append with copy-on-write, release, block tables.
* :mod:`oracle.kvcache` -- slot-mapped cache writes, whole-block copies and
  block swaps between two pools.
* :mod:`oracle.attention` -- attention through the block table (the plain
  definition), split-sequence partials and their log-sum-exp merge.
* :mod:`oracle.quant` -- the e4m3 (FP8) code table and per-token absmax
  quantization of KV rows ("19.2 KV Cache 系统化管理" §19.2.4).

Pins (what each function is checked against, besides itself) are listed in
each module's docstring and exercised by ``tests/test_oracle_*.py``.
"""

from .allocator import OracleBlockPool, OracleNoFreeBlocks  # noqa: F401
from .kvcache import kv_write, copy_blocks, swap_blocks  # noqa: F401
from .quant import e4m3_decode, e4m3_encode, quantize_rows, dequantize, kv_write_fp8  # noqa: F401
from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    paged_attention,
    paged_attention_query,
    split_partials,
    merge_partials,
    query_positions,
)
