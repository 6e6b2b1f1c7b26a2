"""CPU oracle for paged decode and prefill attention, the slot-mapped cache write, the CoW block copy and block swap.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (``paged_kv_cache_159_amd``: HIP kernels, C-ABI library and its
Python binding) never imports it, and this package imports nothing from the
product path. The two share no code; only the seeded input generators in
``workloads/`` feed both.

Everything here is plain numpy: gathers by fancy indexing, a matrix-vector
product, ``exp`` and sums, all in float64. No blocking, fusion or reordering
beyond what each function's docstring states.

Pages cited (title, address):
  [P1] "3.3 页面级显存管理" (page-level GPU memory management),
       aiknowledge.cn/article/68056
  [P2] "vLLM三大核心技术分页内存与共享解码" (the three core vLLM techniques),
       aiqz.cc/article/vllm-core-techniques.html
  [P3] "3.1 PagedAttention的核心原理" (core principle of PagedAttention),
       aiknowledge.cn/article/68054
  [P4] reading notes on "vLLM: Easy, Fast, and Cheap LLM Serving with
       PagedAttention", zmoe.com/3008.html

Pin status of each function (what fixes it other than itself) is stated in its
docstring; the pins live in ``tests/test_oracle.py``. No function here is
"parity unpinned".
"""

from .paged_attention import (  # noqa: F401
    translate,
    num_logical_blocks,
    element_offset,
    upcast,
    gather_sequence_head,
    softmax_weights,
    attention,
    paged_attention_decode,
    partitioned_decode_head,
    merge_partitions,
)
from .cache_ops import reshape_and_cache, copy_blocks, swap_blocks  # noqa: F401
from .prefill import causal_attention, paged_attention_prefill  # noqa: F401
