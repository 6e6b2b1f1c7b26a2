"""MI355X-native paged KV-cache decode attention.

The product is libpaged_kv.so (hand-written gfx950 HIP kernels behind the C
ABI in include/paged_kv.h); this package is its thin torch binding. Importing
the package does not load the library; the first call does, and fails loudly
if it is not built.
"""

from ._lib import PagedKVError, lib  # noqa: F401
from .ops import (  # noqa: F401
    alloc_workspace,
    copy_blocks,
    grouped_workspace_size,
    paged_attention_decode,
    paged_attention_decode_grouped,
    paged_attention_decode_merge,
    paged_attention_decode_noalloc,
    paged_attention_decode_partitions,
    paged_attention_prefill,
    reshape_and_cache,
    swap_blocks,
    workspace_size,
)
