"""Seeded synthetic inputs shared by the oracle side and the GPU side.

``allocator.BlockAllocator`` builds block tables, slot mappings and CoW pairs;
``configs.make_config(i)`` builds the five decode-step workloads. No attention
arithmetic lives here.
"""

from .allocator import BlockAllocator, SwapSpace  # noqa: F401
from .beam import BeamSearch, BeamStep  # noqa: F401
from .configs import (  # noqa: F401
    BLOCK_SIZE, CONFIG_NAMES, Workload, make_config, make_decode_case, make_prefill_case,
    make_shared_case, poison_unused,
)
