"""Oracle: the slot-mapped cache write and the copy-on-write block copy, on bit views.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Both operations move 16-bit words without arithmetic, so the oracle works on
uint16 arrays and the expected result is exact: NaN payloads and -0.0 survive.
Inputs are never modified; each function returns new arrays.
"""

from __future__ import annotations

import numpy as np


def reshape_and_cache(key_bits, value_bits, key_cache_bits, value_cache_bits,
                      slot_mapping, block_size: int):
    """Write each new token's K and V rows into its slot.

    key/value_bits   uint16 [T, H, D]  (new tokens)
    caches           uint16 [num_blocks, block_size, H, D]
    slot_mapping     int    [T]; slot = physical_block * block_size + offset

    For token i with slot s >= 0: cache[s // block_size, s % block_size] = row i
    [P2 "Copy-on-Write共享解码的显存优化原理": the new token's KV is written into
    its block; P1 §3.3.2 "动态页面分配机制": a new page is taken when the token
    count exceeds num_blocks * block_size; P3 §3.1.3: the slot is the token's
    physical block and offset]. Readings where the pages are silent: a negative
    slot marks a padding token and is skipped; slots in one call must be unique
    (otherwise the result would depend on write order), and the function
    refuses duplicates.
    Pinned: round trip through the block table returns the same bits, and every
    other slot is unchanged.
    """
    key_bits = np.asarray(key_bits)
    value_bits = np.asarray(value_bits)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if key_bits.dtype != np.uint16 or key_cache_bits.dtype != np.uint16:
        raise TypeError("expected uint16 bit patterns")
    if key_bits.shape != value_bits.shape or key_bits.shape[0] != slots.shape[0]:
        raise ValueError("key, value and slot_mapping disagree on the token count")
    num_blocks = key_cache_bits.shape[0]
    live = slots[slots >= 0]
    if live.size and live.max() >= num_blocks * block_size:
        raise IndexError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slots in one call")
    K = key_cache_bits.copy()
    V = value_cache_bits.copy()
    for i, s in enumerate(slots.tolist()):
        if s < 0:
            continue
        block, offset = s // block_size, s % block_size
        K[block, offset] = key_bits[i]
        V[block, offset] = value_bits[i]
    return K, V


def copy_blocks(key_cache_bits, value_cache_bits, block_mapping):
    """Copy whole blocks (every token, head and dim of K and of V) src -> dst.

    block_mapping  int [P, 2] rows (src, dst)

    [P2 "Python 演示" copy_on_write: when a shared block (refcount > 1) is about
    to be written, a new block is allocated and the caller copies the data into
    it; P3 §3.1.5 "CoW机制的实现" step 3; P4 "Memory Sharing与写时复制".]
    Reading where the pages are silent: a CoW copy always lands in a freshly
    allocated block, so destinations are unique and never a source in the same
    call; the function refuses mappings that break this (the result would
    otherwise depend on copy order).
    Pinned: afterwards dst equals the old src bit for bit, every source and
    every untouched block is unchanged.
    """
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    num_blocks = key_cache_bits.shape[0]
    if pairs.size and (pairs.min() < 0 or pairs.max() >= num_blocks):
        raise IndexError("block id outside the pool")
    src, dst = pairs[:, 0], pairs[:, 1]
    if np.unique(dst).size != dst.size:
        raise ValueError("duplicate destination blocks")
    if np.intersect1d(src, dst).size:
        raise ValueError("a destination block is also a source")
    K = key_cache_bits.copy()
    V = value_cache_bits.copy()
    for s, d in pairs.tolist():
        K[d] = key_cache_bits[s]
        V[d] = value_cache_bits[s]
    return K, V


def swap_blocks(src_key_bits, src_value_bits, dst_key_bits, dst_value_bits, block_mapping):
    """Copy whole blocks from one pool pair into another: swap-out (device pool
    -> host pool) and swap-in (host pool -> device pool).

    block_mapping  int [P, 2] rows (src block in the source pools, dst block in
    the destination pools)

    [P1 §3.3.3 "显存不足时的处理策略", CPU Swap: the blocks of a sequence being
    swapped out are copied block by block into pre-allocated host buffers and
    its device blocks freed; swapping in copies them back into newly
    allocated device blocks.] Reading where the pages are silent: destination
    blocks are unique in one call (otherwise the result would depend on copy
    order); the function refuses duplicates. The source pools are not changed.
    Pinned: a swap-out followed by a swap-in into other device blocks gives
    the sequence the same attention output through its new block table, bit
    for bit, and every block not named as a destination is unchanged.
    """
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    if src_key_bits.shape[1:] != dst_key_bits.shape[1:]:
        raise ValueError("source and destination blocks differ in shape")
    if pairs.size and (pairs.min() < 0 or pairs[:, 0].max() >= src_key_bits.shape[0]
                       or pairs[:, 1].max() >= dst_key_bits.shape[0]):
        raise IndexError("block id outside its pool")
    if np.unique(pairs[:, 1]).size != pairs.shape[0]:
        raise ValueError("duplicate destination blocks")
    K = dst_key_bits.copy()
    V = dst_value_bits.copy()
    for s, d in pairs.tolist():
        K[d] = src_key_bits[s]
        V[d] = src_value_bits[s]
    return K, V
