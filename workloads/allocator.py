"""Host block allocator: free list + per-block reference counts + per-sequence block tables.

Its only job is to build the block tables, slot mappings and copy-on-write
pairs that tests and benchmarks feed to the kernels. It holds no K/V data.

Pages followed:
  [P1] "3.3 页面级显存管理", §3.3.2 "动态页面分配机制" (bulk allocation at
       prefill, one more page when the token count exceeds the capacity) and
       §3.3.4 "全局块池的设计" (one global pool; any free page serves any request).
  [P2] "vLLM三大核心技术分页内存与共享解码", "Copy-on-Write共享解码的显存优化原理"
       (reference count per physical block; copy only while it is > 1; a block
       returns to the pool when its count reaches 0) and "Python 演示"
       (allocate / share_prefix / copy_on_write / release).
  [P3] "3.1 PagedAttention的核心原理", §3.1.2 "页表管理机制" (block table per
       sequence, lookup errors) and §3.1.5 "CoW机制的实现".
  [P4] zmoe.com/3008 notes, "关键误解 页表": one block table per sequence; the
       reference count lives with the physical block.

Readings where the pages disagree or are silent:
  * Free-list discipline: P1's simulations take from the end of the list, P2
    takes from the head. Taken here: first-in first-out from the head of a list
    whose initial order the caller gives (tests pass a seeded shuffle).
  * Out of blocks: ``MemoryError`` (P2, P3); nothing is half-allocated.
  * Unknown sequence: ``KeyError``; logical block past the table: ``IndexError``
    (P3 §3.1.2); freeing an unknown sequence is a no-op (P1, P3).
  * ``cow`` returns the (src, dst) pair and leaves the data copy to the caller
    (P2 "Python 演示"), who batches the pairs into one block-copy launch.
"""

from __future__ import annotations

from collections import deque

import numpy as np


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self._free = deque(order)
        self._ref = [0] * self.num_blocks
        self._tables: dict = {}
        self._tokens: dict = {}

    # ---- pool -------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def refcount(self, block: int) -> int:
        return self._ref[block]

    def free_blocks(self) -> list:
        return list(self._free)

    def _take(self, n: int) -> list:
        if n > len(self._free):
            raise MemoryError(f"out of blocks: need {n}, {len(self._free)} free")
        out = [self._free.popleft() for _ in range(n)]
        for b in out:
            self._ref[b] = 1
        return out

    def _drop(self, block: int) -> None:
        self._ref[block] -= 1
        if self._ref[block] < 0:
            raise AssertionError(f"refcount of block {block} went negative")
        if self._ref[block] == 0:
            self._free.append(block)

    # ---- sequences --------------------------------------------------------
    def _blocks_for(self, tokens: int) -> int:
        return (tokens + self.block_size - 1) // self.block_size

    def allocate(self, seq, num_tokens: int) -> list:
        """New sequence holding ``num_tokens`` tokens: take all its blocks at once."""
        if seq in self._tables:
            raise ValueError(f"sequence {seq!r} already exists")
        if num_tokens < 0:
            raise ValueError("num_tokens must be >= 0")
        blocks = self._take(self._blocks_for(num_tokens))
        self._tables[seq] = blocks
        self._tokens[seq] = int(num_tokens)
        return list(blocks)

    def append_tokens(self, seq, n: int) -> list:
        """Grow a sequence by ``n`` tokens, taking new blocks only when the
        token count passes the capacity of the blocks it holds. Shared blocks
        are not copied here; use ``append_slot`` for a write that may need CoW."""
        table = self._table(seq)
        new_total = self._tokens[seq] + int(n)
        extra = self._blocks_for(new_total) - len(table)
        if extra > 0:
            table.extend(self._take(extra))
        self._tokens[seq] = new_total
        return list(table)

    def fork(self, src, dst, num_blocks=None) -> list:
        """``dst`` maps the first ``num_blocks`` blocks of ``src`` (all by
        default); each shared block's reference count goes up by one."""
        table = self._table(src)
        if dst in self._tables:
            raise ValueError(f"sequence {dst!r} already exists")
        n = len(table) if num_blocks is None else int(num_blocks)
        if n > len(table):
            raise IndexError("cannot share more blocks than the source holds")
        shared = table[:n]
        for b in shared:
            self._ref[b] += 1
        self._tables[dst] = list(shared)
        self._tokens[dst] = min(self._tokens[src], n * self.block_size)
        return list(shared)

    def cow(self, seq, logical: int):
        """Copy-on-write check before writing into logical block ``logical``.

        Reference count 1: the block is written in place, returns None.
        Greater than 1: take a fresh block, remap the table entry to it, drop one
        reference to the old block, and return (old, new) for the data copy."""
        table = self._table(seq)
        if logical >= len(table) or logical < 0:
            raise IndexError(f"logical block {logical} outside the table of {seq!r}")
        old = table[logical]
        if self._ref[old] <= 1:
            return None
        (new,) = self._take(1)
        self._drop(old)
        table[logical] = new
        return (old, new)

    def append_slot(self, seq):
        """Reserve the slot of the sequence's next token.

        Returns (slot, copy_pair_or_None). A token that starts a block takes a
        fresh block; a token that lands in a shared block triggers ``cow``."""
        table = self._table(seq)
        pos = self._tokens[seq]
        logical = pos // self.block_size
        pair = None
        if logical == len(table):
            table.extend(self._take(1))
        else:
            pair = self.cow(seq, logical)
        self._tokens[seq] = pos + 1
        return self.slot(seq, pos), pair

    def slot(self, seq, pos: int) -> int:
        """Slot (physical block * block_size + offset) of token ``pos``."""
        table = self._table(seq)
        logical, offset = divmod(int(pos), self.block_size)
        if pos < 0 or logical >= len(table):
            raise IndexError(f"token {pos} outside the blocks of {seq!r}")
        return table[logical] * self.block_size + offset

    def free(self, seq) -> None:
        """Release every block of ``seq``; blocks reaching count 0 go back to
        the tail of the free list. Unknown sequences are ignored."""
        if seq not in self._tables:
            return
        for b in self._tables.pop(seq):
            self._drop(b)
        del self._tokens[seq]

    # ---- views ------------------------------------------------------------
    def _table(self, seq) -> list:
        if seq not in self._tables:
            raise KeyError(f"unknown sequence {seq!r}")
        return self._tables[seq]

    def block_table(self, seq) -> list:
        return list(self._table(seq))

    def num_tokens(self, seq) -> int:
        self._table(seq)
        return self._tokens[seq]

    def sequences(self) -> list:
        return list(self._tables)

    def tables_array(self, seqs, max_blocks: int) -> np.ndarray:
        """int32 [len(seqs), max_blocks] block tables padded with -1."""
        out = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self._table(s)
            if len(t) > max_blocks:
                raise ValueError(f"sequence {s!r} holds {len(t)} blocks > {max_blocks}")
            out[i, :len(t)] = t
        return out

    def used_blocks(self) -> set:
        return {b for b in range(self.num_blocks) if self._ref[b] > 0}

    def check_invariants(self) -> None:
        """Free list and referenced blocks partition the pool, and each count
        equals the number of table entries that map the block."""
        free = list(self._free)
        if len(set(free)) != len(free):
            raise AssertionError("block twice in the free list")
        used = self.used_blocks()
        if used & set(free):
            raise AssertionError("a referenced block is in the free list")
        if len(used) + len(free) != self.num_blocks:
            raise AssertionError("free + referenced != pool size")
        counts = [0] * self.num_blocks
        for t in self._tables.values():
            for b in t:
                counts[b] += 1
        if counts != self._ref:
            raise AssertionError("reference counts disagree with the block tables")


class SwapSpace:
    """Host swap space for one device pool: a pool of host blocks with its own
    free list, and the sequences that are swapped out.

    [P1 §3.3.3 "显存不足时的处理策略", CPU Swap and its SwapManager simulation:
    swapping a sequence out copies each block of its table into a host block
    taken from a pre-allocated host pool and frees its device blocks; swapping
    it in takes device blocks again (any free ones) and copies the data back,
    returning the host blocks.] ``swap_out`` and ``swap_in`` return the
    (src, dst) block pairs of the copy; the caller moves the data with one
    ``swap_blocks`` launch, issued on the stream before any later write to a
    block freed here.

    Readings where the pages are silent: a device block the sequence shares
    with others only loses this sequence's reference (the others keep it);
    the copy it gets back on swap-in is private. Out of host blocks on
    swap-out, or of device blocks on swap-in: ``MemoryError``, nothing changed.
    """

    def __init__(self, device: BlockAllocator, num_host_blocks: int, free_order=None):
        if num_host_blocks <= 0:
            raise ValueError("num_host_blocks must be positive")
        self.device = device
        self.num_blocks = int(num_host_blocks)
        order = list(range(num_host_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_host_blocks)):
            raise ValueError("free_order must be a permutation of range(num_host_blocks)")
        self._free = deque(order)
        self._swapped: dict = {}     # seq -> (host blocks in logical order, token count)

    @property
    def num_free(self) -> int:
        return len(self._free)

    def swapped(self) -> list:
        return list(self._swapped)

    def host_table(self, seq) -> list:
        return list(self._swapped[seq][0])

    def swap_out(self, seq) -> np.ndarray:
        """Move ``seq`` to host blocks; returns int32 [n, 2] (device, host) pairs
        in logical-block order."""
        if seq in self._swapped:
            raise ValueError(f"sequence {seq!r} is already swapped out")
        table = self.device.block_table(seq)           # KeyError if unknown
        tokens = self.device.num_tokens(seq)
        if len(table) > len(self._free):
            raise MemoryError(f"out of host swap blocks: need {len(table)}, {len(self._free)} free")
        host = [self._free.popleft() for _ in table]
        self.device.free(seq)
        self._swapped[seq] = (host, tokens)
        return np.asarray(list(zip(table, host)), dtype=np.int32).reshape(-1, 2)

    def swap_in(self, seq) -> np.ndarray:
        """Bring ``seq`` back into newly allocated device blocks; returns int32
        [n, 2] (host, device) pairs in logical-block order."""
        host, tokens = self._swapped[seq]                # KeyError if not swapped out
        if len(host) > self.device.num_free:
            raise MemoryError(f"out of device blocks: need {len(host)}, "
                              f"{self.device.num_free} free")
        table = self.device.allocate(seq, tokens)
        if len(table) != len(host):
            raise AssertionError("a swapped sequence's token count no longer fits its blocks")
        del self._swapped[seq]
        self._free.extend(host)
        return np.asarray(list(zip(host, table)), dtype=np.int32).reshape(-1, 2)

    def check_invariants(self) -> None:
        held = [b for host, _ in self._swapped.values() for b in host]
        free = list(self._free)
        if len(set(held)) != len(held) or set(held) & set(free):
            raise AssertionError("a host block is held twice or held and free")
        if len(held) + len(free) != self.num_blocks:
            raise AssertionError("held + free != host pool size")
        if set(self._swapped) & set(self.device.sequences()):
            raise AssertionError("a sequence is both resident and swapped out")
