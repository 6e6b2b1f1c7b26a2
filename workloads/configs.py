"""Seeded synthetic workloads for the paged decode step.

This module draws random numbers and builds block tables with the host
allocator. It holds none of the attention arithmetic and is the only code that
both the oracle side and the GPU side consume.

One decode step, in launch order:
  1. copy_blocks(copy_pairs)                      (CoW copies, may be empty)
  2. reshape_and_cache(new_key, new_value, slot_mapping)
  3. paged_attention_decode(query, caches, block_tables, context_lens)
``key_cache``/``value_cache`` hold the pool state before step 1;
``context_lens`` count the tokens after step 2.

Five workloads (shapes from the LLaMA-7B page structure of [P3] "3.1
PagedAttention的核心原理" §3.1.2 "页面结构设计": 32 heads x 128 dims, fp16, 16
tokens per page, so 16 KiB of K+V per token and 256 KiB per page):
  1 tiny        4 seqs, 4 heads x 64, ctx {35, 16, 1, 50}, 32-block pool
  2 llama7b     64 seqs, ctx uniform in [128, 2048]
  3 write       256 seqs, ctx = clip(round(Exponential(512)), 1, 2048)
  4 shared      16 prompts x 8 samples, bf16, 328-token shared prefix (21
                blocks, refcount 8), suffix uniform in [1, 256]; the partly
                filled prefix block is copied on divergence
  5 long        8 seqs x 32768 tokens
Every sequence's newest token(s) are written by step 2: the context length is
the length after the write, so a sequence holds ctx-1 tokens before the step
(config 4: the whole suffix is written). Pools are sized to ceil(1.1 x blocks
in use) (the 10% slack of [P1] §3.3.4's admission rule), and the free list
starts as a seeded shuffle, so block tables are non-contiguous.

Values: every slot of both pools, the queries and the new tokens are N(0, 1)
drawn as float32 and rounded to nearest-even into fp16 or bf16. Random streams
come from numpy.random.SeedSequence(1000 + config index).spawn(...).
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .allocator import BlockAllocator

BLOCK_SIZE = 16
_CHUNK = 1 << 22
_NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}

CONFIG_NAMES = {1: "tiny", 2: "llama7b_decode", 3: "cache_write_decode",
                4: "shared_prefix_sampling", 5: "long_context"}


@dataclass
class Workload:
    index: int
    name: str
    dtype: str                      # "f16" or "bf16"
    num_seqs: int
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float                    # float32 value 1/sqrt(head_dim)
    query: np.ndarray               # uint16 [S, H, D]
    key_cache: np.ndarray           # uint16 [NB, bs, H, D], before the step
    value_cache: np.ndarray
    block_tables: np.ndarray        # int32 [S, MB], -1 padded
    context_lens: np.ndarray        # int32 [S], after the write
    new_key: np.ndarray             # uint16 [T, H, D]
    new_value: np.ndarray
    slot_mapping: np.ndarray        # int64 [T]
    copy_pairs: np.ndarray          # int32 [P, 2] (src, dst)
    group_start: np.ndarray | None = None   # int32 [G+1] sequence ranges sharing a prefix
    shared_blocks: np.ndarray | None = None  # int32 [G] leading blocks identical in a group
    query_start: np.ndarray | None = None    # prefill only: int32 [S+1] rows of each chunk
    allocator: BlockAllocator | None = field(default=None, repr=False)

    @property
    def kv_bytes_per_token(self) -> int:
        """Bytes of K plus V of one token over all heads (16 KiB at 32 x 128 fp16)."""
        return 2 * self.num_heads * self.head_dim * 2

    @property
    def total_context(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())


def _seed_streams(index: int, n: int = 8):
    return np.random.SeedSequence(1000 + index).spawn(n)


def _normal_bits(seed: np.random.SeedSequence, count: int, dtype: str,
                 threads: int = 8) -> np.ndarray:
    """``count`` N(0,1) values as 16-bit words, generated in fixed-size chunks
    with one child stream per chunk, so the result does not depend on the
    number of threads."""
    out = np.empty(count, dtype=np.uint16)
    nchunks = max(1, (count + _CHUNK - 1) // _CHUNK)
    seeds = seed.spawn(nchunks)

    def fill(i):
        lo = i * _CHUNK
        n = min(_CHUNK, count - lo)
        if n <= 0:
            return
        x = np.random.Generator(np.random.PCG64(seeds[i])).standard_normal(n, dtype=np.float32)
        if dtype == "f16":
            out[lo:lo + n] = x.astype(np.float16).view(np.uint16)
        else:
            import torch  # round-to-nearest-even float32 -> bfloat16
            out[lo:lo + n] = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def _finish(index, name, dtype, H, D, alloc, seqs, ctx, MB, streams, new_tokens,
            slots, pairs, group_start=None, shared_blocks=None):
    S = len(seqs)
    NB = alloc.num_blocks
    bs = alloc.block_size
    T = len(slots)
    q = _normal_bits(streams[2], S * H * D, dtype).reshape(S, H, D)
    kc = _normal_bits(streams[3], NB * bs * H * D, dtype).reshape(NB, bs, H, D)
    vc = _normal_bits(streams[4], NB * bs * H * D, dtype).reshape(NB, bs, H, D)
    nk = _normal_bits(streams[5], T * H * D, dtype).reshape(T, H, D)
    nv = _normal_bits(streams[6], T * H * D, dtype).reshape(T, H, D)
    return Workload(
        index=index, name=name, dtype=dtype, num_seqs=S, num_heads=H, head_dim=D,
        block_size=bs, num_blocks=NB, max_blocks_per_seq=MB,
        scale=float(np.float32(1.0 / math.sqrt(D))),
        query=q, key_cache=kc, value_cache=vc,
        block_tables=alloc.tables_array(seqs, MB),
        context_lens=np.asarray(ctx, dtype=np.int32),
        new_key=nk, new_value=nv,
        slot_mapping=np.asarray(slots, dtype=np.int64).reshape(T),
        copy_pairs=np.asarray(pairs, dtype=np.int32).reshape(-1, 2),
        group_start=group_start, shared_blocks=shared_blocks, allocator=alloc,
    )


def _blocks(tokens: int, bs: int = BLOCK_SIZE) -> int:
    return (tokens + bs - 1) // bs


def _decode_batch(index, name, dtype, H, D, ctx, MB, streams, pool=None, bs=BLOCK_SIZE):
    """Sequences hold ctx-1 tokens; the step writes token ctx-1 of each."""
    S = len(ctx)
    needed = sum(_blocks(int(c), bs) for c in ctx)
    if pool is None:
        pool = math.ceil(1.1 * needed)
    order = np.random.Generator(np.random.PCG64(streams[1])).permutation(pool)
    alloc = BlockAllocator(pool, bs, free_order=order)
    seqs = list(range(S))
    for s in seqs:
        alloc.allocate(s, int(ctx[s]) - 1)
    slots = []
    for s in seqs:
        slot, pair = alloc.append_slot(s)
        assert pair is None
        slots.append(slot)
    return _finish(index, name, dtype, H, D, alloc, seqs, ctx, MB, streams, S, slots, [])


def make_decode_case(ctx, num_heads: int, head_dim: int, dtype: str = "f16", seed: int = 0,
                     max_blocks: int | None = None, pool: int | None = None,
                     block_size: int = BLOCK_SIZE) -> Workload:
    """A decode step over the given context lengths (each sequence's last token
    is written by the step), for edge-case tests. Same recipe as the numbered
    workloads, seeded by ``seed``."""
    st = np.random.SeedSequence(seed).spawn(8)
    ctx = [int(c) for c in ctx]
    if min(ctx) < 1:
        raise ValueError("context lengths must be >= 1")
    mb = max_blocks if max_blocks is not None else max(_blocks(c, block_size) for c in ctx)
    return _decode_batch(0, "custom", dtype, num_heads, head_dim, ctx, mb, st, pool, block_size)


def make_config(index: int, block_size: int = BLOCK_SIZE) -> Workload:
    """Build workload ``index`` (1..5) over blocks of ``block_size`` tokens.
    Deterministic for a given (index, block_size); the context lengths do not
    depend on the block size, the pools (sized in blocks) do."""
    st = _seed_streams(index)
    bs = block_size
    if index == 1:
        ctx = [35, 16, 1, 50]
        pool = 32 * BLOCK_SIZE // bs
        return _decode_batch(1, CONFIG_NAMES[1], "f16", 4, 64, ctx, _blocks(max(ctx), bs), st,
                             pool=pool, bs=bs)
    if index == 2:
        ctx = np.random.Generator(np.random.PCG64(st[0])).integers(128, 2048, size=64, endpoint=True)
        return _decode_batch(2, CONFIG_NAMES[2], "f16", 32, 128, ctx, 2048 // bs, st, bs=bs)
    if index == 3:
        x = np.random.Generator(np.random.PCG64(st[0])).exponential(512.0, size=256)
        ctx = np.clip(np.rint(x), 1, 2048).astype(np.int64)
        return _decode_batch(3, CONFIG_NAMES[3], "f16", 32, 128, ctx, 2048 // bs, st, bs=bs)
    if index == 4:
        return _shared_prefix(st, bs=bs)
    if index == 5:
        ctx = [32768] * 8
        return _decode_batch(5, CONFIG_NAMES[5], "f16", 32, 128, ctx, 32768 // bs, st, bs=bs)
    raise ValueError(f"no workload {index}")


def _shared_prefix(st, index=4, name=CONFIG_NAMES[4], prompts=16, samples=8, prefix=328,
                   suffix_lo=1, suffix_hi=256, H=32, D=128, dtype="bf16",
                   bs=BLOCK_SIZE) -> Workload:
    """Each prompt's prefix is allocated once and forked to its samples
    (refcount = samples); then every sample appends its own suffix in index
    order, copying the shared, partly filled last prefix block on its first
    write while that block is still shared."""
    suffix = np.random.Generator(np.random.PCG64(st[0])).integers(suffix_lo, suffix_hi,
                                                                 size=prompts * samples,
                                                                 endpoint=True)
    ctx = prefix + suffix
    prefix_blocks = _blocks(prefix, bs)
    full_prefix_blocks = prefix // bs
    partial = prefix % bs != 0
    # blocks in use at the end: one prefix per prompt, a CoW copy of a partly
    # filled last prefix block for every writing sample but the last of each
    # prompt, and each sample's own further blocks
    copies = 0
    if partial:
        for g in range(prompts):
            writers = int((suffix[g * samples:(g + 1) * samples] > 0).sum())
            copies += max(writers - 1, 0)
    needed = prompts * prefix_blocks + copies + sum(
        max(_blocks(int(c), bs) - prefix_blocks, 0) for c in ctx)
    pool = math.ceil(1.1 * needed)
    order = np.random.Generator(np.random.PCG64(st[1])).permutation(pool)
    alloc = BlockAllocator(pool, bs, free_order=order)
    seqs = list(range(prompts * samples))
    for g in range(prompts):
        alloc.allocate(g * samples, prefix)
        for j in range(1, samples):
            alloc.fork(g * samples, g * samples + j)
    slots, pairs = [], []
    for s in seqs:                                       # samples diverge in index order
        for _ in range(int(suffix[s])):
            slot, pair = alloc.append_slot(s)
            slots.append(slot)
            if pair is not None:
                pairs.append(pair)
    MB = _blocks(prefix + suffix_hi, bs)
    group_start = np.arange(0, prompts * samples + 1, samples, dtype=np.int32)
    shared = np.full(prompts, full_prefix_blocks, dtype=np.int32)
    return _finish(index, name, dtype, H, D, alloc, seqs, ctx, MB, st, len(slots),
                   slots, pairs, group_start=group_start, shared_blocks=shared)


def make_shared_case(prompts, samples, prefix, suffix_lo, suffix_hi, num_heads, head_dim,
                     dtype="f16", seed=0, block_size=BLOCK_SIZE) -> Workload:
    """A shared-prefix decode step (the recipe of the parallel-sampling
    workload) with free sizes, for edge-case tests."""
    st = np.random.SeedSequence(seed).spawn(8)
    return _shared_prefix(st, 0, "custom_shared", prompts, samples, prefix, suffix_lo, suffix_hi,
                          num_heads, head_dim, dtype, block_size)


def make_prefill_case(chunk_lens, cached_lens, num_heads: int, head_dim: int, dtype: str = "f16",
                      seed: int = 0, block_size: int = BLOCK_SIZE, max_blocks: int | None = None,
                      name: str = "prefill") -> Workload:
    """A prefill / chunked-prefill step: sequence s holds cached_lens[s] tokens
    and the step appends a chunk of chunk_lens[s] tokens (pages taken as
    needed, [P1] §3.3.2), writes their K/V with reshape_and_cache and attends
    from each of them causally. ``query`` and the new K/V are packed [T, H, D]
    with T = sum(chunk_lens); ``query_start`` gives each sequence's rows."""
    chunk_lens = [int(c) for c in chunk_lens]
    cached_lens = [int(c) for c in cached_lens]
    if len(chunk_lens) != len(cached_lens) or min(chunk_lens) < 0 or min(cached_lens) < 0:
        raise ValueError("one non-negative chunk and cached length per sequence")
    st = np.random.SeedSequence(seed).spawn(8)
    bs = block_size
    ctx = [a + b for a, b in zip(chunk_lens, cached_lens)]
    if min(ctx) < 1:
        raise ValueError("every sequence needs at least one token")
    needed = sum(_blocks(c, bs) for c in ctx)
    pool = math.ceil(1.1 * needed) + 2
    order = np.random.Generator(np.random.PCG64(st[1])).permutation(pool)
    alloc = BlockAllocator(pool, bs, free_order=order)
    seqs = list(range(len(ctx)))
    for s in seqs:
        alloc.allocate(s, cached_lens[s])
    slots = []
    for s in seqs:
        alloc.append_tokens(s, chunk_lens[s])
        slots += [alloc.slot(s, p) for p in range(cached_lens[s], ctx[s])]
    mb = max_blocks if max_blocks is not None else max(_blocks(c, bs) for c in ctx)
    w = _finish(0, name, dtype, num_heads, head_dim, alloc, seqs, ctx, mb, st, len(slots), slots, [])
    T = len(slots)
    w.query = _normal_bits(st[7], T * num_heads * head_dim, dtype).reshape(T, num_heads, head_dim)
    w.query_start = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int32)
    return w


def poison_unused(w: Workload) -> Workload:
    """Fill every slot that holds no valid token after the step with NaN bits.

    Valid after the step: positions [0, ctx) of every sequence (the written
    token included). Everything else (rows past ctx in last blocks, free blocks,
    stale rows) becomes a quiet-NaN pattern, so any read of it shows up."""
    nan = np.uint16(_NAN_BITS[w.dtype])
    valid = np.zeros((w.num_blocks, w.block_size), dtype=bool)
    alloc = w.allocator
    for s in range(w.num_seqs):
        for pos in range(int(w.context_lens[s])):
            b, o = divmod(alloc.slot(s, pos), w.block_size)
            valid[b, o] = True
    kc = w.key_cache.copy()
    vc = w.value_cache.copy()
    # CoW destinations are overwritten whole by the copy
    for _, dst in w.copy_pairs.tolist():
        kc[dst] = nan
        vc[dst] = nan
    # the slots written by the step are valid afterwards but stale before it
    for slot in w.slot_mapping.tolist():
        b, o = divmod(int(slot), w.block_size)
        kc[b, o] = nan
        vc[b, o] = nan
    kc[~valid] = nan
    vc[~valid] = nan
    import dataclasses
    return dataclasses.replace(w, key_cache=kc, value_cache=vc)
