"""Seeded beam-search decoding over many steps: fork, copy-on-write and
grouped decode with groups that change every step.

[P4 "Memory Sharing与写时复制" and its second question: beam search keeps the
top k candidates at every step, all of which share the prompt's KV, so one
copy serves every branch; a block is counted by the readers in its metadata,
and a shared block that is about to be written is copied first and the
writer's table remapped. P2 "Copy-on-Write共享解码的显存优化原理": copy only
while the count is above one.]

One step, for every prompt: k parents are drawn (with replacement) from the k
current beams, standing in for the top-k choice of a real model: a softmax of
seeded normal scores times ``skew``, so a few beams have many children and
lineages die out. Each child is forked from its parent (all blocks shared),
the old generation is freed, then every child appends its new token in order:
a partly filled last block still shared with a sibling is copied first. The
device step is then copy_blocks(pairs) -> reshape_and_cache(new tokens) ->
decode over the children.

Children are ordered by parent, so siblings are neighbours. ``groups``:
  "prompt":  one group per prompt; its shared blocks are the leading full
             blocks identical in all k beams (the prompt, and more once the
             lineages have merged);
  "parent":  one group per parent; siblings share every full block.
Nothing here does attention arithmetic; the oracle and the GPU both read the
same step inputs.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .allocator import BlockAllocator
from .configs import _normal_bits


@dataclass
class BeamStep:
    copy_pairs: np.ndarray      # int32 [P, 2] CoW (src, dst), before the write
    new_key: np.ndarray         # uint16 [S, H, D] one new token per beam
    new_value: np.ndarray
    slot_mapping: np.ndarray    # int64 [S]
    query: np.ndarray           # uint16 [S, H, D]
    block_tables: np.ndarray    # int32 [S, MB], -1 padded
    context_lens: np.ndarray    # int32 [S], after the write
    group_start: np.ndarray     # int32 [G + 1]
    shared_blocks: np.ndarray   # int32 [G]
    parents: np.ndarray         # int32 [S] previous-step index of each beam's parent
    blocks_in_use: int          # physical blocks referenced after the step
    blocks_unshared: int        # blocks the beams would hold without sharing


class BeamSearch:
    def __init__(self, prompts=16, beams=8, prompt_lo=256, prompt_hi=1024, steps=32,
                 num_heads=32, head_dim=128, dtype="f16", block_size=16, seed=0, skew=2.0,
                 groups="prompt"):
        if groups not in ("prompt", "parent"):
            raise ValueError("groups must be 'prompt' or 'parent'")
        self.P, self.k, self.H, self.D = prompts, beams, num_heads, head_dim
        self.dtype, self.bs, self.steps, self.skew, self.groups = dtype, block_size, steps, skew, groups
        self._st = np.random.SeedSequence(seed).spawn(8)
        self._rng = np.random.Generator(np.random.PCG64(self._st[0]))
        self.prompt_lens = self._rng.integers(prompt_lo, prompt_hi, size=prompts, endpoint=True)
        bs = block_size
        self.max_blocks = -(-(int(self.prompt_lens.max()) + steps) // bs)
        per_beam = -(-steps // bs) + 2
        needed = int(sum(-(-int(n) // bs) for n in self.prompt_lens)) + prompts * beams * per_beam
        self.num_blocks = math.ceil(1.1 * needed)
        order = np.random.Generator(np.random.PCG64(self._st[1])).permutation(self.num_blocks)
        self.allocator = BlockAllocator(self.num_blocks, bs, free_order=order)
        n = self.num_blocks * bs * num_heads * head_dim
        self.key_cache = _normal_bits(self._st[2], n, dtype).reshape(
            self.num_blocks, bs, num_heads, head_dim)
        self.value_cache = _normal_bits(self._st[3], n, dtype).reshape(
            self.num_blocks, bs, num_heads, head_dim)
        self.scale = float(np.float32(1.0 / math.sqrt(head_dim)))
        self._next_id = 0
        self.beams = []
        for g in range(prompts):
            pid = self._new_id()
            self.allocator.allocate(pid, int(self.prompt_lens[g]))
            kids = [self._new_id() for _ in range(beams)]
            for c in kids:
                self.allocator.fork(pid, c)
            self.allocator.free(pid)
            self.beams.append(kids)
        self.step_index = 0

    def _new_id(self):
        self._next_id += 1
        return self._next_id

    @property
    def num_seqs(self) -> int:
        return self.P * self.k

    def step(self) -> BeamStep:
        """Advance every prompt's beams by one token; returns the device inputs."""
        if self.step_index >= self.steps:
            raise RuntimeError("all steps taken")
        a, k = self.allocator, self.k
        rng = self._rng
        new_beams, parents, group_sizes = [], [], []
        for g in range(self.P):
            old = self.beams[g]
            w = np.exp(self.skew * rng.standard_normal(k))
            pick = np.sort(rng.choice(k, size=k, p=w / w.sum()))
            kids = []
            for j in pick.tolist():
                c = self._new_id()
                a.fork(old[j], c)
                kids.append(c)
                parents.append(g * k + j)
            new_beams.append(kids)
            if self.groups == "parent":
                group_sizes += np.unique(pick, return_counts=True)[1].tolist()
            else:
                group_sizes.append(k)
        for g in range(self.P):
            for s in self.beams[g]:
                a.free(s)
        self.beams = new_beams
        seqs = [s for kids in new_beams for s in kids]
        slots, pairs = [], []
        for s in seqs:
            slot, pair = a.append_slot(s)
            slots.append(slot)
            if pair is not None:
                pairs.append(pair)
        tables = a.tables_array(seqs, self.max_blocks)
        ctx = np.array([a.num_tokens(s) for s in seqs], dtype=np.int32)
        gs = np.concatenate([[0], np.cumsum(group_sizes)]).astype(np.int32)
        shared = np.zeros(len(group_sizes), dtype=np.int32)
        for i in range(len(group_sizes)):
            rows = tables[gs[i]:gs[i + 1]]
            full = int(ctx[gs[i]:gs[i + 1]].min()) // self.bs
            same = (rows[:, :full] == rows[0, :full]).all(axis=0)
            shared[i] = full if same.all() else int(np.argmin(same))
        S, H, D = len(seqs), self.H, self.D
        sub = self._st[4].spawn(3)      # fresh children every step (spawn counts up)
        nk = _normal_bits(sub[0], S * H * D, self.dtype).reshape(S, H, D)
        nv = _normal_bits(sub[1], S * H * D, self.dtype).reshape(S, H, D)
        q = _normal_bits(sub[2], S * H * D, self.dtype).reshape(S, H, D)
        self.step_index += 1
        unshared = int(sum(-(-int(c) // self.bs) for c in ctx))
        return BeamStep(
            copy_pairs=np.asarray(pairs, dtype=np.int32).reshape(-1, 2), new_key=nk,
            new_value=nv, slot_mapping=np.asarray(slots, dtype=np.int64), query=q,
            block_tables=tables, context_lens=ctx, group_start=gs, shared_blocks=shared,
            parents=np.asarray(parents, dtype=np.int32), blocks_in_use=len(a.used_blocks()),
            blocks_unshared=unshared)
