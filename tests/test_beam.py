"""Beam-search workload (host side): fork / free / copy-on-write over many
steps keeps the allocator consistent, the groups' shared blocks really are
identical full blocks, and every CoW pair copies a shared partial block into
a fresh one."""

import numpy as np
import pytest

from workloads import BeamSearch


@pytest.mark.parametrize("groups,bs", [("prompt", 16), ("parent", 16), ("prompt", 8), ("parent", 32)])
def test_beam_steps_keep_invariants(groups, bs):
    b = BeamSearch(prompts=3, beams=4, prompt_lo=20, prompt_hi=70, steps=40, num_heads=2,
                   head_dim=64, block_size=bs, seed=11, groups=groups)
    lens = b.prompt_lens.copy()
    for t in range(40):
        st = b.step()
        a = b.allocator
        a.check_invariants()
        S = b.num_seqs
        assert st.context_lens.shape == (S,) and st.block_tables.shape == (S, b.max_blocks)
        for g in range(b.P):                               # all beams of a prompt: same length
            assert (st.context_lens[g * b.k:(g + 1) * b.k] == lens[g] + t + 1).all()
        gs, sb = st.group_start, st.shared_blocks
        assert gs[0] == 0 and gs[-1] == S and (np.diff(gs) > 0).all()
        for i in range(len(sb)):
            rows = st.block_tables[gs[i]:gs[i + 1]]
            n = int(sb[i])
            assert n * bs <= st.context_lens[gs[i]:gs[i + 1]].min()
            assert (rows[:, :n] == rows[0, :n]).all()
            full = int(st.context_lens[gs[i]]) // bs
            if n < full:                                   # maximal: the next full block differs
                assert not (rows[:, n] == rows[0, n]).all()
        if groups == "parent":      # siblings share every block that was full before the write
            for i in range(len(sb)):
                assert sb[i] >= (int(st.context_lens[gs[i]]) - 1) // bs
        dst = st.copy_pairs[:, 1]
        assert np.unique(dst).size == dst.size and not np.intersect1d(dst, st.copy_pairs[:, 0]).size
        for src, d in st.copy_pairs.tolist():               # the copy landed in a beam's table
            assert a.refcount(d) >= 1
        for s in range(S):                                  # the written slot is the last token
            pos = int(st.context_lens[s]) - 1
            assert st.slot_mapping[s] == st.block_tables[s, pos // bs] * bs + pos % bs
        assert st.blocks_in_use <= st.blocks_unshared
    assert st.blocks_in_use < st.blocks_unshared


def test_beam_is_deterministic():
    a = BeamSearch(prompts=2, beams=3, prompt_lo=10, prompt_hi=40, steps=5, num_heads=2,
                   head_dim=64, seed=4)
    b = BeamSearch(prompts=2, beams=3, prompt_lo=10, prompt_hi=40, steps=5, num_heads=2,
                   head_dim=64, seed=4)
    assert np.array_equal(a.key_cache, b.key_cache)
    for _ in range(5):
        x, y = a.step(), b.step()
        for f in ("copy_pairs", "new_key", "slot_mapping", "query", "block_tables", "shared_blocks"):
            assert np.array_equal(getattr(x, f), getattr(y, f)), f
    with pytest.raises(RuntimeError):
        a.step()
