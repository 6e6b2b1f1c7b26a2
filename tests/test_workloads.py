"""The seeded workloads: determinism, shapes, non-contiguous tables, slots that
agree with the oracle's address translation, page byte counts."""

import math

import numpy as np
import pytest

import oracle
from workloads import make_config, poison_unused
from oracle_pins import page_facts


@pytest.fixture(scope="module")
def small():
    return {i: make_config(i) for i in (1, 2, 4)}


def test_deterministic():
    a, b = make_config(1), make_config(1)
    for f in ("query", "key_cache", "value_cache", "block_tables", "context_lens",
              "new_key", "new_value", "slot_mapping"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_tiny_shapes(small):
    w = small[1]
    assert (w.num_seqs, w.num_heads, w.head_dim, w.block_size, w.num_blocks) == (4, 4, 64, 16, 32)
    assert list(w.context_lens) == [35, 16, 1, 50]
    assert w.scale == 0.125
    assert w.block_tables.shape == (4, 4)
    used = np.sort(w.block_tables[w.block_tables >= 0])
    assert not np.array_equal(used, np.arange(used.size))      # not the first ids in order


def test_pool_sizes_and_tables(small):
    for w in small.values():
        nblocks = [oracle.num_logical_blocks(int(c), 16) for c in w.context_lens]
        for s, n in enumerate(nblocks):
            row = w.block_tables[s]
            assert (row[:n] >= 0).all() and (row[:n] < w.num_blocks).all()
            assert (row[n:] == -1).all()
        if w.index != 1:
            used = np.unique(w.block_tables[w.block_tables >= 0]).size
            assert w.num_blocks == math.ceil(1.1 * used)


def test_slots_match_oracle_translation(small):
    """Every written slot equals the oracle's element offset of the token divided
    by kv_dim, for the token the step appends."""
    for w in small.values():
        kv_dim = w.num_heads * w.head_dim
        if w.index == 4:
            i = 0
            for s in range(w.num_seqs):                      # the whole suffix after the 328-token prefix
                for pos in range(328, int(w.context_lens[s])):
                    off = oracle.element_offset(w.block_tables[s], pos, 16, kv_dim)
                    assert off % kv_dim == 0 and off // kv_dim == w.slot_mapping[i]
                    i += 1
            assert i == len(w.slot_mapping)
        else:
            for s in range(w.num_seqs):
                pos = int(w.context_lens[s]) - 1
                off = oracle.element_offset(w.block_tables[s], pos, 16, kv_dim)
                assert off // kv_dim == w.slot_mapping[s]


def test_llama7b_bytes_per_token(small):
    f = page_facts()["llama7b_page"]
    w = small[2]
    assert (w.num_heads, w.head_dim) == (f["num_heads"], f["head_dim"])
    assert w.kv_bytes_per_token == f["kv_bytes_per_token"]
    assert w.kv_bytes_per_token * w.block_size == f["page_bytes"]
    p = page_facts()["preallocation"]
    assert p["preallocated_tokens"] * p["kv_bytes_per_token"] == p["preallocated_bytes"]
    assert (p["preallocated_tokens"] - p["used_tokens"]) * p["kv_bytes_per_token"] == p["idle_bytes"]


def test_value_distribution(small):
    x = oracle.upcast(small[2].key_cache.reshape(-1)[:1 << 20], "f16")
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    y = oracle.upcast(small[4].value_cache.reshape(-1)[:1 << 20], "bf16")
    assert abs(y.mean()) < 0.01 and abs(y.std() - 1.0) < 0.01


def test_shared_prefix_groups(small):
    w = small[4]
    assert w.dtype == "bf16" and w.num_seqs == 128
    assert list(w.group_start) == list(range(0, 129, 8))
    assert (w.shared_blocks == 20).all()
    assert ((w.context_lens >= 329) & (w.context_lens <= 584)).all()
    for g in range(16):
        t = w.block_tables[g * 8:(g + 1) * 8, :20]
        assert (t == t[0]).all()


def test_poison_keeps_valid_tokens(small):
    """After the step, reading only valid tokens through the oracle gives the
    same result with and without the NaN canaries."""
    w = small[1]
    p = poison_unused(w)
    outs = []
    for x in (w, p):
        K, V = oracle.reshape_and_cache(x.new_key, x.new_value, x.key_cache, x.value_cache,
                                        x.slot_mapping, 16)
        outs.append(oracle.paged_attention_decode(x.query, K, V, x.block_tables, x.context_lens,
                                                  x.scale, 16, x.dtype))
    assert np.isfinite(outs[1]).all()
    assert np.array_equal(outs[0], outs[1])
    assert np.isnan(oracle.upcast(p.key_cache, "f16")).sum() > 0


@pytest.mark.parametrize("bs", [8, 32])
def test_block_size_variants(bs):
    """The same workloads over 8- and 32-token blocks: same context lengths,
    tables of ceil(ctx / bs) valid entries, slots that match the oracle's
    translation at that block size, prefix blocks shared within each group."""
    for i in (1, 4):
        w, w16 = make_config(i, bs), make_config(i)
        assert w.block_size == bs and w.key_cache.shape[1] == bs
        assert np.array_equal(w.context_lens, w16.context_lens)
        kv_dim = w.num_heads * w.head_dim
        for s in range(w.num_seqs):
            n = oracle.num_logical_blocks(int(w.context_lens[s]), bs)
            row = w.block_tables[s]
            assert (row[:n] >= 0).all() and (row[:n] < w.num_blocks).all() and (row[n:] == -1).all()
        first = 328 if i == 4 else None
        k = 0
        for s in range(w.num_seqs):
            lo = first if first is not None else int(w.context_lens[s]) - 1
            for pos in range(lo, int(w.context_lens[s])):
                off = oracle.element_offset(w.block_tables[s], pos, bs, kv_dim)
                assert off // kv_dim == w.slot_mapping[k]
                k += 1
        assert k == len(w.slot_mapping)
        w.allocator.check_invariants()
    w = make_config(4, bs)
    assert (w.shared_blocks == 328 // bs).all()
    assert len(w.copy_pairs) == (0 if 328 % bs == 0 else 112)
    for g in range(16):
        t = w.block_tables[g * 8:(g + 1) * 8, :328 // bs]
        assert (t == t[0]).all()
