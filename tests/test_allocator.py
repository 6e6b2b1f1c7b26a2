"""Host block allocator: the pages' demo sequences, refcount semantics, invariants, errors."""

import json
import os

import numpy as np
import pytest

from workloads import BlockAllocator, SwapSpace, make_config

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _demos():
    with open(os.path.join(GOLDEN, "allocator_demos.json")) as f:
        return json.load(f)


def test_p2_demo_sequence():
    d = _demos()["p2_demo"]
    a = BlockAllocator(d["num_blocks"], d["block_size"])
    assert a.allocate("req1", 32) == d["tables"]["req1"]
    assert a.allocate("req2", 48) == d["tables"]["req2"]
    assert a.fork("req1", "req3", 2) == d["tables"]["req3_before_cow"]
    assert {str(b): a.refcount(b) for b in (0, 1)} == d["refcounts_after_share"]
    assert a.cow("req3", 1) == tuple(d["cow_pair"])
    assert a.block_table("req3") == d["tables"]["req3_after_cow"]
    assert {str(b): a.refcount(b) for b in (0, 1, 5)} == d["refcounts_after_cow"]
    assert a.allocate("req4", 64) == d["tables"]["req4"]
    assert a.num_free == d["free_after_schedule"]
    a.check_invariants()
    a.free("req1")
    assert 1 in a.free_blocks() and a.refcount(1) == 0      # block 1 returns at req1's release
    assert 0 not in a.free_blocks() and a.refcount(0) == 1  # block 0 still mapped by req3
    a.free("req2")
    a.free("req3")
    assert a.num_free == d["free_after_release"]
    a.check_invariants()


def test_p1_global_pool_demo_counts():
    d = _demos()["p1_global_pool_demo"]
    a = BlockAllocator(d["num_blocks"], d["block_size"])
    assert a.num_free == d["free_initial"]
    for i, n in enumerate(d["prompts"], start=1):
        a.allocate(i, n)
    assert a.num_free == d["free_after_admit"]
    for _ in range(d["decode_steps"]):
        for i in (1, 2, 3):
            a.append_tokens(i, 1)
    assert a.num_free == d["free_after_decode"]
    a.free(1)
    assert a.num_free == d["free_after_complete_1"]
    a.check_invariants()


def test_cow_only_when_shared():
    a = BlockAllocator(8, 16)
    a.allocate("x", 20)
    assert a.cow("x", 1) is None                 # refcount 1: write in place
    a.fork("x", "y")
    pair = a.cow("y", 1)
    assert pair is not None and pair[0] == a.block_table("x")[1]
    assert a.refcount(pair[0]) == 1 and a.refcount(pair[1]) == 1
    assert a.cow("x", 1) is None                 # x is the only holder again
    a.check_invariants()


def test_append_slot_fresh_block_and_cow():
    a = BlockAllocator(10, 16)
    a.allocate("p", 16)                           # exactly one full block
    slot, pair = a.append_slot("p")               # token 16 opens a fresh block
    assert pair is None and slot == a.block_table("p")[1] * 16
    a.fork("p", "q")                              # q shares both blocks (17 tokens)
    slot, pair = a.append_slot("q")               # token 17 lands in the shared block 1
    assert pair is not None and slot == pair[1] * 16 + 1
    a.check_invariants()


def test_errors_follow_page_conventions():
    a = BlockAllocator(4, 16)
    a.allocate("a", 40)                           # 3 blocks
    with pytest.raises(MemoryError):
        a.allocate("b", 40)                       # needs 3, 1 free
    assert a.num_free == 1                        # nothing half-allocated
    with pytest.raises(KeyError):
        a.block_table("nope")
    with pytest.raises(IndexError):
        a.slot("a", 48)
    with pytest.raises(IndexError):
        a.cow("a", 3)
    a.free("nope")                                # unknown: no-op
    a.check_invariants()


def test_refcount_zero_exactly_when_block_returns():
    """Random allocate / fork / cow / append / free sequences: after every
    operation the free list and the referenced blocks partition the pool, and
    a block sits in the free list exactly when its count is 0."""
    rng = np.random.default_rng(2024)
    for trial in range(20):
        nb = int(rng.integers(8, 64))
        a = BlockAllocator(nb, 16, free_order=rng.permutation(nb))
        live, next_id = [], 0
        for _ in range(200):
            op = rng.integers(0, 5)
            try:
                if op == 0 or not live:
                    a.allocate(next_id, int(rng.integers(0, 60)))
                    live.append(next_id)
                    next_id += 1
                elif op == 1:
                    src = live[int(rng.integers(len(live)))]
                    a.fork(src, next_id)
                    live.append(next_id)
                    next_id += 1
                elif op == 2:
                    a.append_slot(live[int(rng.integers(len(live)))])
                elif op == 3:
                    s = live[int(rng.integers(len(live)))]
                    if a.block_table(s):
                        a.cow(s, int(rng.integers(len(a.block_table(s)))))
                else:
                    s = live.pop(int(rng.integers(len(live))))
                    before = {b: a.refcount(b) for b in a.block_table(s)}
                    a.free(s)
                    for b, rc in before.items():
                        assert (b in a.free_blocks()) == (a.refcount(b) == 0)
            except MemoryError:
                pass
            a.check_invariants()
            free = set(a.free_blocks())
            for b in range(nb):
                assert (b in free) == (a.refcount(b) == 0)
        for s in live:
            a.free(s)
        assert a.num_free == nb


def test_shared_prefix_refcounts():
    """Workload 4: 21 prefix blocks at refcount 8 after the fork; after every
    sample has written its suffix, the 20 full blocks stay at 8, the partly
    filled one is at 1 (7 samples copied it, the last writes in place), and
    freeing everything returns the whole pool."""
    w = make_config(4)
    a = w.allocator
    assert len(w.copy_pairs) == 16 * 7
    for g in range(16):
        seqs = range(g * 8, g * 8 + 8)
        tables = [a.block_table(s) for s in seqs]
        prefix = tables[0][:20]
        for t in tables:
            assert t[:20] == prefix
        assert all(a.refcount(b) == 8 for b in prefix)
        last = [t[20] for t in tables]
        assert len(set(last)) == 8 and all(a.refcount(b) == 1 for b in last)
        srcs = {int(p[0]) for p in w.copy_pairs[g * 7:(g + 1) * 7]}
        assert srcs == {last[7]}                                  # all copied from the original
        assert {int(p[1]) for p in w.copy_pairs[g * 7:(g + 1) * 7]} == set(last[:7])
    a.check_invariants()
    for s in a.sequences():
        a.free(s)
    assert a.num_free == a.num_blocks
    a.check_invariants()


def test_p1_swap_demo_counts():
    d = _demos()["p1_swap_demo"]
    bs = d["block_size"]
    a = BlockAllocator(d["num_blocks"], bs)
    a.allocate(1, d["req1_blocks"] * bs)
    a.allocate(2, d["req2_blocks"] * bs)
    assert a.num_free == d["free_before_swap"]
    sw = SwapSpace(a, d["host_blocks"])
    pairs = sw.swap_out(1)
    assert pairs.shape == (d["req1_blocks"], 2)
    assert a.num_free == d["free_after_swap_out"]
    assert sw.num_free == d["host_free_after_swap_out"]
    assert (a.num_free >= d["req3_blocks_in_demo"]) == d["req3_fits"]
    with pytest.raises(MemoryError):
        a.allocate(3, d["req3_blocks_in_demo"] * bs)
    a.allocate(3, a.num_free * bs)                      # what does fit
    with pytest.raises(MemoryError):                    # no device room to swap back in
        sw.swap_in(1)
    assert sw.swapped() == [1] and sw.num_free == d["host_free_after_swap_out"]
    a.free(3)
    back = sw.swap_in(1)
    assert back.shape == (d["req1_blocks"], 2)
    assert list(back[:, 0]) == list(pairs[:, 1])        # the same host blocks, in order
    assert a.num_free == d["free_before_swap"] and sw.num_free == d["host_blocks"]
    a.check_invariants()
    sw.check_invariants()


def test_swap_space_random_operations_keep_invariants():
    rng = np.random.default_rng(7)
    a = BlockAllocator(64, 16, free_order=rng.permutation(64))
    sw = SwapSpace(a, 48, free_order=rng.permutation(48))
    live, out = set(), set()
    for step in range(400):
        op = rng.integers(0, 5)
        try:
            if op == 0:
                s = int(step)
                a.allocate(s, int(rng.integers(1, 80)))
                live.add(s)
            elif op == 1 and live:
                s = int(rng.choice(sorted(live)))
                a.append_tokens(s, int(rng.integers(1, 20)))
            elif op == 2 and live:
                s = int(rng.choice(sorted(live)))
                table, tokens = a.block_table(s), a.num_tokens(s)
                pairs = sw.swap_out(s)
                assert list(pairs[:, 0]) == table and sw.host_table(s) == list(pairs[:, 1])
                live.discard(s)
                out.add(s)
                assert len(sw.host_table(s)) == len(table)
                assert tokens == (sw._swapped[s][1])
            elif op == 3 and out:
                s = int(rng.choice(sorted(out)))
                host = sw.host_table(s)
                pairs = sw.swap_in(s)
                assert list(pairs[:, 0]) == host and list(pairs[:, 1]) == a.block_table(s)
                out.discard(s)
                live.add(s)
            elif op == 4 and live:
                s = int(rng.choice(sorted(live)))
                a.free(s)
                live.discard(s)
        except MemoryError:
            pass
        a.check_invariants()
        sw.check_invariants()
        assert set(a.sequences()) == live and set(sw.swapped()) == out


def test_swap_out_of_a_shared_prefix_keeps_the_other_readers():
    a = BlockAllocator(16, 16)
    a.allocate("p", 40)                                  # 3 blocks
    a.fork("p", "q")
    sw = SwapSpace(a, 8)
    pairs = sw.swap_out("q")
    assert list(pairs[:, 0]) == a.block_table("p")       # the shared blocks are copied
    assert all(a.refcount(b) == 1 for b in a.block_table("p"))
    assert a.num_free == 13                              # nothing freed: "p" still maps them
    back = sw.swap_in("q")
    assert not set(back[:, 1]) & set(a.block_table("p"))  # private copies now
    sw.swap_out("p")
    with pytest.raises(ValueError):                      # already swapped out
        sw.swap_out("p")
    with pytest.raises(KeyError):
        sw.swap_in("nobody")
    a.check_invariants()
    sw.check_invariants()
