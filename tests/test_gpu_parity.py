"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every test runs one decode step (CoW block copy -> cache write -> decode
attention) on the GPU and on the oracle from the same seeded inputs.
Cache write and block copy: bit-exact over both whole pools. Attention: every
output element finite, max |gpu - oracle| <= 2e-3 and mean <= 2e-4 (the
oracle's float64 result is not rounded; the GPU rounds to fp16/bf16 once).
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_config, make_decode_case, poison_unused
from workloads.device import device_to_bits, device_to_float64, upload

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
MEAN_ABS = 2e-4


def _pkv():
    import paged_kv_cache_159_amd as pkv
    return pkv


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def gpu_step(w, dw, two_stage=False):
    pkv = _pkv()
    if len(w.copy_pairs):
        pkv.copy_blocks(dw.key_cache, dw.value_cache, dw.copy_pairs)
    pkv.reshape_and_cache(dw.new_key, dw.new_value, dw.key_cache, dw.value_cache, dw.slot_mapping)
    ws = pkv.alloc_workspace(w.num_seqs, w.num_heads, w.head_dim, w.max_blocks_per_seq,
                             w.block_size)
    if two_stage:
        pkv.paged_attention_decode_partitions(dw.out, dw.query, dw.key_cache, dw.value_cache,
                                              dw.block_tables, dw.context_lens, w.scale, ws)
        pkv.paged_attention_decode_merge(dw.out, dw.context_lens, w.max_blocks_per_seq, ws,
                                         block_size=w.block_size)
    else:
        pkv.paged_attention_decode(dw.out, dw.query, dw.key_cache, dw.value_cache,
                                   dw.block_tables, dw.context_lens, w.scale, workspace=ws)
    torch.cuda.synchronize()


def oracle_step(w, pairs=None):
    K, V = w.key_cache, w.value_cache
    if len(w.copy_pairs):
        K, V = oracle.copy_blocks(K, V, w.copy_pairs)
    K, V = oracle.reshape_and_cache(w.new_key, w.new_value, K, V, w.slot_mapping, w.block_size)
    out = oracle.paged_attention_decode(w.query, K, V, w.block_tables, w.context_lens, w.scale,
                                        w.block_size, w.dtype, pairs=pairs)
    return K, V, out


def half_ulp(x, dtype):
    """Half the spacing of the output format at |x| (normal range; the
    subnormal spacing below it)."""
    mant, emin = (10, -14) if dtype == "f16" else (7, -126)
    a = np.maximum(np.abs(x), 2.0 ** emin)
    return 0.5 * np.exp2(np.floor(np.log2(a)) - mant)


def assert_attention_close(got, want, pairs=None, what="", format_bound=None):
    """Default: the 2e-3 max / 2e-4 mean bar. With ``format_bound`` (a dtype),
    the per-element bound is the larger of 2e-3 and half an output ulp of the
    value plus 1e-5 (fp32 arithmetic), and the mean bar is dropped: rounding
    a bf16 output of magnitude >= 1 alone can exceed 2e-3 (half an ulp in
    [1, 2) is 3.9e-3), which only happens for very short contexts."""
    if pairs is not None:
        got = np.stack([got[s, h] for s, h in pairs])
        want = np.stack([want[s, h] for s, h in pairs])
    assert np.isfinite(got).all(), f"{what}: non-finite GPU output"
    err = np.abs(got - want)
    worst = np.unravel_index(np.argmax(err), err.shape)
    say(f"{what}: max abs {err.max():.3e} at {worst} (value {want[worst]:.4f}), "
        f"mean abs {err.mean():.3e}")
    if format_bound is None:
        assert err.max() <= MAX_ABS, f"{what}: max abs error {err.max():.3e}"
        assert err.mean() <= MEAN_ABS, f"{what}: mean abs error {err.mean():.3e}"
    else:
        bound = np.maximum(MAX_ABS, half_ulp(np.maximum(np.abs(want), np.abs(got)), format_bound) + 1e-5)
        bad = err > bound
        assert not bad.any(), f"{what}: {bad.sum()} elements beyond half an output ulp + 1e-5"


def check_full_step(w, pairs=None, check_caches=True, two_stage=False, format_bound=None):
    say(f"config {w.index} {w.name}: bs={w.block_size} S={w.num_seqs} H={w.num_heads} D={w.head_dim} {w.dtype} "
        f"NB={w.num_blocks} MB={w.max_blocks_per_seq} T={len(w.slot_mapping)} "
        f"pairs={len(w.copy_pairs)} two_stage={two_stage}")
    dw = upload(w)
    gpu_step(w, dw, two_stage=two_stage)
    K, V, want = oracle_step(w, pairs)
    if check_caches:
        assert np.array_equal(device_to_bits(dw.key_cache), K), "key cache differs"
        assert np.array_equal(device_to_bits(dw.value_cache), V), "value cache differs"
    got = device_to_float64(dw.out)
    assert_attention_close(got, want, pairs, what=f"config {w.index}", format_bound=format_bound)
    return dw, got


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_tiny_step():
    check_full_step(make_config(1))


def test_tiny_canaries_not_read():
    """NaN in every slot that holds no valid token after the step (free blocks,
    rows past the context in last blocks, the slots being written): output
    bit-identical to the clean run and finite."""
    w = make_config(1)
    _, clean = check_full_step(w)
    _, poisoned = check_full_step(poison_unused(w), check_caches=False)
    assert np.array_equal(clean, poisoned)


def test_tiny_permutation_bit_identical():
    """Relabelling physical blocks (pool rows and table entries together, and
    the slots) leaves the GPU output bit-identical."""
    w = make_config(1)
    dw = upload(w)
    gpu_step(w, dw)
    base = device_to_bits(dw.out)
    perm = np.random.default_rng(77).permutation(w.num_blocks)
    import dataclasses
    kc = np.empty_like(w.key_cache)
    vc = np.empty_like(w.value_cache)
    kc[perm] = w.key_cache
    vc[perm] = w.value_cache
    bt = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    slots = perm[w.slot_mapping // 16] * 16 + w.slot_mapping % 16
    w2 = dataclasses.replace(w, key_cache=kc, value_cache=vc, block_tables=bt,
                             slot_mapping=slots.astype(np.int64))
    dw2 = upload(w2)
    gpu_step(w2, dw2)
    assert np.array_equal(device_to_bits(dw2.out), base)


def test_llama7b_step():
    check_full_step(make_config(2))


def test_llama7b_two_stage_equals_single_call():
    w = make_config(2)
    dw = upload(w)
    gpu_step(w, dw)
    one = device_to_bits(dw.out)
    dw2 = upload(w)
    gpu_step(w, dw2, two_stage=True)
    assert np.array_equal(device_to_bits(dw2.out), one)


def test_decode_deterministic():
    w = make_config(2)
    dw = upload(w)
    gpu_step(w, dw)
    a = device_to_bits(dw.out)
    pkv = _pkv()
    ws = pkv.alloc_workspace(w.num_seqs, w.num_heads, w.head_dim, w.max_blocks_per_seq)
    for _ in range(3):
        pkv.paged_attention_decode(dw.out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                                   dw.context_lens, w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(device_to_bits(dw.out), a)


def test_cache_write_step():
    check_full_step(make_config(3))


def test_shared_prefix_step():
    check_full_step(make_config(4))


def test_shared_prefix_canaries_not_read():
    w = poison_unused(make_config(4))
    check_full_step(w, check_caches=True)


def test_long_context_sampled():
    """8 x 32768 tokens (64 partitions per head): caches bit-exact; attention
    on 2 heads of every sequence (each a full 128-element output row)."""
    w = make_config(5)
    rng = np.random.default_rng(5)
    pairs = [(s, int(h)) for s in range(w.num_seqs) for h in rng.choice(w.num_heads, 2, replace=False)]
    dw, got = check_full_step(w, pairs=pairs)
    assert np.isfinite(got).all()


EDGE_CTX = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025, 1536, 2047,
            2048]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_edge_context_lengths(dtype, head_dim):
    """Block and partition boundaries, one-token contexts and the table's
    maximum (128 blocks); 3 heads so heads are not a power of two."""
    w = make_decode_case(EDGE_CTX, 3, head_dim, dtype, seed=head_dim + (dtype == "bf16"),
                         max_blocks=128)
    bound = "bf16" if dtype == "bf16" else None
    _, clean = check_full_step(w, format_bound=bound)
    _, poisoned = check_full_step(poison_unused(w), check_caches=False, format_bound=bound)
    assert np.array_equal(clean, poisoned)


def test_one_token_context_returns_v_exactly():
    """ctx = 1: softmax weight 1, so the output is the written V row itself."""
    w = make_decode_case([1] * 5, 4, 128, "bf16", seed=9)
    dw = upload(w)
    gpu_step(w, dw)
    assert np.array_equal(device_to_bits(dw.out), w.new_value)


def test_single_sequence_and_many_heads():
    w = make_decode_case([777], 64, 128, "f16", seed=4)
    check_full_step(w)


def test_padding_slots_skipped_and_empty_calls():
    pkv = _pkv()
    w = make_config(1)
    dw = upload(w)
    before_k = device_to_bits(dw.key_cache)
    slots = dw.slot_mapping.clone()
    slots[1] = -1
    pkv.reshape_and_cache(dw.new_key, dw.new_value, dw.key_cache, dw.value_cache, slots)
    empty_pairs = torch.zeros(0, 2, dtype=torch.int32, device="cuda")
    pkv.copy_blocks(dw.key_cache, dw.value_cache, empty_pairs)
    pkv.reshape_and_cache(dw.new_key[:0], dw.new_value[:0], dw.key_cache, dw.value_cache, slots[:0])
    torch.cuda.synchronize()
    sl = w.slot_mapping.copy()
    sl[1] = -1
    K, _ = oracle.reshape_and_cache(w.new_key, w.new_value, w.key_cache, w.value_cache, sl, 16)
    after_k = device_to_bits(dw.key_cache)
    assert np.array_equal(after_k, K)
    assert not np.array_equal(after_k, before_k)


def test_copy_blocks_random_pairs_bit_exact():
    pkv = _pkv()
    w = make_config(2)
    rng = np.random.default_rng(12)
    ids = rng.permutation(w.num_blocks)[:600]
    pairs = np.stack([ids[:300], ids[300:]], axis=1).astype(np.int32)
    dw = upload(w)
    pkv.copy_blocks(dw.key_cache, dw.value_cache, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    K, V = oracle.copy_blocks(w.key_cache, w.value_cache, pairs)
    assert np.array_equal(device_to_bits(dw.key_cache), K)
    assert np.array_equal(device_to_bits(dw.value_cache), V)


# ------------------------------------------------------------ grouped (shared prefix)

def grouped_step(w, dw, shared_blocks=None, group_start=None):
    pkv = _pkv()
    if len(w.copy_pairs):
        pkv.copy_blocks(dw.key_cache, dw.value_cache, dw.copy_pairs)
    pkv.reshape_and_cache(dw.new_key, dw.new_value, dw.key_cache, dw.value_cache, dw.slot_mapping)
    gs = torch.from_numpy(np.ascontiguousarray(w.group_start if group_start is None else group_start,
                                               dtype=np.int32)).cuda()
    sb = torch.from_numpy(np.ascontiguousarray(w.shared_blocks if shared_blocks is None
                                               else shared_blocks, dtype=np.int32)).cuda()
    pkv.paged_attention_decode_grouped(dw.out, dw.query, dw.key_cache, dw.value_cache,
                                       dw.block_tables, dw.context_lens, gs, sb, w.scale)
    torch.cuda.synchronize()


def check_grouped(w, shared_blocks=None, group_start=None, format_bound=None, check_caches=True):
    say(f"grouped {w.name}: bs={w.block_size} S={w.num_seqs} H={w.num_heads} D={w.head_dim} {w.dtype} "
        f"groups={len(w.group_start if group_start is None else group_start) - 1} "
        f"shared={(w.shared_blocks if shared_blocks is None else shared_blocks)[:4]}")
    dw = upload(w)
    grouped_step(w, dw, shared_blocks, group_start)
    K, V, want = oracle_step(w)
    if check_caches:
        assert np.array_equal(device_to_bits(dw.key_cache), K), "key cache differs"
        assert np.array_equal(device_to_bits(dw.value_cache), V), "value cache differs"
    got = device_to_float64(dw.out)
    assert_attention_close(got, want, what=f"grouped {w.name}", format_bound=format_bound)
    dw2 = upload(w)
    gpu_step(w, dw2)
    plain = device_to_float64(dw2.out)
    diff = np.abs(got - plain)
    say(f"grouped vs ungrouped: max {diff.max():.3e} mean {diff.mean():.3e}")
    if format_bound is None:
        assert diff.max() <= MAX_ABS
    return got


def test_grouped_shared_prefix():
    """16 prompts x 8 samples, bf16: 20 shared blocks per group on MFMA, tails
    and the CoW-copied partial block on the partition kernel, one merge."""
    check_grouped(make_config(4))


def test_grouped_canaries_not_read():
    w = make_config(4)
    clean = check_grouped(w)
    poisoned = check_grouped(poison_unused(w), check_caches=True)
    assert np.array_equal(clean, poisoned)


def test_grouped_large_groups_head_dim_64():
    """Groups of 20 (two 16-query tiles), a full-block prefix (no CoW), some
    samples with no suffix (whole context shared), 3 heads x 64, fp16."""
    from workloads import make_shared_case
    check_grouped(make_shared_case(2, 20, 80, 0, 30, 3, 64, "f16", seed=5))


def test_grouped_fully_shared_no_tail():
    from workloads import make_shared_case
    w = make_shared_case(3, 4, 64, 0, 0, 4, 128, "bf16", seed=6)
    assert (w.context_lens == 64).all() and (w.shared_blocks == 4).all()
    check_grouped(w, format_bound="bf16")


def test_grouped_without_shared_blocks_matches_plain():
    """shared_blocks = 0: everything runs through the tail partitions."""
    w = make_config(4)
    check_grouped(w, shared_blocks=np.zeros(16, np.int32))


def test_grouped_singleton_groups():
    """One sequence per group, each sharing its own full blocks with itself:
    the MFMA path with a single query per tile."""
    w = make_decode_case([17, 64, 300, 1000, 2048, 33], 4, 128, "f16", seed=21, max_blocks=128)
    gs = np.arange(w.num_seqs + 1, dtype=np.int32)
    sb = ((w.context_lens - 1) // 16).astype(np.int32)
    check_grouped(w, shared_blocks=sb, group_start=gs)


def test_grouped_deterministic():
    w = make_config(4)
    dw = upload(w)
    grouped_step(w, dw)
    a = device_to_bits(dw.out)
    dw2 = upload(w)
    grouped_step(w, dw2)
    assert np.array_equal(device_to_bits(dw2.out), a)


# ------------------------------------------------------------ block sizes 8 and 32

@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_block_size_step(bs, index):
    """The workloads' context lengths over 8- or 32-token blocks (pools and
    tables rebuilt by the allocator at that size), plain decode path."""
    check_full_step(make_config(index, bs))


@pytest.mark.parametrize("bs", [8, 32])
def test_block_size_long_context_sampled(bs):
    w = make_config(5, bs)
    rng = np.random.default_rng(bs)
    pairs = [(s, int(h)) for s in range(w.num_seqs) for h in rng.choice(w.num_heads, 2, replace=False)]
    check_full_step(w, pairs=pairs)


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("dtype,head_dim", [("f16", 128), ("bf16", 64)])
def test_block_size_edge_contexts(bs, dtype, head_dim):
    """Block and partition boundaries at the other block sizes, with NaN
    canaries in every unused slot (output bit-identical to the clean run)."""
    w = make_decode_case(EDGE_CTX, 3, head_dim, dtype, seed=bs + head_dim, max_blocks=2048 // bs,
                         block_size=bs)
    bound = "bf16" if dtype == "bf16" else None
    _, clean = check_full_step(w, format_bound=bound)
    _, poisoned = check_full_step(poison_unused(w), check_caches=False, format_bound=bound)
    assert np.array_equal(clean, poisoned)


@pytest.mark.parametrize("bs", [8, 32])
def test_block_size_grouped_shared_prefix(bs):
    """Shared-prefix workload over 8-token blocks (41 shared blocks: an odd
    last block goes with the tails, no CoW) and 32-token blocks (10 shared
    blocks, each two MFMA tiles; CoW of the partial 11th block)."""
    check_grouped(make_config(4, bs))


@pytest.mark.parametrize("bs", [8, 32])
def test_block_size_grouped_singleton_groups(bs):
    """One sequence per group sharing all its full blocks but the last: odd
    shared-block counts at block size 8 leave half a tile to the tail."""
    w = make_decode_case([17, 64, 300, 1000, 2048, 33, 9], 4, 128, "f16", seed=22 + bs,
                         max_blocks=2048 // bs, block_size=bs)
    gs = np.arange(w.num_seqs + 1, dtype=np.int32)
    sb = ((w.context_lens - 1) // bs).astype(np.int32)
    check_grouped(w, shared_blocks=sb, group_start=gs)


@pytest.mark.parametrize("bs", [8, 32])
def test_block_size_two_stage_equals_single_call(bs):
    w = make_config(2, bs)
    dw1, a = check_full_step(w)
    dw2, b = check_full_step(w, two_stage=True)
    assert np.array_equal(device_to_bits(dw1.out), device_to_bits(dw2.out))
