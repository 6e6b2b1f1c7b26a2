"""Host logic of bench.py (no GPU): the code-only digest that decides whether
committed counter traffic still belongs to the kernels, the algorithmic byte
counts the roofline fractions divide by, and the prefill flop count."""

import os
import shutil

import numpy as np
import pytest

import bench
from workloads import make_config, make_prefill_case


def test_code_only_strips_comments_keeps_literals():
    src = ('int a = 1;  // trailing\n/* block\n comment */ const char* s = "x // y /* z */";\n'
           "char c = '/'; int b = a / 2; // end")
    assert bench._code_only(src) == ('int a = 1; const char* s = "x // y /* z */"; '
                                     "char c = '/'; int b = a / 2;")


def test_code_only_escaped_quote_in_string():
    src = 'const char* s = "a \\" // not a comment"; // comment\nint x;'
    assert bench._code_only(src) == 'const char* s = "a \\" // not a comment"; int x;'


@pytest.mark.parametrize("grouped", [False, True])
def test_digest_follows_code_not_comments(tmp_path, grouped, monkeypatch):
    files = bench.GROUPED_SOURCES if grouped else bench.DECODE_SOURCES
    for p in files:
        dst = tmp_path / p
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, p), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.source_digest(grouped)
    # a comment edit and a re-indented line leave the digest alone
    f = tmp_path / files[1]
    text = f.read_text()
    f.write_text("// a new comment line\n" + text.replace("\n", "\n  ", 3) + "\n/* trailing */\n")
    assert bench.source_digest(grouped) == base
    # a code edit changes it
    f.write_text(text + "\nconstexpr int kDigestProbe = 1;\n")
    assert bench.source_digest(grouped) != base


def test_algorithmic_bytes_llama7b_decode():
    """Workload 2 (64 sequences, 32 x 128 fp16): 63,185 tokens x 16 KiB of K+V,
    q and out (2 x 64 x 8 KiB), 3,977 valid table entries and 64 context
    lengths x 4 B = 1,036,287,780 B, the figure the committed profiles divide by."""
    w = make_config(2)
    assert w.total_context == 63185
    nblocks = int(((w.context_lens.astype(np.int64) + 15) // 16).sum())
    assert nblocks == 3977
    dec, write, copy, logical = bench.algorithmic_bytes(w)
    assert dec == 1_036_287_780 == logical
    assert write == 64 * (2 * 16384 + 8)
    assert copy == 0


def test_unique_bytes_shared_prefix():
    """Workload 4: every physical block's valid rows counted once (the shared
    prefix once per group): 23,461 distinct token rows, 386,497,724 B."""
    w = make_config(4)
    assert bench.unique_kv_tokens(w) == 23461
    dec, _, copy, logical = bench.algorithmic_bytes(w)
    assert dec == 386_497_724
    assert logical > 2.4 * dec
    assert copy == len(w.copy_pairs) * 2 * 2 * 16 * 32 * 128 * 2 + 8 * len(w.copy_pairs)


def test_unique_tokens_brute_force():
    """unique_kv_tokens against a set of (block, row) pairs on a tiny case."""
    w = make_config(1)
    seen = set()
    for s in range(w.num_seqs):
        for t in range(int(w.context_lens[s])):
            seen.add((int(w.block_tables[s, t // w.block_size]), t % w.block_size))
    assert bench.unique_kv_tokens(w) == len(seen)


def test_prefill_flops_brute_force():
    """4 * D flops per (query, visible key) pair per head, counted by loops."""
    w = make_prefill_case([5, 1, 7], [0, 9, 3], 2, 64, "f16", seed=3)
    pairs = 0
    qs = w.query_start
    for s in range(w.num_seqs):
        n = int(qs[s + 1] - qs[s])
        first = int(w.context_lens[s]) - n
        for i in range(n):
            pairs += first + i + 1
    assert bench.prefill_flops(w) == 4 * 64 * 2 * pairs
