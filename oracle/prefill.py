"""Oracle: multi-token (prefill / chunked-prefill) attention over a paged KV cache, float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix: a prompt's KV is written into pages allocated in one go
at prefill [P1 §3.3.2 "动态页面分配机制", prefill batch allocation: a
320-token prompt takes 20 pages], through the same address translation as
decode [P3 §3.1.3]; prefix pages may be shared at prefill as at decode [P2
"Copy-on-Write共享解码的显存优化原理"].

What the pages leave open, and the reading taken here (plainest one): the
attention of the prompt's tokens is causal scaled dot-product attention. A
call may cover only the last q_len tokens of a sequence (a chunk after a
cached prefix; q_len = context length is a whole prompt, q_len = 1 is
decode): query i of sequence s sits at position p = ctx_s - q_len_s + i and
attends over the tokens 0..p of its sequence, read through its block table,
its own chunk included (the chunk's K/V are in the cache before the call).
"""

from __future__ import annotations

import numpy as np

from .paged_attention import gather_sequence_head, upcast


def causal_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                     first_pos: int) -> np.ndarray:
    """Rows of softmax(scale * Q K^T with keys after each query's position
    masked) V. Q [n, D] are the queries at positions first_pos .. first_pos+n-1;
    K, V [ctx, D] the keys and values at positions 0 .. ctx-1. float64.
    The row maximum is subtracted before exp (a reading: same value).
    Pinned: equals torch's scaled_dot_product_attention with is_causal (whole
    prompt) and with the explicit mask (chunk), and a pure-Python loop.
    """
    n, ctx = Q.shape[0], K.shape[0]
    if first_pos < 0 or first_pos + n > ctx:
        raise ValueError("query positions must lie inside the context")
    X = float(scale) * (Q @ K.T)                                   # [n, ctx]
    pos = first_pos + np.arange(n)[:, None]
    X = np.where(np.arange(ctx)[None, :] <= pos, X, -np.inf)
    W = np.exp(X - X.max(axis=1, keepdims=True))
    W /= W.sum(axis=1, keepdims=True)
    return W @ V


def paged_attention_prefill(query_bits, key_cache_bits, value_cache_bits, block_tables,
                            context_lens, query_start, scale: float, block_size: int,
                            dtype: str, heads=None, seqs=None) -> np.ndarray:
    """Chunked causal attention for every sequence (or the listed ``seqs``)
    and head (or the listed ``heads``).

    query_bits      uint16 [T, H, D], sequence s's queries in rows
                    query_start[s] .. query_start[s+1]-1 (its last q_len_s tokens)
    key/value_cache uint16 [num_blocks, block_size, H, D]
    block_tables    int [S, max_blocks]; context_lens int [S] (after the write)
    Returns float64 [T, H, D]; rows or heads not computed are NaN.
    """
    q_all = np.asarray(query_bits)
    T, H, D = q_all.shape
    qs = np.asarray(query_start, dtype=np.int64)
    S = qs.shape[0] - 1
    if qs[0] != 0 or qs[-1] != T or (np.diff(qs) < 0).any():
        raise ValueError("query_start must rise from 0 to the number of query rows")
    out = np.full((T, H, D), np.nan)
    for s in (range(S) if seqs is None else seqs):
        ctx = int(context_lens[s])
        q0, q1 = int(qs[s]), int(qs[s + 1])
        if q1 == q0:
            continue
        if q1 - q0 > ctx:
            raise ValueError("a chunk longer than its sequence's context")
        for h in (range(H) if heads is None else heads):
            K = gather_sequence_head(key_cache_bits, dtype, block_tables[s], ctx, h, block_size)
            V = gather_sequence_head(value_cache_bits, dtype, block_tables[s], ctx, h, block_size)
            Q = upcast(q_all[q0:q1, h], dtype)
            out[q0:q1, h] = causal_attention(Q, K, V, scale, ctx - (q1 - q0))
    return out
