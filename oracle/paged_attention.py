"""Oracle: single-query decode attention over a paged KV cache, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix, and where:
  * Address translation [P3 §3.1.3 "逻辑地址到物理地址的转换" (logical-to-physical
    address translation); P4 "疑问 1 ... 转化" (translation); P2 "KV Cache逻辑块物理块映射
    机制" (logical/physical block mapping)]: for token t of a sequence,
    logical block = t // block_size, offset = t % block_size, physical block =
    block_table[logical]; the element address inside a pool is
    physical * block_size * kv_dim + offset * kv_dim.
  * Pool layout [P3 §3.1.2 "页面结构设计" (page structure)]: a page holds
    block_size tokens; each token holds a Key row and a Value row of
    num_heads * head_dim elements (separate Key cache and Value cache).
  * Paging changes where K/V live, not what is computed [P3 §3.1.1, the
    PagedAttention advantages list: no extra computation]. So the result is the
    plain attention of the query over the sequence's tokens in logical order.

What the pages leave open, and the reading taken here (plainest one):
  * The attention formula is not on the pages. Reading: scaled dot-product
    attention with a caller-supplied scale, x_t = scale * <q, K_t>,
    w = softmax(x), out = sum_t w_t V_t, one query per (sequence, head).
  * Inside a token row the order is [head][dim] (kv_dim = num_heads*head_dim).
  * Rows of the last block at positions >= context length are never read, nor
    are block-table entries past ceil(ctx / block_size).
  * Stored fp16/bf16 values are upcast exactly to float64; the result is kept
    in float64 (never rounded to the storage type).
"""

from __future__ import annotations

import numpy as np

_FP16 = "f16"
_BF16 = "bf16"


def translate(t: int, block_size: int) -> tuple[int, int]:
    """Logical block and in-block offset of token ``t``.

    [P3 §3.1.3 steps 1-2; P4 "疑问 1" steps 1-2: token 35 with block size 16
    lies in logical block 2 at offset 3.] Pinned by that worked example.
    """
    if t < 0 or block_size <= 0:
        raise ValueError("token index must be >= 0 and block_size > 0")
    return t // block_size, t % block_size


def num_logical_blocks(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` tokens occupies: ceil division.

    [P2 "KV Cache逻辑块物理块映射机制": 35 tokens need 3 blocks (16, 16, 3);
    P1 §3.3.2 "动态页面分配机制": a 320-token prompt needs 20 pages.]
    Pinned by those examples and by the demo comments of P1 §3.3.4.
    """
    if num_tokens < 0:
        raise ValueError("num_tokens must be >= 0")
    return (num_tokens + block_size - 1) // block_size


def element_offset(block_table_row, t: int, block_size: int, kv_dim: int) -> int:
    """Element offset of token ``t``'s row inside one K (or V) pool.

    [P3 §3.1.3 steps 3-4]: physical = block_table[logical];
    address = physical * block_size * kv_dim + offset * kv_dim.
    Pinned by the block table [3, 7, 12] of P2 "KV Cache逻辑块物理块映射机制"
    combined with the token-35 example of P4.
    """
    logical, offset = translate(t, block_size)
    if logical >= len(block_table_row):
        raise IndexError(f"logical block {logical} beyond the block table")
    physical = int(block_table_row[logical])
    return physical * block_size * kv_dim + offset * kv_dim


def upcast(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored 16-bit words.

    fp16: IEEE binary16 reinterpretation. bf16: the top 16 bits of an IEEE
    binary32, so the value is the word shifted left by 16 and reinterpreted.
    Both conversions to float64 are exact. Pinned by known bit patterns
    (1.0, -2.0, largest finite, infinity).
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("expected uint16 bit patterns")
    if dtype == _FP16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == _BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def gather_sequence_head(cache_bits: np.ndarray, dtype: str, block_table_row, ctx: int,
                         head: int, block_size: int) -> np.ndarray:
    """Rows [ctx, head_dim] of one head of one sequence, in logical order, float64.

    Each token t in [0, ctx) is translated [P3 §3.1.3] and its row read from
    pool[physical, offset, head, :]. Tokens >= ctx, and table entries past
    ceil(ctx / block_size), are not touched. Pinned: equal to a contiguous
    layout (identity table) and invariant under relabelling of physical ids.
    """
    if ctx < 1:
        raise ValueError("context length must be >= 1")
    t = np.arange(ctx)
    logical = t // block_size
    offset = t % block_size
    table = np.asarray(block_table_row)
    if logical[-1] >= table.shape[0]:
        raise IndexError("context longer than the block table")
    physical = table[logical].astype(np.int64)
    if physical.min() < 0 or physical.max() >= cache_bits.shape[0]:
        raise IndexError("block table entry outside the pool")
    return upcast(cache_bits[physical, offset, head, :], dtype)


def softmax_weights(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Attention weights of one query over rows K: softmax(scale * K q), float64.

    The maximum is subtracted before exp (a reading: it does not change the
    value). Pinned: weights sum to 1; the full attention equals torch's
    scaled_dot_product_attention in float64 and a pure-Python loop.
    """
    x = float(scale) * (K @ q)
    w = np.exp(x - x.max())
    return w / w.sum()


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """out = sum_t w_t V_t with w = softmax(scale * K q); float64 in and out."""
    return softmax_weights(q, K, scale) @ V


def paged_attention_decode(query_bits, key_cache_bits, value_cache_bits, block_tables,
                           context_lens, scale: float, block_size: int, dtype: str,
                           pairs=None) -> np.ndarray:
    """Decode attention for every (sequence, head), or for the listed ``pairs``.

    query_bits        uint16 [S, H, D]
    key/value_cache   uint16 [num_blocks, block_size, H, D]
    block_tables      int    [S, max_blocks_per_seq]
    context_lens      int    [S]
    Returns float64 [S, H, D] (entries not in ``pairs`` are NaN when ``pairs``
    is given, so a caller cannot mistake them for computed values).

    For each (s, h): gather K and V through the block table, then plain
    attention [P3 §3.1.3 translation; reading of the formula in the module
    docstring].
    """
    q_all = np.asarray(query_bits)
    S, H, D = q_all.shape
    if key_cache_bits.shape[1] != block_size or key_cache_bits.shape[2:] != (H, D):
        raise ValueError("cache shape does not match [num_blocks, block_size, H, D]")
    out = np.full((S, H, D), np.nan if pairs is not None else 0.0, dtype=np.float64)
    todo = pairs if pairs is not None else [(s, h) for s in range(S) for h in range(H)]
    for s, h in todo:
        ctx = int(context_lens[s])
        K = gather_sequence_head(key_cache_bits, dtype, block_tables[s], ctx, h, block_size)
        V = gather_sequence_head(value_cache_bits, dtype, block_tables[s], ctx, h, block_size)
        q = upcast(q_all[s, h], dtype)
        out[s, h] = attention(q, K, V, scale)
    return out


def partitioned_decode_head(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                            partition_tokens: int):
    """Split-K form of one head's attention: per-partition partials, then merge.

    The context is cut into consecutive partitions of ``partition_tokens``
    tokens (the last may be shorter). For partition p over tokens T_p:
      m_p = max_{t in T_p} x_t,  l_p = sum exp(x_t - m_p),
      o_p = sum exp(x_t - m_p) V_t / l_p.
    Returns (m, l, o) as arrays [P], [P], [P, D]. The pages do not describe a
    partitioned form; this is the log-sum-exp decomposition of the softmax, and
    ``merge_partitions`` of it must equal ``attention`` (pinned in the tests for
    partition sizes 1, 16, 512 and the whole context).
    """
    x = float(scale) * (K @ q)
    ctx = x.shape[0]
    ms, ls, os_ = [], [], []
    for start in range(0, ctx, partition_tokens):
        xs = x[start:start + partition_tokens]
        m = xs.max()
        e = np.exp(xs - m)
        ms.append(m)
        ls.append(e.sum())
        os_.append((e @ V[start:start + partition_tokens]) / e.sum())
    return np.array(ms), np.array(ls), np.array(os_)


def merge_partitions(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Log-sum-exp merge of partition partials:
    M = max_p m_p, c_p = l_p exp(m_p - M), out = sum_p c_p o_p / sum_p c_p."""
    M = m.max()
    c = l * np.exp(m - M)
    return (c @ o) / c.sum()
