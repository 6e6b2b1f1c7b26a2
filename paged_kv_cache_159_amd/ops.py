"""Python binding: torch tensors in, C ABI calls out. Argument marshalling only.

Every function checks devices, dtypes, shapes and contiguity, passes raw
device pointers and torch's current HIP stream to libpaged_kv.so, and raises
``PagedKVError`` on a non-zero status. All computation happens in the
library's kernels; nothing here computes on the tensors.

Tensor layouts (see include/paged_kv.h):
  query, out         [num_seqs, num_heads, head_dim]          float16 | bfloat16
  key/value_cache    [num_blocks, block_size, num_heads, head_dim]  (block_size 8, 16 or 32)
  block_tables       int32 [num_seqs, max_blocks_per_seq]
  context_lens       int32 [num_seqs]
  key, value         [num_tokens, num_heads, head_dim]
  slot_mapping       int64 [num_tokens]
  block_mapping      int32 [num_pairs, 2]  (src, dst)
  host pools         swap_blocks only: [num_cpu_blocks, block_size, num_heads, head_dim]
                     in pinned CPU memory (torch pin_memory=True)

Functions that take the caches read the block size from their shape; a
``block_size`` argument, if given, must agree with it.
"""

from __future__ import annotations

import torch

from ._lib import PKV_BF16, PKV_F16, check, lib

_DTYPES = {torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(*ts) -> int:
    dt = ts[0].dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}; expected float16 or bfloat16")
    for t in ts[1:]:
        if t.dtype != dt:
            raise TypeError(f"dtype mismatch: {t.dtype} vs {dt}")
    return _DTYPES[dt]


def _on_gpu(*ts) -> None:
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU (device 'cuda')")
    for t in ts:
        if t.device != dev:
            raise ValueError(f"device mismatch: {t.device} vs {dev}")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(t: torch.Tensor, dtype, ndim: int, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def workspace_size(num_seqs: int, num_heads: int, head_dim: int, max_blocks_per_seq: int,
                   block_size: int = 16) -> int:
    return int(lib().paged_attention_workspace_size(num_seqs, num_heads, head_dim,
                                                    max_blocks_per_seq, block_size))


def alloc_workspace(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size=16,
                    device="cuda"):
    """A zeroed decode workspace: any content gives the same result, and zeroed
    claim flags let the first of a backed-up item's two workgroups compute it
    (the calls leave the flags at zero)."""
    n = workspace_size(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def _block_size(key_cache, block_size):
    bs = key_cache.shape[1] if key_cache.dim() == 4 else -1
    if block_size is not None and block_size != bs:
        raise ValueError(f"block_size {block_size} disagrees with the cache's {bs}")
    return bs


def _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, block_size):
    _on_gpu(out, query, key_cache, value_cache, block_tables, context_lens)
    dt = _dtype_code(out, query, key_cache, value_cache)
    _expect(block_tables, torch.int32, 2, "block_tables")
    _expect(context_lens, torch.int32, 1, "context_lens")
    if query.dim() != 3 or key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("query [S,H,D] and caches [NB,bs,H,D] expected")
    S, H, D = query.shape
    NB, bs, H2, D2 = key_cache.shape
    _block_size(key_cache, block_size)
    if out.shape != query.shape or (H2, D2) != (H, D):
        raise ValueError("out/query/cache shapes disagree")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables and context_lens need one row per sequence")
    return dt, S, H, D, NB, block_tables.shape[1], bs


def paged_attention_decode(out, query, key_cache, value_cache, block_tables, context_lens,
                           scale: float, block_size: int | None = None,
                           workspace=None) -> torch.Tensor:
    """Decode attention into ``out`` (both launches). Returns ``out``."""
    dt, S, H, D, NB, MB, block_size = _decode_args(out, query, key_cache, value_cache,
                                                   block_tables, context_lens, block_size)
    if workspace is None:
        workspace = alloc_workspace(S, H, D, MB, block_size, out.device)
    rc = lib().paged_attention_decode(out.data_ptr(), query.data_ptr(), key_cache.data_ptr(),
                                      value_cache.data_ptr(), block_tables.data_ptr(),
                                      context_lens.data_ptr(), S, H, D, NB, block_size, MB,
                                      float(scale), dt, workspace.data_ptr(), workspace.numel(),
                                      _stream(out))
    check("paged_attention_decode", rc)
    return out


def paged_attention_decode_noalloc(out, query, key_cache, value_cache, block_tables,
                                   context_lens, scale: float,
                                   block_size: int | None = None) -> torch.Tensor:
    """paged_attention_decode without a workspace: the library's fixed
    per-device scratch array holds the partials, and nothing is allocated.
    Calls overlapping on one GPU race on that array. Returns ``out``."""
    dt, S, H, D, NB, MB, block_size = _decode_args(out, query, key_cache, value_cache,
                                                   block_tables, context_lens, block_size)
    rc = lib().paged_attention_decode_noalloc(out.data_ptr(), query.data_ptr(),
                                              key_cache.data_ptr(), value_cache.data_ptr(),
                                              block_tables.data_ptr(), context_lens.data_ptr(),
                                              S, H, D, NB, block_size, MB, float(scale), dt,
                                              _stream(out))
    check("paged_attention_decode_noalloc", rc)
    return out


def grouped_workspace_size(num_seqs: int, num_heads: int, head_dim: int,
                           max_blocks_per_seq: int, block_size: int = 16) -> int:
    return int(lib().paged_attention_grouped_workspace_size(num_seqs, num_heads, head_dim,
                                                            max_blocks_per_seq, block_size))


def paged_attention_decode_grouped(out, query, key_cache, value_cache, block_tables, context_lens,
                                   group_start, shared_blocks, scale: float,
                                   block_size: int | None = None,
                                   workspace=None) -> torch.Tensor:
    """Decode attention with shared prefix blocks read once per group (MFMA).
    group_start: int32 [G+1]; shared_blocks: int32 [G] (see include/paged_kv.h)."""
    dt, S, H, D, NB, MB, block_size = _decode_args(out, query, key_cache, value_cache,
                                                   block_tables, context_lens, block_size)
    _on_gpu(out, group_start, shared_blocks)
    _expect(group_start, torch.int32, 1, "group_start")
    _expect(shared_blocks, torch.int32, 1, "shared_blocks")
    G = shared_blocks.shape[0]
    if group_start.shape[0] != G + 1:
        raise ValueError("group_start needs num_groups + 1 entries")
    if workspace is None:
        n = grouped_workspace_size(S, H, D, MB, block_size)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=out.device)
    rc = lib().paged_attention_decode_grouped(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), group_start.data_ptr(),
        shared_blocks.data_ptr(), G, S, H, D, NB, block_size, MB, float(scale), dt,
        workspace.data_ptr(), workspace.numel(), _stream(out))
    check("paged_attention_decode_grouped", rc)
    return out


def paged_attention_prefill(out, query, key_cache, value_cache, block_tables, context_lens,
                            query_start, scale: float, max_query_len: int | None = None,
                            block_size: int | None = None) -> torch.Tensor:
    """Causal attention of each sequence's chunk of new tokens (packed rows
    query_start[s] .. query_start[s+1] of query and out, [T, H, D]) over its
    paged context; the chunk's K/V must already be in the cache. Returns out.
    ``max_query_len`` bounds every chunk; if omitted it is read from
    query_start (one device-to-host copy)."""
    _on_gpu(out, query, key_cache, value_cache, block_tables, context_lens, query_start)
    dt = _dtype_code(out, query, key_cache, value_cache)
    _expect(block_tables, torch.int32, 2, "block_tables")
    _expect(context_lens, torch.int32, 1, "context_lens")
    _expect(query_start, torch.int32, 1, "query_start")
    if query.dim() != 3 or key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("query [T,H,D] and caches [NB,bs,H,D] expected")
    T, H, D = query.shape
    NB, bs, H2, D2 = key_cache.shape
    _block_size(key_cache, block_size)
    if out.shape != query.shape or (H2, D2) != (H, D):
        raise ValueError("out/query/cache shapes disagree")
    S = context_lens.shape[0]
    if block_tables.shape[0] != S or query_start.shape[0] != S + 1:
        raise ValueError("block_tables needs S rows and query_start S + 1 entries")
    if max_query_len is None:
        max_query_len = int(torch.diff(query_start).max().item()) if S else 0
    rc = lib().paged_attention_prefill(out.data_ptr(), query.data_ptr(), key_cache.data_ptr(),
                                       value_cache.data_ptr(), block_tables.data_ptr(),
                                       context_lens.data_ptr(), query_start.data_ptr(), S,
                                       int(max_query_len), H, D, NB, bs, block_tables.shape[1],
                                       float(scale), dt, _stream(out))
    check("paged_attention_prefill", rc)
    return out


def paged_attention_decode_partitions(out, query, key_cache, value_cache, block_tables,
                                      context_lens, scale: float, workspace,
                                      block_size: int | None = None) -> None:
    dt, S, H, D, NB, MB, block_size = _decode_args(out, query, key_cache, value_cache,
                                                   block_tables, context_lens, block_size)
    rc = lib().paged_attention_decode_partitions(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), S, H, D, NB, block_size, MB,
        float(scale), dt, workspace.data_ptr(), workspace.numel(), _stream(out))
    check("paged_attention_decode_partitions", rc)


def paged_attention_decode_merge(out, context_lens, max_blocks_per_seq: int, workspace,
                                 block_size: int = 16) -> None:
    _on_gpu(out, context_lens, workspace)
    dt = _dtype_code(out)
    _expect(context_lens, torch.int32, 1, "context_lens")
    S, H, D = out.shape
    rc = lib().paged_attention_decode_merge(out.data_ptr(), context_lens.data_ptr(), S, H, D,
                                            block_size, max_blocks_per_seq, dt,
                                            workspace.data_ptr(), workspace.numel(), _stream(out))
    check("paged_attention_decode_merge", rc)


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping,
                      block_size: int | None = None):
    """Scatter new tokens' K/V rows into their slots (in place)."""
    _on_gpu(key, value, key_cache, value_cache, slot_mapping)
    dt = _dtype_code(key, value, key_cache, value_cache)
    _expect(slot_mapping, torch.int64, 1, "slot_mapping")
    if key.dim() != 3 or key.shape != value.shape or key_cache.dim() != 4:
        raise ValueError("key/value [T,H,D] and caches [NB,bs,H,D] expected")
    T, H, D = key.shape
    NB, bs, H2, D2 = key_cache.shape
    block_size = _block_size(key_cache, block_size)
    if value_cache.shape != key_cache.shape or (H2, D2) != (H, D):
        raise ValueError("key/value and cache shapes disagree")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping needs one entry per token")
    rc = lib().reshape_and_cache(key.data_ptr(), value.data_ptr(), key_cache.data_ptr(),
                                 value_cache.data_ptr(), slot_mapping.data_ptr(), T, H, D, NB,
                                 block_size, dt, _stream(key))
    check("reshape_and_cache", rc)


def copy_blocks(key_cache, value_cache, block_mapping, block_size: int | None = None):
    """Copy whole blocks src -> dst in both pools (in place)."""
    _on_gpu(key_cache, value_cache, block_mapping)
    dt = _dtype_code(key_cache, value_cache)
    _expect(block_mapping, torch.int32, 2, "block_mapping")
    if key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("caches [NB,bs,H,D] expected")
    if block_mapping.shape[0] and block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [P, 2]")
    NB, bs, H, D = key_cache.shape
    block_size = _block_size(key_cache, block_size)
    rc = lib().copy_blocks(key_cache.data_ptr(), value_cache.data_ptr(), block_mapping.data_ptr(),
                           block_mapping.shape[0], H, D, NB, block_size, dt, _stream(key_cache))
    check("copy_blocks", rc)


def _pool_tensor(t, name):
    if t.device.type == "cpu" and not t.is_pinned():
        raise ValueError(f"{name} is in pageable host memory; swap pools on the host must be "
                         "pinned (pin_memory=True)")
    if t.device.type not in ("cpu", "cuda"):
        raise ValueError(f"{name} must be a GPU tensor or a pinned CPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def swap_blocks(src_key, src_value, dst_key, dst_value, block_mapping, method: str = "kernel",
                staging=None):
    """Copy whole blocks src -> dst from the (src_key, src_value) pools into the
    (dst_key, dst_value) pools, one of which lives in pinned host memory:
    swap-out (device -> host) or swap-in (host -> device), on the current
    stream of the GPU involved.
    method "kernel": one launch; ``block_mapping`` int32 [P, 2] on that GPU or
    pinned. method "dma": DMA copies per run of consecutive blocks;
    ``block_mapping`` int32 [P, 2] on the CPU (read during the call).
    method "staged": DMA of runs of consecutive source blocks into ``staging``
    (a uint8 GPU tensor), then one scatter launch per chunk; mapping on the
    CPU."""
    if method not in ("kernel", "dma", "staged"):
        raise ValueError("method must be 'kernel', 'dma' or 'staged'")
    if method != "kernel" and block_mapping.device.type != "cpu":
        raise ValueError(f"method '{method}' reads block_mapping on the host: pass a CPU tensor")
    if method == "staged" and (staging is None or staging.device.type != "cuda"):
        raise ValueError("method 'staged' needs a GPU staging tensor")
    for t, n in ((src_key, "src_key"), (src_value, "src_value"), (dst_key, "dst_key"),
                 (dst_value, "dst_value")):
        _pool_tensor(t, n)
    if method == "kernel":
        _pool_tensor(block_mapping, "block_mapping")
    elif not block_mapping.is_contiguous():
        raise ValueError("block_mapping must be contiguous")
    dt = _dtype_code(src_key, src_value, dst_key, dst_value)
    _expect(block_mapping, torch.int32, 2, "block_mapping")
    if block_mapping.shape[0] and block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [P, 2]")
    if src_key.dim() != 4 or src_value.shape != src_key.shape or dst_value.shape != dst_key.shape:
        raise ValueError("pools [NB,bs,H,D] expected, K and V alike")
    NBs, bs, H, D = src_key.shape
    NBd, bs2, H2, D2 = dst_key.shape
    if (bs2, H2, D2) != (bs, H, D):
        raise ValueError("source and destination pools disagree in block_size, heads or head_dim")
    gpus = {t.device for t in (src_key, src_value, dst_key, dst_value, block_mapping)
            if t.device.type == "cuda"}
    if len(gpus) != 1:
        raise ValueError("exactly one GPU must be involved")
    dev = next(iter(gpus))
    st = torch.cuda.current_stream(dev).cuda_stream
    args = (src_key.data_ptr(), src_value.data_ptr(), dst_key.data_ptr(), dst_value.data_ptr(),
            block_mapping.data_ptr(), block_mapping.shape[0], H, D, NBs, NBd, bs, dt)
    if method == "staged":
        fn = "swap_blocks_staged"
        rc = lib().swap_blocks_staged(*args, staging.data_ptr(), staging.numel(), st)
    else:
        fn = "swap_blocks" if method == "kernel" else "swap_blocks_dma"
        rc = getattr(lib(), fn)(*args, st)
    check(fn, rc)
