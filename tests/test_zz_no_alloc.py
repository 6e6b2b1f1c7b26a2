"""paged_attention_decode_noalloc (partials in the library's fixed per-device
scratch array) against paged_attention_decode (partials in a caller
workspace), through the C ABI: bit-identical outputs on two calls in a row,
the second with a smaller input, and the scratch limit refused on the host."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from workloads import make_config, make_decode_case
from workloads.device import device_to_bits, device_to_float64, upload

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _both(w):
    """One decode step's cache write, then the same attention through both
    entry points; returns (noalloc bits, workspace bits, noalloc output)."""
    import paged_kv_cache_159_amd as pkv
    from paged_kv_cache_159_amd._lib import PKV_BF16, PKV_F16
    L = pkv.lib()
    dw = upload(w)
    pkv.reshape_and_cache(dw.new_key, dw.new_value, dw.key_cache, dw.value_cache, dw.slot_mapping)
    ref = torch.empty_like(dw.query)
    pkv.paged_attention_decode(ref, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                               dw.context_lens, w.scale)
    out = torch.full_like(dw.query, float("nan"))
    st = torch.cuda.current_stream().cuda_stream
    rc = L.paged_attention_decode_noalloc(
        out.data_ptr(), dw.query.data_ptr(), dw.key_cache.data_ptr(), dw.value_cache.data_ptr(),
        dw.block_tables.data_ptr(), dw.context_lens.data_ptr(), w.num_seqs, w.num_heads,
        w.head_dim, w.num_blocks, w.block_size, w.max_blocks_per_seq, ctypes.c_float(w.scale),
        PKV_F16 if w.dtype == "f16" else PKV_BF16, ctypes.c_void_p(st))
    assert rc == 0, rc
    torch.cuda.synchronize()
    return device_to_bits(out), device_to_bits(ref), out


def test_noalloc_matches_workspace_call_twice():
    import paged_kv_cache_159_amd as pkv
    # 256 sequences, 8 partitions each slot: 34 MB of partials in the array
    w1 = make_config(3)
    say(f"noalloc call 1: {w1.name} S={w1.num_seqs} MB={w1.max_blocks_per_seq} scratch "
        f"{pkv.workspace_size(w1.num_seqs, w1.num_heads, w1.head_dim, w1.max_blocks_per_seq)} B")
    a, b, _ = _both(w1)
    assert np.array_equal(a, b), "noalloc output differs from the workspace call (large input)"
    # smaller input right after: the array holds the first call's partials
    w2 = make_decode_case([300, 1000, 17, 513, 2048, 1], 4, 128, "bf16", seed=77, max_blocks=128)
    say(f"noalloc call 2: S={w2.num_seqs} ctx={w2.context_lens.tolist()}")
    a, b, out = _both(w2)
    assert np.array_equal(a, b), "noalloc output differs from the workspace call (small input)"
    K, V = oracle.reshape_and_cache(w2.new_key, w2.new_value, w2.key_cache, w2.value_cache,
                                    w2.slot_mapping, w2.block_size)
    want = oracle.paged_attention_decode(w2.query, K, V, w2.block_tables, w2.context_lens,
                                         w2.scale, w2.block_size, w2.dtype)
    err = np.abs(device_to_float64(out) - want)
    assert np.isfinite(err).all() and err.max() <= 4e-3, err.max()   # bf16 outputs >= 1 occur


def test_noalloc_refuses_past_its_scratch():
    import paged_kv_cache_159_amd as pkv
    from paged_kv_cache_159_amd._lib import NOALLOC_SCRATCH_BYTES, PagedKVError
    S, H, D, MB = 1024, 32, 128, 128
    assert pkv.workspace_size(S, H, D, MB) > NOALLOC_SCRATCH_BYTES
    q = torch.zeros(S, H, D, dtype=torch.float16, device="cuda")
    kc = torch.zeros(4, 16, H, D, dtype=torch.float16, device="cuda")
    bt = torch.zeros(S, MB, dtype=torch.int32, device="cuda")
    cl = torch.ones(S, dtype=torch.int32, device="cuda")
    with pytest.raises(PagedKVError, match="PKV_ERR_SCRATCH"):
        pkv.paged_attention_decode_noalloc(torch.empty_like(q), q, kc, kc, bt, cl, 0.125)
