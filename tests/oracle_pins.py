"""Pins of the CPU oracle: checks that tie it to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
page's worked example, a closed form, an independent library routine
(torch's scaled_dot_product_attention in float64), brute force on a tiny
input, or an invariant the pages state. The functions look the oracle up
through its modules at call time, so ``test_oracle.py`` can plant a mistake in
the oracle (on the CPU) and check that at least one pin catches it.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from workloads import BlockAllocator

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def page_facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        return json.load(f)


def _sdpa(q, K, V, scale):
    """Library attention in float64 on the CPU: one query row over ctx rows."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None, None, :]
    Kt = torch.from_numpy(np.ascontiguousarray(K, np.float64))[None, None]
    Vt = torch.from_numpy(np.ascontiguousarray(V, np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[0, 0, 0].numpy()


def _torch_upcast(bits, dtype):
    """Independent upcast route through torch's own 16-bit types."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.to(torch.float64).numpy()


def _rand_bits(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def paged_case(seed, ctxs, H, D, dtype, extra_blocks=3, bs=16):
    """Random contiguous K/V per sequence scattered into a shuffled paged pool
    through the allocator's slots (flat index = slot), with NaN in every slot
    that holds no token."""
    rng = np.random.default_rng(seed)
    need = sum((c + bs - 1) // bs for c in ctxs)
    nb = need + extra_blocks
    alloc = BlockAllocator(nb, bs, free_order=rng.permutation(nb))
    nan = np.uint16(0x7E00 if dtype == "f16" else 0x7FC0)
    kc = np.full((nb * bs, H, D), nan, dtype=np.uint16)
    vc = np.full((nb * bs, H, D), nan, dtype=np.uint16)
    Ks, Vs = [], []
    for s, c in enumerate(ctxs):
        alloc.allocate(s, c)
        K = _rand_bits(rng, (c, H, D), dtype)
        V = _rand_bits(rng, (c, H, D), dtype)
        for pos in range(c):
            slot = alloc.slot(s, pos)
            kc[slot] = K[pos]
            vc[slot] = V[pos]
        Ks.append(K)
        Vs.append(V)
    q = _rand_bits(rng, (len(ctxs), H, D), dtype)
    mb = max((c + bs - 1) // bs for c in ctxs)
    tables = alloc.tables_array(list(range(len(ctxs))), mb)
    return dict(q=q, kc=kc.reshape(nb, bs, H, D), vc=vc.reshape(nb, bs, H, D), tables=tables,
                ctx=np.array(ctxs, np.int32), Ks=Ks, Vs=Vs, bs=bs, dtype=dtype, H=H, D=D,
                alloc=alloc)


# --------------------------------------------------------------------------- pins


def pin_translate(pa):
    f = page_facts()
    for e in f["translate"]:
        assert pa.translate(e["token"], e["block_size"]) == (e["logical"], e["offset"])
    for e in f["block_fill"]:
        assert pa.num_logical_blocks(e["tokens"], e["block_size"]) == e["blocks"]
        fill = [sum(1 for t in range(e["tokens"]) if pa.translate(t, e["block_size"])[0] == b)
                for b in range(e["blocks"])]
        assert fill == e["fill"]
    for e in f["block_counts"]:
        assert pa.num_logical_blocks(e["tokens"], e["block_size"]) == e["blocks"]
    mc = f["max_concurrency"]
    assert mc["pool_blocks"] // pa.num_logical_blocks(2048, 16) == mc["requests"]
    bt = f["block_table"]
    a = f["address"]
    assert pa.element_offset(a["table"], a["token"], a["block_size"], a["kv_dim"]) == a["element_offset"]
    # the table example: first token of each logical block lands in its physical block
    for logical, physical in bt["logical_to_physical"]:
        off = pa.element_offset(bt["table"], logical * 16, 16, 1)
        assert off == physical * 16


def pin_upcast(pa):
    cases_f16 = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24, 0x8000: -0.0,
                 0x7C00: math.inf, 0x3555: 0.333251953125}
    cases_bf16 = {0x3F80: 1.0, 0xC000: -2.0, 0x7F7F: 3.3895313892515355e38, 0x0001: 2.0 ** -133,
                  0x7F80: math.inf, 0x3EAB: 0.333984375}
    for dtype, cases in (("f16", cases_f16), ("bf16", cases_bf16)):
        bits = np.array(list(cases), dtype=np.uint16)
        got = pa.upcast(bits, dtype)
        assert list(got) == list(cases.values()), (dtype, got)
        assert np.array_equal(got, _torch_upcast(bits, dtype))
    rng = np.random.default_rng(7)
    for dtype in ("f16", "bf16"):
        bits = _rand_bits(rng, (4096,), dtype)
        assert np.array_equal(pa.upcast(bits, dtype), _torch_upcast(bits, dtype))


def pin_sdpa(pa):
    """Plain attention on contiguous rows equals the library routine."""
    rng = np.random.default_rng(11)
    for ctx, D, scale in ((1, 64, 0.125), (7, 128, 0.08838834764831845), (100, 128, 0.3),
                          (513, 64, 1.7)):
        q = rng.standard_normal(D)
        K = rng.standard_normal((ctx, D))
        V = rng.standard_normal((ctx, D))
        got = pa.attention(q, K, V, scale)
        assert np.allclose(got, _sdpa(q, K, V, scale), rtol=0, atol=1e-12)


def pin_bruteforce(pa):
    """Tiny case against a pure-Python loop with math.exp."""
    rng = np.random.default_rng(3)
    ctx, D, scale = 5, 3, 0.7
    q = rng.standard_normal(D)
    K = rng.standard_normal((ctx, D))
    V = rng.standard_normal((ctx, D))
    x = [scale * sum(q[d] * K[t][d] for d in range(D)) for t in range(ctx)]
    e = [math.exp(v) for v in x]
    z = sum(e)
    want = [sum(e[t] / z * V[t][d] for t in range(ctx)) for d in range(D)]
    got = pa.attention(q, K, V, scale)
    assert np.allclose(got, want, rtol=0, atol=1e-13)


def pin_contiguous(pa):
    """Paged decode equals the library attention over the contiguous rows.
    The rows were placed through the allocator's slots, and every other slot
    holds NaN, so a wrong translation or a read past the context shows. At
    block sizes 8, 16 and 32, with contexts on both sides of block edges."""
    for dtype, H, D, bs in (("f16", 3, 64, 16), ("bf16", 2, 128, 16), ("f16", 2, 64, 8),
                            ("bf16", 3, 64, 32)):
        c = paged_case(21 + bs, [1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 40, 70], H, D, dtype, bs=bs)
        scale = 1.0 / math.sqrt(D)
        out = pa.paged_attention_decode(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], scale,
                                        c["bs"], dtype)
        assert np.isfinite(out).all()
        for s in range(len(c["ctx"])):
            K = _torch_upcast(c["Ks"][s], dtype)
            V = _torch_upcast(c["Vs"][s], dtype)
            q = _torch_upcast(c["q"][s], dtype)
            for h in range(H):
                want = _sdpa(q[h], K[:, h], V[:, h], scale)
                assert np.allclose(out[s, h], want, rtol=0, atol=1e-12), (dtype, bs, s, h)


def pin_permutation(pa):
    """Relabelling physical blocks (pool and tables together) leaves the
    output bit-identical: any free block may serve any sequence."""
    c = paged_case(5, [33, 16, 1, 50], 2, 64, "f16", extra_blocks=5)
    nb = c["kc"].shape[0]
    perm = np.random.default_rng(9).permutation(nb)
    kc2 = np.empty_like(c["kc"])
    vc2 = np.empty_like(c["vc"])
    kc2[perm] = c["kc"]
    vc2[perm] = c["vc"]
    t2 = np.where(c["tables"] >= 0, perm[np.maximum(c["tables"], 0)], -1).astype(np.int32)
    a = pa.paged_attention_decode(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], 0.125, 16, "f16")
    b = pa.paged_attention_decode(c["q"], kc2, vc2, t2, c["ctx"], 0.125, 16, "f16")
    assert np.array_equal(a, b)


def pin_one_token(pa):
    """A one-token context returns that token's V exactly."""
    c = paged_case(8, [1, 1], 2, 128, "bf16")
    out = pa.paged_attention_decode(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], 0.3, 16, "bf16")
    for s in range(2):
        assert np.array_equal(out[s], _torch_upcast(c["Vs"][s][0], "bf16"))


def pin_weights_sum(pa):
    rng = np.random.default_rng(4)
    for ctx in (1, 2, 31, 1000):
        w = pa.softmax_weights(rng.standard_normal(64), rng.standard_normal((ctx, 64)), 0.125)
        assert abs(w.sum() - 1.0) <= 1e-12 and (w >= 0).all()


def pin_partitioned(pa):
    """The split-K form merged by log-sum-exp equals plain attention for any
    partition size."""
    rng = np.random.default_rng(12)
    for ctx in (1, 17, 512, 1500):
        q = rng.standard_normal(128)
        K = rng.standard_normal((ctx, 128)) * 2.0
        V = rng.standard_normal((ctx, 128))
        want = _sdpa(q, K, V, 0.0883883476)
        for part in (1, 16, 512, ctx):
            m, l, o = pa.partitioned_decode_head(q, K, V, 0.0883883476, part)
            assert m.shape[0] == -(-ctx // part)
            got = pa.merge_partitions(m, l, o)
            assert np.allclose(got, want, rtol=0, atol=1e-12), (ctx, part)


def pin_reshape_and_cache(co):
    """Round trip: a written token read back through its slot has the same
    bits; every other slot is untouched; padding slots (-1) are skipped.
    At block sizes 8, 16 and 32."""
    for bs in (8, 16, 32):
        _reshape_round_trip(co, bs)


def _reshape_round_trip(co, bs):
    rng = np.random.default_rng(31 + bs)
    H, D = 2, 64
    alloc = BlockAllocator(12, bs, free_order=rng.permutation(12))
    lens = [5, 16, 31]
    for s, n in enumerate(lens):
        alloc.allocate(s, n)
    slots = [alloc.append_slot(s)[0] for s in range(3)] + [-1]
    kc = rng.integers(0, 1 << 16, size=(12, bs, H, D), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(12, bs, H, D), dtype=np.uint16)
    nk = rng.integers(0, 1 << 16, size=(4, H, D), dtype=np.uint16)
    nv = rng.integers(0, 1 << 16, size=(4, H, D), dtype=np.uint16)
    nk[0, 0, :4] = [0x7E01, 0xFE00, 0x8000, 0x7C00]   # NaN payloads, -0, inf survive
    K2, V2 = co.reshape_and_cache(nk, nv, kc, vc, np.array(slots), bs)
    flatK, flatV = K2.reshape(-1, H, D), V2.reshape(-1, H, D)
    for s, n in enumerate(lens):
        slot = alloc.slot(s, n)
        assert np.array_equal(flatK[slot], nk[s]) and np.array_equal(flatV[slot], nv[s])
    mask = np.ones(12 * bs, bool)
    mask[slots[:3]] = False
    assert np.array_equal(flatK[mask], kc.reshape(-1, H, D)[mask])
    assert np.array_equal(flatV[mask], vc.reshape(-1, H, D)[mask])


def pin_copy_blocks(co):
    rng = np.random.default_rng(32)
    kc = rng.integers(0, 1 << 16, size=(10, 16, 2, 8), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(10, 16, 2, 8), dtype=np.uint16)
    pairs = np.array([[3, 7], [3, 8], [0, 1]])
    K2, V2 = co.copy_blocks(kc, vc, pairs)
    for s, d in pairs:
        assert np.array_equal(K2[d], kc[s]) and np.array_equal(V2[d], vc[s])
    for b in (0, 2, 3, 4, 5, 6, 9):
        assert np.array_equal(K2[b], kc[b]) and np.array_equal(V2[b], vc[b])


def pin_swap_blocks(co):
    """Swap a sequence out to a host pool, let its freed device blocks be
    overwritten, swap it back into whatever blocks the allocator gives: its
    attention through the new table is bit-identical to before; the host
    blocks not written keep their bits; source pools are never changed."""
    from oracle import paged_attention as pa
    from workloads import SwapSpace
    for bs in (8, 16):
        c = paged_case(41 + bs, [20, 33, 50, 7], 2, 64, "f16", extra_blocks=6, bs=bs)
        alloc, kc, vc = c["alloc"], c["kc"], c["vc"]
        rng = np.random.default_rng(bs)
        sw = SwapSpace(alloc, 16, free_order=rng.permutation(16))
        before = pa.paged_attention_decode(c["q"], kc, vc, c["tables"], c["ctx"], 0.125, bs, "f16")
        hk = rng.integers(0, 1 << 16, size=(16, bs, 2, 64), dtype=np.uint16)
        hv = rng.integers(0, 1 << 16, size=(16, bs, 2, 64), dtype=np.uint16)
        kc0, vc0, hk0, hv0 = kc.copy(), vc.copy(), hk.copy(), hv.copy()
        out_pairs = sw.swap_out(1)
        HK, HV = co.swap_blocks(kc, vc, hk, hv, out_pairs)
        assert np.array_equal(kc, kc0) and np.array_equal(vc, vc0)      # source untouched
        held = set(out_pairs[:, 1].tolist())
        for b in range(16):
            if b not in held:
                assert np.array_equal(HK[b], hk0[b]) and np.array_equal(HV[b], hv0[b])
        kc2, vc2 = kc.copy(), vc.copy()
        for b in alloc.free_blocks():                                    # reuse overwrites them
            kc2[b] = rng.integers(0, 1 << 16, size=kc2[b].shape, dtype=np.uint16)
            vc2[b] = rng.integers(0, 1 << 16, size=vc2[b].shape, dtype=np.uint16)
        in_pairs = sw.swap_in(1)
        assert set(in_pairs[:, 1].tolist()) != set(out_pairs[:, 0].tolist())  # other blocks
        K3, V3 = co.swap_blocks(HK, HV, kc2, vc2, in_pairs)
        tables = alloc.tables_array(list(range(4)), c["tables"].shape[1])
        after = pa.paged_attention_decode(c["q"], K3, V3, tables, c["ctx"], 0.125, bs, "f16")
        assert np.array_equal(before, after)
        dst = set(in_pairs[:, 1].tolist())
        for b in range(kc.shape[0]):
            if b not in dst:
                assert np.array_equal(K3[b], kc2[b]) and np.array_equal(V3[b], vc2[b])


ATTENTION_PINS = [pin_translate, pin_upcast, pin_sdpa, pin_bruteforce, pin_contiguous,
                  pin_permutation, pin_one_token, pin_weights_sum, pin_partitioned]
CACHE_PINS = [pin_reshape_and_cache, pin_copy_blocks, pin_swap_blocks]


# --------------------------------------------------------------------------- prefill pins

def _prefill_case(seed, ctxs, qlens, H, D, dtype, bs=16):
    """paged_case plus packed chunk queries: sequence s asks for its last
    qlens[s] tokens."""
    c = paged_case(seed, ctxs, H, D, dtype, bs=bs)
    rng = np.random.default_rng(seed + 100)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int64)
    c["Q"] = _rand_bits(rng, (int(qs[-1]), H, D), dtype)
    c["qs"] = qs
    return c


def _sdpa_masked(Q, K, V, scale, first_pos):
    q = torch.from_numpy(Q)[None, None]
    k = torch.from_numpy(K)[None, None]
    v = torch.from_numpy(V)[None, None]
    n, ctx = Q.shape[0], K.shape[0]
    if first_pos == 0 and n == ctx:
        out = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    else:                             # bottom-right aligned: query i sits at first_pos + i
        mask = torch.arange(ctx)[None, :] <= (first_pos + torch.arange(n))[:, None]
        out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return out[0, 0].numpy()


def pin_prefill_sdpa(pf):
    """Whole prompts (q_len = ctx) equal torch's causal scaled_dot_product_attention
    over the contiguous rows, and chunks (q_len < ctx) equal it with the
    bottom-right causal mask; rows placed through the allocator's slots with
    NaN everywhere else, at block sizes 16 and 8."""
    for bs, ctxs, qlens in ((16, [1, 17, 40, 70], [1, 17, 40, 70]), (16, [33, 70, 5], [8, 1, 5]),
                            (8, [9, 31, 64], [9, 16, 3])):
        c = _prefill_case(61 + bs + len(ctxs), ctxs, qlens, 2, 64, "f16", bs=bs)
        scale = 0.125
        out = pf.paged_attention_prefill(c["Q"], c["kc"], c["vc"], c["tables"], c["ctx"], c["qs"],
                                         scale, bs, "f16")
        assert np.isfinite(out).all()
        for s, (ctx, n) in enumerate(zip(ctxs, qlens)):
            K = _torch_upcast(c["Ks"][s], "f16")
            V = _torch_upcast(c["Vs"][s], "f16")
            Q = _torch_upcast(c["Q"][c["qs"][s]:c["qs"][s + 1]], "f16")
            for h in range(2):
                want = _sdpa_masked(Q[:, h], K[:, h], V[:, h], scale, ctx - n)
                got = out[c["qs"][s]:c["qs"][s + 1], h]
                assert np.allclose(got, want, rtol=0, atol=1e-12), (bs, s, h)


def pin_prefill_decode(pf):
    """One query per sequence (q_len = 1) is the decode of the pinned decode
    oracle."""
    from oracle import paged_attention as pa
    c = _prefill_case(71, [1, 15, 16, 17, 40], [1] * 5, 3, 64, "bf16")
    got = pf.paged_attention_prefill(c["Q"], c["kc"], c["vc"], c["tables"], c["ctx"], c["qs"],
                                     0.2, 16, "bf16")
    want = pa.paged_attention_decode(c["Q"], c["kc"], c["vc"], c["tables"], c["ctx"], 0.2, 16, "bf16")
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def pin_prefill_bruteforce(pf):
    """A 6-token prompt, pure-Python loops and math.exp, causal by hand."""
    c = _prefill_case(72, [6], [6], 1, 4, "f16")
    out = pf.paged_attention_prefill(c["Q"], c["kc"], c["vc"], c["tables"], c["ctx"], c["qs"],
                                     0.5, 16, "f16")
    K = _torch_upcast(c["Ks"][0], "f16")[:, 0].tolist()
    V = _torch_upcast(c["Vs"][0], "f16")[:, 0].tolist()
    Q = _torch_upcast(c["Q"], "f16")[:, 0].tolist()
    for i in range(6):
        xs = [0.5 * sum(Q[i][d] * K[j][d] for d in range(4)) for j in range(i + 1)]
        m = max(xs)
        ws = [math.exp(x - m) for x in xs]
        z = sum(ws)
        for d in range(4):
            want = sum(ws[j] * V[j][d] for j in range(i + 1)) / z
            assert abs(out[i, 0, d] - want) <= 1e-12


def pin_prefill_chunks(pf):
    """Chunks see the cached prefix: the last 20 queries of a 50-token prompt
    asked as one chunk equal the same rows of the whole-prompt call."""
    c = _prefill_case(73, [50], [50], 2, 64, "f16")
    whole = pf.paged_attention_prefill(c["Q"], c["kc"], c["vc"], c["tables"], c["ctx"], c["qs"],
                                       0.125, 16, "f16")
    tail = pf.paged_attention_prefill(c["Q"][30:], c["kc"], c["vc"], c["tables"], c["ctx"],
                                      np.array([0, 20]), 0.125, 16, "f16")
    assert np.allclose(tail, whole[30:], rtol=0, atol=1e-12)


PREFILL_PINS = [pin_prefill_sdpa, pin_prefill_decode, pin_prefill_bruteforce, pin_prefill_chunks]
