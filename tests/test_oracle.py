"""The CPU oracle against its pins, and planted mistakes that the pins must catch."""

import numpy as np
import pytest

import oracle
from oracle import cache_ops as co
from oracle import paged_attention as pa

from oracle_pins import ATTENTION_PINS, CACHE_PINS


@pytest.mark.parametrize("pin", ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_pin(pin):
    pin(pa)


@pytest.mark.parametrize("pin", CACHE_PINS, ids=lambda f: f.__name__)
def test_cache_pin(pin):
    pin(co)


def test_translate_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.translate(-1, 16)
    with pytest.raises(IndexError):
        oracle.element_offset([3, 7, 12], 48, 16, 256)


def test_gather_rejects_table_outside_pool():
    kc = np.zeros((2, 16, 1, 8), np.uint16)
    with pytest.raises(IndexError):
        oracle.gather_sequence_head(kc, "f16", [5], 3, 0, 16)
    with pytest.raises(IndexError):
        oracle.gather_sequence_head(kc, "f16", [0], 17, 0, 16)


def test_cache_ops_refuse_ambiguous_inputs():
    kc = np.zeros((4, 16, 1, 8), np.uint16)
    k = np.ones((2, 1, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(k, k, kc, kc, [3, 3], 16)
    with pytest.raises(IndexError):
        oracle.reshape_and_cache(k, k, kc, kc, [3, 64], 16)
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, kc, [[0, 1], [2, 1]])
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, kc, [[0, 1], [1, 2]])
    with pytest.raises(IndexError):
        oracle.copy_blocks(kc, kc, [[0, 4]])


# ---------------------------------------------------------------- planted mistakes
# Each mutant replaces one oracle function with a plausible wrong version. The
# pins, run against the mutated oracle, must fail at least once.

def _gather_swapped(cache_bits, dtype, row, ctx, head, bs):
    t = np.arange(ctx)
    return pa.upcast(cache_bits[np.asarray(row)[t % bs], t // bs, head, :], dtype)


def _gather_shifted(cache_bits, dtype, row, ctx, head, bs):
    t = np.arange(ctx) + 1
    return pa.upcast(cache_bits[np.asarray(row)[t // bs], t % bs, head, :], dtype)


def _gather_one_short(cache_bits, dtype, row, ctx, head, bs):
    t = np.arange(max(ctx - 1, 1))
    return pa.upcast(cache_bits[np.asarray(row)[t // bs], t % bs, head, :], dtype)


def _weights_no_scale(q, K, scale):
    x = K @ q
    w = np.exp(x - x.max())
    return w / w.sum()


def _weights_sign(q, K, scale):
    x = scale * (K @ q)
    w = np.exp(x.max() - x)
    return w / w.sum()


def _weights_unnormalised(q, K, scale):
    x = scale * (K @ q)
    return np.exp(x - x.max())


def _attention_kv_swapped(q, K, V, scale):
    return pa.softmax_weights(q, V, scale) @ K


def _merge_without_l(m, l, o):
    M = m.max()
    c = np.exp(m - M)
    return (c @ o) / c.sum()


def _partitioned_unnormalised(q, K, V, scale, part):
    x = scale * (K @ q)
    ms, ls, os_ = [], [], []
    for s in range(0, x.shape[0], part):
        xs = x[s:s + part]
        e = np.exp(xs - xs.max())
        ms.append(xs.max())
        ls.append(e.sum())
        os_.append(e @ V[s:s + part])
    return np.array(ms), np.array(ls), np.array(os_)


def _upcast_bf16_wrong(bits, dtype):
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def _translate_ceil(t, bs):
    return -(-t // bs), t % bs


def _offset_transposed(row, t, bs, kv_dim):
    lg, off = pa.translate(t, bs)
    return int(row[lg]) * kv_dim + off * bs * kv_dim


ATTN_MUTANTS = {
    "gather_swapped": ("gather_sequence_head", _gather_swapped),
    "gather_shifted": ("gather_sequence_head", _gather_shifted),
    "gather_one_short": ("gather_sequence_head", _gather_one_short),
    "weights_no_scale": ("softmax_weights", _weights_no_scale),
    "weights_sign": ("softmax_weights", _weights_sign),
    "weights_unnormalised": ("softmax_weights", _weights_unnormalised),
    "attention_kv_swapped": ("attention", _attention_kv_swapped),
    "merge_without_l": ("merge_partitions", _merge_without_l),
    "partitioned_unnormalised": ("partitioned_decode_head", _partitioned_unnormalised),
    "upcast_bf16_wrong": ("upcast", _upcast_bf16_wrong),
    "translate_ceil": ("translate", _translate_ceil),
    "offset_transposed": ("element_offset", _offset_transposed),
}


def _fails_some_pin(pins, module):
    for pin in pins:
        try:
            pin(module)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_pins_catch_planted_attention_mistake(name, monkeypatch):
    attr, fn = ATTN_MUTANTS[name]
    monkeypatch.setattr(pa, attr, fn)
    with np.errstate(all="ignore"):
        assert _fails_some_pin(ATTENTION_PINS, pa), f"no pin caught mutant {name}"


def _write_swapped(key_bits, value_bits, kc, vc, slots, bs):
    K, V = kc.copy(), vc.copy()
    for i, s in enumerate(np.asarray(slots).tolist()):
        if s >= 0:
            K[s % kc.shape[0], s // kc.shape[0] % bs] = key_bits[i]
            V[s % kc.shape[0], s // kc.shape[0] % bs] = value_bits[i]
    return K, V


def _write_drops_value(key_bits, value_bits, kc, vc, slots, bs):
    K, V = kc.copy(), vc.copy()
    for i, s in enumerate(np.asarray(slots).tolist()):
        if s >= 0:
            K[s // bs, s % bs] = key_bits[i]
    return K, V


def _copy_reversed(kc, vc, pairs):
    K, V = kc.copy(), vc.copy()
    for s, d in np.asarray(pairs).tolist():
        K[s] = kc[d]
        V[s] = vc[d]
    return K, V


def _copy_key_only(kc, vc, pairs):
    K = kc.copy()
    for s, d in np.asarray(pairs).tolist():
        K[d] = kc[s]
    return K, vc.copy()


def _swap_reversed(sk, sv, dk, dv, pairs):
    K, V = dk.copy(), dv.copy()
    for s, d in np.asarray(pairs).tolist():
        if s < K.shape[0] and d < sk.shape[0]:
            K[s] = sk[d]
            V[s] = sv[d]
    return K, V


def _swap_key_only(sk, sv, dk, dv, pairs):
    K = dk.copy()
    for s, d in np.asarray(pairs).tolist():
        K[d] = sk[s]
    return K, dv.copy()


CACHE_MUTANTS = {
    "swap_reversed": ("swap_blocks", _swap_reversed),
    "swap_key_only": ("swap_blocks", _swap_key_only),
    "write_swapped": ("reshape_and_cache", _write_swapped),
    "write_drops_value": ("reshape_and_cache", _write_drops_value),
    "copy_reversed": ("copy_blocks", _copy_reversed),
    "copy_key_only": ("copy_blocks", _copy_key_only),
}


@pytest.mark.parametrize("name", sorted(CACHE_MUTANTS))
def test_pins_catch_planted_cache_mistake(name, monkeypatch):
    attr, fn = CACHE_MUTANTS[name]
    monkeypatch.setattr(co, attr, fn)
    with np.errstate(all="ignore"):                 # a mutant may leave NaN canaries in play
        assert _fails_some_pin(CACHE_PINS, co), f"no pin caught mutant {name}"


# --------------------------------------------------------------------------- prefill

from oracle import prefill as pf  # noqa: E402
from oracle_pins import PREFILL_PINS  # noqa: E402


@pytest.mark.parametrize("pin", PREFILL_PINS, ids=lambda f: f.__name__)
def test_prefill_pin(pin):
    pin(pf)


def test_prefill_refuses_bad_chunks():
    kc = np.zeros((2, 16, 1, 8), np.uint16)
    q = np.zeros((5, 1, 8), np.uint16)
    with pytest.raises(ValueError):                       # chunk longer than the context
        oracle.paged_attention_prefill(q, kc, kc, [[0, 1]], [4], [0, 5], 1.0, 16, "f16")
    with pytest.raises(ValueError):                       # query_start must cover the rows
        oracle.paged_attention_prefill(q, kc, kc, [[0, 1]], [8], [0, 4], 1.0, 16, "f16")


def _mask(ctx, n, first_pos, strict=False):
    pos = first_pos + np.arange(n)[:, None]
    j = np.arange(ctx)[None, :]
    return (j < pos) if strict else (j <= pos)


def _softmax_rows(X):
    W = np.exp(X - X.max(axis=1, keepdims=True))
    return W / W.sum(axis=1, keepdims=True)


def _ca_no_mask(Q, K, V, scale, first_pos):
    return _softmax_rows(scale * (Q @ K.T)) @ V


def _ca_no_diagonal(Q, K, V, scale, first_pos):
    X = np.where(_mask(K.shape[0], Q.shape[0], first_pos, strict=True), scale * (Q @ K.T), -np.inf)
    X[:, 0] = np.where(np.isinf(X[:, 0]), 0.0, X[:, 0])     # keep rows finite
    return _softmax_rows(X) @ V


def _ca_top_left(Q, K, V, scale, first_pos):
    X = np.where(_mask(K.shape[0], Q.shape[0], 0), scale * (Q @ K.T), -np.inf)
    return _softmax_rows(X) @ V


def _ca_no_scale(Q, K, V, scale, first_pos):
    X = np.where(_mask(K.shape[0], Q.shape[0], first_pos), Q @ K.T, -np.inf)
    return _softmax_rows(X) @ V


def _ca_k_for_v(Q, K, V, scale, first_pos):
    X = np.where(_mask(K.shape[0], Q.shape[0], first_pos), scale * (Q @ K.T), -np.inf)
    return _softmax_rows(X) @ K


PREFILL_MUTANTS = {
    "no_causal_mask": _ca_no_mask,
    "mask_drops_diagonal": _ca_no_diagonal,
    "mask_top_left_aligned": _ca_top_left,
    "scale_dropped": _ca_no_scale,
    "keys_for_values": _ca_k_for_v,
}


@pytest.mark.parametrize("name", sorted(PREFILL_MUTANTS))
def test_pins_catch_planted_prefill_mistake(name, monkeypatch):
    monkeypatch.setattr(pf, "causal_attention", PREFILL_MUTANTS[name])
    with np.errstate(all="ignore"):
        assert _fails_some_pin(PREFILL_PINS, pf), f"no pin caught mutant {name}"
