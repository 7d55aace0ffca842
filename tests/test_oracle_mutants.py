"""Plausible mistakes planted in copies of the oracle (on the CPU) must fail a pin.

This shows the pins in oracle_pins.py are sharp enough to catch a dropped term, a wrong
sign or index, a transposed operand or a wrong tie rule in the oracle."""
import numpy as np
import pytest

import oracle_pins as P
from oracle import dsa_oracle as O


def _no_relu(q, w, keys):
    return ((keys @ q.T) @ w + 0.0).astype(np.float32)


def _relu_after_weight(q, w, keys):
    return (np.maximum((keys @ q.T) @ w, 0.0) + 0.0).astype(np.float32)


def _unweighted(q, w, keys):
    return (np.maximum(keys @ q.T, 0.0).sum(1) + 0.0).astype(np.float32)


def _max_over_heads(q, w, keys):
    return (np.max(np.maximum(keys @ q.T, 0.0) * w, axis=1) + 0.0).astype(np.float32)


def _ties_high_index(scores, n, k):
    out = np.full(k, -1, np.int32)
    if n <= k:
        out[:n] = np.arange(n)
        return out
    v = scores[:n].astype(np.float64)
    order = np.lexsort((-np.arange(n), -v))
    out[:] = np.sort(order[:k])
    return out


def _ascending_scores(scores, n, k):
    out = np.full(k, -1, np.int32)
    if n <= k:
        out[:n] = np.arange(n)
        return out
    order = np.lexsort((np.arange(n), scores[:n].astype(np.float64)))
    out[:] = np.sort(order[:k])
    return out


def _unsorted_output(scores, n, k):
    out = np.full(k, -1, np.int32)
    if n <= k:
        out[:n] = np.arange(n)
        return out
    order = np.lexsort((np.arange(n), -scores[:n].astype(np.float64)))
    out[:] = order[:k]
    return out


def _signed_zero_distinct(scores, n, k):
    out = np.full(k, -1, np.int32)
    if n <= k:
        out[:n] = np.arange(n)
        return out
    key = np.where(np.signbit(scores[:n]), -1e-30, 0.0) + scores[:n].astype(np.float64)
    order = np.lexsort((np.arange(n), -key))
    out[:] = np.sort(order[:k])
    return out


def _value_includes_rope(q, rows, Dl, sc):
    o, l = O.mla_absorbed(q, rows, rows.shape[1], sc)
    return o[:, :Dl] * 0 + o[:, rows.shape[1] - Dl:], l


def _value_is_rope_shifted(q, rows, Dl, sc):
    lg = sc * q @ rows.T
    p = np.exp(lg - lg.max(1, keepdims=True))
    z = p.sum(1)
    return (p @ rows[:, 1:Dl + 1]) / z[:, None], lg.max(1) + np.log(z)


def _keys_latent_only(q, rows, Dl, sc):
    lg = sc * q[:, :Dl] @ rows[:, :Dl].T
    p = np.exp(lg - lg.max(1, keepdims=True))
    z = p.sum(1)
    return (p @ rows[:, :Dl]) / z[:, None], lg.max(1) + np.log(z)


def _no_scale(q, rows, Dl, sc):
    return O.mla_absorbed(q, rows, Dl, 1.0)


def _lse_missing_max(q, rows, Dl, sc):
    o, l = O.mla_absorbed(q, rows, Dl, sc)
    lg = sc * q @ rows.T
    return o, l - lg.max(1)


def _transposed_block(pool, bt, n):
    s = np.arange(n)
    return pool[bt[s % len(bt)], s // 64 % 64]


def _ignores_table(pool, bt, n):
    s = np.arange(n)
    return pool[s // 64, s % 64]


MUTANTS = {
    "indexer_no_relu": ("indexer_scores", _no_relu, P.check_indexer),
    "indexer_relu_after_weight": ("indexer_scores", _relu_after_weight, P.check_indexer),
    "indexer_unweighted": ("indexer_scores", _unweighted, P.check_indexer),
    "indexer_max_heads": ("indexer_scores", _max_over_heads, P.check_indexer),
    "topk_ties_high": ("topk_positions", _ties_high_index, P.check_topk),
    "topk_ascending": ("topk_positions", _ascending_scores, P.check_topk),
    "topk_unsorted": ("topk_positions", _unsorted_output, P.check_topk),
    "topk_signed_zero": ("topk_positions", _signed_zero_distinct, P.check_topk),
    "attn_value_rope": ("mla_absorbed", _value_includes_rope, P.check_attention),
    "attn_value_shift": ("mla_absorbed", _value_is_rope_shifted, P.check_attention),
    "attn_keys_latent_only": ("mla_absorbed", _keys_latent_only, P.check_attention),
    "attn_no_scale": ("mla_absorbed", _no_scale, P.check_attention),
    "attn_lse": ("mla_absorbed", _lse_missing_max, P.check_attention),
    "paging_transposed": ("logical_rows", _transposed_block, P.check_paging),
    "paging_no_table": ("logical_rows", _ignores_table, P.check_paging),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    attr, fn, check = MUTANTS[name]
    impl = P.real_impl()
    setattr(impl, attr, fn)
    with pytest.raises(AssertionError):
        check(impl)
