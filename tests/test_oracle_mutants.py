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


def _bf16_shift15(bits):
    u = bits.astype(np.uint16).astype(np.uint32) << np.uint32(15)
    return u.view(np.float32).astype(np.float64)


def _bf16_unsigned(bits):
    u = (bits.astype(np.uint16).astype(np.uint32) & np.uint32(0x7FFF)) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


_GROUP = O.group_token     # the real composition (the mutants below wrap it)


def _mha_no_rope(qn, qr, lat, rp, wuk, wuv, sc):
    return O.mla_mha(qn, qr * 0, lat, rp, wuk, wuv, sc)


def _mha_keys_without_rope(qn, qr, lat, rp, wuk, wuv, sc):
    return O.mla_mha(qn, qr, lat, rp * 0, wuk, wuv, sc)


def _mha_value_dims_reversed(qn, qr, lat, rp, wuk, wuv, sc):
    return O.mla_mha(qn, qr, lat, rp, wuk, wuv[:, :, ::-1], sc)


def _mha_no_scale(qn, qr, lat, rp, wuk, wuv, sc):
    return O.mla_mha(qn, qr, lat, rp, wuk, wuv, 1.0)


def _sees_before_own(q_pos):
    return int(q_pos)                 # off by one: the query does not see its own key


def _layers_select_own(q_idx, w, key_rows, n, k, layers, Dl, sm_scale):
    """Each shared layer picks its own top-k from its own (head-summed) attention logits."""
    scores, idx, res = _GROUP(q_idx, w, key_rows, n, k, layers[:1], Dl, sm_scale)
    for q, rows_of in layers[1:]:
        own = (rows_of(np.arange(n)) @ q.T).sum(1).astype(np.float32)
        sel = O.topk_positions(own, n, k)
        res.append(O.mla_absorbed(q, rows_of(sel[sel >= 0]), Dl, sm_scale))
    return scores, idx, res


def _layers_use_q0(q_idx, w, key_rows, n, k, layers, Dl, sm_scale):
    q0 = layers[0][0]
    return _GROUP(q_idx, w, key_rows, n, k, [(q0, r) for _, r in layers], Dl, sm_scale)


def _layers_use_pool0(q_idx, w, key_rows, n, k, layers, Dl, sm_scale):
    r0 = layers[0][1]
    return _GROUP(q_idx, w, key_rows, n, k, [(q, r0) for q, _ in layers], Dl, sm_scale)


def _ws_step_variant(evict_mru=False, evict_hits=False, recent_descending=False, keep_stale=False,
                     misses_reversed=False):
    def step(state, sel):
        pos_of, order, slot_of = state["pos_of"], state["order"], state["slot_of"]
        sel = [int(p) for p in sel]
        pre = {p: slot_of[p] for p in sel if p in slot_of}
        hit_slots = set(pre.values())
        misses = [p for p in sel if p not in slot_of]
        cands = list(order) if evict_hits else [s for s in order if s not in hit_slots]
        if evict_mru:
            cands = cands[::-1]
        if misses_reversed:
            misses = misses[::-1]
        if len(misses) > len(cands):
            raise ValueError("too small")
        loads, evicted = [], []
        for p, s in zip(misses, cands):
            if pos_of[s] >= 0:
                evicted.append(pos_of[s])
                if not keep_stale:
                    del slot_of[pos_of[s]]
            pos_of[s] = p
            slot_of[p] = s
            loads.append((p, s))
        # the slots of hits as looked up before the loads (a hit evicted by a load keeps the
        # slot it had, which now holds another position)
        slots = [pre[p] if p in pre else slot_of[p] for p in sel]
        rest = [s for s in order if s not in set(slots)]
        state["order"] = rest + (slots[::-1] if recent_descending else slots)
        return slots, loads, evicted
    return step


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
    "bf16_shift15": ("bf16_bits_to_f64", _bf16_shift15, P.check_bf16_decode),
    "bf16_unsigned": ("bf16_bits_to_f64", _bf16_unsigned, P.check_bf16_decode),
    "visibility_off_by_one": ("visible_count", _sees_before_own, P.check_composition),
    "indexshare_layers_select_own": ("group_token", _layers_select_own, P.check_composition),
    "indexshare_layers_use_q0": ("group_token", _layers_use_q0, P.check_composition),
    "indexshare_layers_use_pool0": ("group_token", _layers_use_pool0, P.check_composition),
    "mha_no_rope": ("mla_mha", _mha_no_rope, P.check_mha),
    "mha_keys_without_rope": ("mla_mha", _mha_keys_without_rope, P.check_mha),
    "mha_value_dims_reversed": ("mla_mha", _mha_value_dims_reversed, P.check_mha),
    "mha_no_scale": ("mla_mha", _mha_no_scale, P.check_mha),
    "working_set_evicts_most_recent": ("working_set_step", _ws_step_variant(evict_mru=True), P.check_working_set),
    "working_set_evicts_hits": ("working_set_step", _ws_step_variant(evict_hits=True), P.check_working_set),
    "working_set_recent_descending": ("working_set_step", _ws_step_variant(recent_descending=True),
                                      P.check_working_set),
    "working_set_keeps_stale_map": ("working_set_step", _ws_step_variant(keep_stale=True), P.check_working_set),
    "working_set_misses_reversed": ("working_set_step", _ws_step_variant(misses_reversed=True),
                                    P.check_working_set),
    "working_set_exact_keeps_stale_map": ("working_set_step", _ws_step_variant(keep_stale=True),
                                          P.check_working_set_exact),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    attr, fn, check = MUTANTS[name]
    impl = P.real_impl()
    setattr(impl, attr, fn)
    with pytest.raises(AssertionError):
        check(impl)


# ---- MHA-mode composition (oracle/run.py expected_token_mha): mistakes planted in copies of it

def _mha_token(inp, t, visible=None, swap_q=False, unfiltered=False, values_from_keys=False):
    from oracle import run as R
    cfg = inp["cfg"]
    b = int(inp["q_row"][t])
    n = (visible or O.visible_count)(int(inp["q_pos"][t]))
    bt = inp["block_table"][b].cpu().numpy()
    scores = O.indexer_scores(R.to_f64(inp["q_idx"][t]), R.to_f64(inp["w"][t]), R.request_rows(inp["k_pool"], bt, n))
    idx = O.topk_positions(scores, n, cfg.k)
    rows = R.selected_rows(inp["kv_pools"][0], bt, idx if unfiltered else idx[idx >= 0])
    q = R.to_f64(inp["q_mha"][t])
    dn = inp["w_uk"].shape[2]
    qn, qr = (q[:, q.shape[1] - dn:], q[:, :q.shape[1] - dn]) if swap_q else (q[:, :dn], q[:, dn:])
    wuv = R.to_f64(inp["w_uk"])[:, :, :inp["w_uv"].shape[2]] if values_from_keys else R.to_f64(inp["w_uv"])
    out, lse = O.mla_mha(qn, qr, rows[:, :cfg.Dl], rows[:, cfg.Dl:], R.to_f64(inp["w_uk"]), wuv, cfg.sm_scale)
    return dict(out=out, lse=lse, idx=idx, n=n)


MHA_COMPOSITION_MUTANTS = {
    "mha_token_sees_before_own": lambda inp, t: _mha_token(inp, t, visible=_sees_before_own),
    "mha_token_query_halves_swapped": lambda inp, t: _mha_token(inp, t, swap_q=True),
    "mha_token_padding_rows_attended": lambda inp, t: _mha_token(inp, t, unfiltered=True),
    "mha_token_values_from_key_weights": lambda inp, t: _mha_token(inp, t, values_from_keys=True),
}


@pytest.fixture(scope="module")
def mha_inputs():
    return P.mha_composition_inputs()


@pytest.mark.parametrize("name", sorted(MHA_COMPOSITION_MUTANTS))
def test_mha_composition_mutant_is_caught(name, mha_inputs, monkeypatch):
    from oracle import run as R
    monkeypatch.setattr(R, "expected_token_mha", MHA_COMPOSITION_MUTANTS[name])
    with pytest.raises(AssertionError):
        P.check_mha_composition(inputs=mha_inputs)


def test_mha_composition_copy_passes(mha_inputs, monkeypatch):
    """The unmutated copy passes, so each failure above comes from its planted mistake."""
    from oracle import run as R
    monkeypatch.setattr(R, "expected_token_mha", _mha_token)
    P.check_mha_composition(inputs=mha_inputs)

