"""Pins of the CPU oracle against things other than itself.

Each `check_*` takes an implementation (a namespace with the oracle's functions) and
raises AssertionError if it disagrees with brute force, a closed form, an invariant or
a textbook routine.  tests/test_oracle_pins.py runs them on the real oracle;
tests/test_oracle_mutants.py runs them on deliberately broken copies of the oracle and
requires every mutant to be caught.
"""
from __future__ import annotations

import math
import types

import numpy as np
import scipy.special

from oracle import dsa_oracle as O


def real_impl():
    return types.SimpleNamespace(indexer_scores=O.indexer_scores, topk_positions=O.topk_positions,
                                 mla_absorbed=O.mla_absorbed, logical_rows=O.logical_rows,
                                 decode_token=O.decode_token, bf16_bits_to_f64=O.bf16_bits_to_f64,
                                 visible_count=O.visible_count, group_token=O.group_token,
                                 mla_mha=O.mla_mha, working_set_init=O.working_set_init,
                                 working_set_step=O.working_set_step)


# ------------------------------------------------------------------ indexer

def _brute_scores(q, w, keys):
    """Exact integer brute force: sum_j w_j * max(0, q_j . k) in Python ints."""
    out = []
    for krow in keys.tolist():
        tot = 0
        for qj, wj in zip(q.tolist(), w.tolist()):
            d = sum(int(a) * int(b) for a, b in zip(qj, krow))
            tot += int(wj) * max(0, d)
        out.append(tot)
    return out


def check_indexer(impl, seed=0):
    rng = np.random.default_rng(seed)
    for (Hi, Di, n, r, wm) in [(4, 32, 256, 3, 2), (3, 5, 17, 4, 3), (64, 128, 40, 4, 3)]:
        q = rng.integers(-r, r + 1, (Hi, Di)).astype(np.float64)
        w = rng.integers(0, wm + 1, Hi).astype(np.float64)
        keys = rng.integers(-r, r + 1, (n, Di)).astype(np.float64)
        got = impl.indexer_scores(q, w, keys)
        assert got.dtype == np.float32 and got.shape == (n,)
        assert [int(v) for v in got.tolist()] == _brute_scores(q, w, keys)
    # closed form: w == 0 gives all-zero scores (and +0.0, never -0.0)
    q = rng.integers(-3, 4, (4, 8)).astype(np.float64)
    keys = rng.integers(-3, 4, (9, 8)).astype(np.float64)
    z = impl.indexer_scores(q, np.zeros(4), keys)
    assert np.all(z == 0) and not np.any(np.signbit(z))
    # closed form: one-hot key e_c scores sum_j w_j * max(0, q_j[c])
    w = np.array([1.0, 2.0, 0.0, 3.0])
    for c in range(8):
        e = np.zeros((1, 8))
        e[0, c] = 1
        want = sum(w[j] * max(0.0, q[j, c]) for j in range(4))
        assert impl.indexer_scores(q, w, e)[0] == want
    # a key anti-aligned with every head contributes nothing (ReLU clips it)
    q1 = np.ones((3, 4))
    assert impl.indexer_scores(q1, np.ones(3), -np.ones((1, 4)))[0] == 0.0
    # head weights act per head: only head 1 weighted
    q2 = np.array([[1.0, 0], [0, 1.0]])
    k2 = np.array([[5.0, 2.0]])
    assert impl.indexer_scores(q2, np.array([0.0, 1.0]), k2)[0] == 2.0
    assert impl.indexer_scores(q2, np.array([1.0, 0.0]), k2)[0] == 5.0


# ------------------------------------------------------------------ top-k

def _brute_topk(scores, n, k):
    if n <= k:
        return list(range(n)) + [-1] * (k - n)
    sel = sorted(range(n), key=lambda s: (-float(scores[s]), s))[:k]
    return sorted(sel)


def check_topk(impl, seed=1):
    rng = np.random.default_rng(seed)
    for trial in range(300):
        n = int(rng.integers(1, 60))
        k = int(rng.integers(1, 20))
        kind = trial % 4
        if kind == 0:       # heavy ties: few distinct integer values
            s = rng.integers(0, 3, n).astype(np.float32)
        elif kind == 1:     # distinct
            s = rng.permutation(n).astype(np.float32)
        elif kind == 2:     # floats incl. negatives and zeros of both signs
            s = rng.standard_normal(n).astype(np.float32)
            s[rng.integers(0, n, 3)] = -0.0
        else:
            s = rng.integers(-5, 6, n).astype(np.float32) * 0.5
        pad = np.concatenate([s, rng.standard_normal(7).astype(np.float32)])  # junk past n
        got = impl.topk_positions(pad, n, k)
        assert got.dtype == np.int32 and got.shape == (k,)
        assert got.tolist() == _brute_topk(s, n, k), (trial, n, k)
    # invariants at a realistic size
    n, k = 5000, 256
    s = rng.integers(0, 400, n).astype(np.float32)
    base = impl.topk_positions(s, n, k)
    # (i) n <= k keeps everything
    assert impl.topk_positions(s, k, k).tolist() == list(range(k))
    assert impl.topk_positions(s, 10, k).tolist() == list(range(10)) + [-1] * (k - 10)
    # (ii) all-equal scores keep the k lowest positions
    assert impl.topk_positions(np.full(n, 7.0, np.float32), n, k).tolist() == list(range(k))
    # (iii) a strictly increasing map of the scores (exact here) leaves the set unchanged
    assert np.array_equal(impl.topk_positions(2 * s + 1, n, k), base)
    # (iv) permuting the values strictly below the k-th score among their positions
    theta = np.sort(s)[::-1][k - 1]
    low = np.where(s < theta)[0]
    s2 = s.copy()
    s2[low] = s[rng.permutation(low)]
    assert np.array_equal(impl.topk_positions(s2, n, k), base)
    # ties at theta: exactly k - count(> theta) of them, the lowest positions
    gt = int((s > theta).sum())
    eq_pos = np.where(s == theta)[0][: k - gt]
    want = np.sort(np.concatenate([np.where(s > theta)[0], eq_pos]))
    assert np.array_equal(base, want)
    # -0.0 and +0.0 are the same score: the lower position wins
    z = np.array([-0.0, 0.0, -1.0], np.float32)
    assert impl.topk_positions(z, 3, 1).tolist() == [0]
    z = np.array([0.0, -0.0, -1.0], np.float32)
    assert impl.topk_positions(z, 3, 1).tolist() == [0]


# ------------------------------------------------------------------ attention

def _brute_attention(q, rows, Dl, scale):
    H, S = len(q), len(rows)
    out, lse = [], []
    for h in range(H):
        lg = [scale * sum(a * b for a, b in zip(q[h], rows[s])) for s in range(S)]
        m = max(lg)
        e = [math.exp(x - m) for x in lg]
        z = sum(e)
        out.append([sum(e[s] * rows[s][c] for s in range(S)) / z for c in range(Dl)])
        lse.append(m + math.log(z))
    return np.array(out), np.array(lse)


def check_attention(impl, seed=2):
    rng = np.random.default_rng(seed)
    for (H, Dl, Dr, S) in [(3, 5, 2, 7), (8, 64, 16, 33), (2, 4, 4, 1)]:
        q = rng.standard_normal((H, Dl + Dr))
        rows = rng.standard_normal((S, Dl + Dr))
        sc = 1.0 / math.sqrt(Dl + Dr)
        o, l = impl.mla_absorbed(q, rows, Dl, sc)
        bo, bl = _brute_attention(q.tolist(), rows.tolist(), Dl, sc)
        assert o.shape == (H, Dl) and l.shape == (H,)
        assert np.allclose(o, bo, rtol=1e-12, atol=1e-12)
        assert np.allclose(l, bl, rtol=1e-12, atol=1e-12)
        # textbook routines: softmax-weighted values and logsumexp of the logits
        lg = sc * q @ rows.T
        assert np.allclose(o, scipy.special.softmax(lg, axis=1) @ rows[:, :Dl], rtol=1e-12, atol=1e-12)
        assert np.allclose(l, scipy.special.logsumexp(lg, axis=1), rtol=1e-12, atol=1e-12)
    # closed forms
    rows = rng.standard_normal((9, 12))
    o, l = impl.mla_absorbed(np.zeros((4, 12)), rows, 8, 0.3)
    assert np.allclose(o, np.tile(rows[:, :8].mean(0), (4, 1)), atol=1e-13)   # q = 0 -> mean of values
    assert np.allclose(l, math.log(9), atol=1e-13)                          # lse = log |S|
    o, l = impl.mla_absorbed(rng.standard_normal((4, 12)), rows[3:4], 8, 0.3)
    assert np.allclose(o, np.tile(rows[3, :8], (4, 1)), atol=1e-13)         # |S| = 1 -> the row
    same = np.tile(rows[5], (6, 1))
    o, _ = impl.mla_absorbed(rng.standard_normal((4, 12)), same, 8, 0.3)
    assert np.allclose(o, np.tile(rows[5, :8], (4, 1)), atol=1e-13)         # identical rows
    # keys use the rope dims too: q nonzero only on the rope part still reweights
    q = np.zeros((1, 12))
    q[0, 8:] = 1.0
    o, _ = impl.mla_absorbed(q, rows, 8, 1.0)
    lg = rows[:, 8:].sum(1)
    assert np.allclose(o[0], scipy.special.softmax(lg) @ rows[:, :8], atol=1e-12)
    # large logits: no overflow (max subtraction)
    o, l = impl.mla_absorbed(np.full((1, 12), 40.0), rows, 8, 10.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


# ------------------------------------------------------------------ paging + composition

def check_paging(impl, seed=3):
    rng = np.random.default_rng(seed)
    nblk, D, n = 7, 5, 7 * 64 - 13
    logical = rng.standard_normal((nblk * 64, D))
    perm = rng.permutation(nblk)
    pool = np.empty((nblk, 64, D))
    for lb in range(nblk):
        pool[perm[lb]] = logical[lb * 64:(lb + 1) * 64]
    got = impl.logical_rows(pool, perm, n)
    assert np.array_equal(got, logical[:n])
    ident = logical.reshape(nblk, 64, D)
    assert np.array_equal(impl.logical_rows(ident, np.arange(nblk), n), logical[:n])


def check_sparse_equals_dense(impl, seed=4):
    rng = np.random.default_rng(seed)
    Hi, Di, H, Dl, Dr, k = 4, 8, 3, 6, 2, 16
    for n in (1, 5, 15, 16):
        q_idx = rng.integers(-3, 4, (Hi, Di)).astype(np.float64)
        w = rng.integers(0, 3, Hi).astype(np.float64)
        keys = rng.integers(-3, 4, (n, Di)).astype(np.float64)
        q = rng.standard_normal((H, Dl + Dr))
        kv = rng.standard_normal((n, Dl + Dr))
        _, idx, out, lse = impl.decode_token(q_idx, w, keys, q, kv, n, k, Dl, 0.5)
        assert idx.tolist() == list(range(n)) + [-1] * (k - n)
        bo, bl = _brute_attention(q.tolist(), kv.tolist(), Dl, 0.5)
        assert np.allclose(out, bo, atol=1e-12) and np.allclose(lse, bl, atol=1e-12)
    # n > k: attention runs over exactly the brute-force top-k rows
    n = 40
    q_idx = rng.integers(-3, 4, (Hi, Di)).astype(np.float64)
    w = rng.integers(0, 3, Hi).astype(np.float64)
    keys = rng.integers(-3, 4, (n, Di)).astype(np.float64)
    q = rng.standard_normal((H, Dl + Dr))
    kv = rng.standard_normal((n, Dl + Dr))
    sc, idx, out, lse = impl.decode_token(q_idx, w, keys, q, kv, n, k, Dl, 0.5)
    want = _brute_topk(_brute_scores(q_idx, w, keys), n, k)
    assert idx.tolist() == want
    bo, bl = _brute_attention(q.tolist(), kv[want].tolist(), Dl, 0.5)
    assert np.allclose(out, bo, atol=1e-12) and np.allclose(lse, bl, atol=1e-12)


ALL_CHECKS = [check_indexer, check_topk, check_attention, check_paging, check_sparse_equals_dense]


# ------------------------------------------------------------------ bf16 decode

def check_bf16_decode(impl):
    """Every one of the 65 536 bfloat16 bit patterns decodes to the value torch's own CPU
    bfloat16 -> float32 conversion gives (NaN patterns: NaN)."""
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):          # signalling-NaN patterns widen to NaN
        got = impl.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    nan = np.isnan(ref)
    assert got.shape == (65536,) and got.dtype == np.float64
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero survives: pattern 0x8000 is -0.0
    assert np.signbit(got[0x8000]) and got[0x8000] == 0.0 and not np.signbit(got[0])


# ------------------------------------------------------------------ composition used by the GPU tests

def _brute_token(inp, t, layers):
    """Token t of an input set, from scratch in Python: integer scores over positions
    0..q_pos (Python ints), the stable order (score desc, position asc), and pure-Python
    attention of each layer (its own q and pool) over the first layer's selection.
    Values are read with torch's own dtype conversion, rows through the block table."""
    cfg = inp["cfg"]
    b = int(inp["q_row"][t])
    n = int(inp["q_pos"][t]) + 1
    bt = inp["block_table"][b].tolist()
    qi = [[int(round(x)) for x in row] for row in inp["q_idx"][t].float().tolist()]
    w = [int(round(x)) for x in inp["w"][t].float().tolist()]
    kp = inp["k_pool"].float()
    scores = []
    for s in range(n):
        key = [int(round(x)) for x in kp[bt[s // 64], s % 64].tolist()]
        scores.append(sum(wj * max(0, sum(a * c for a, c in zip(qj, key))) for qj, wj in zip(qi, w)))
    if n <= cfg.k:
        sel = list(range(n))
    else:
        sel = sorted(sorted(range(n), key=lambda s: (-scores[s], s))[:cfg.k])
    res = []
    for l in layers:
        pool = inp["kv_pools"][l].float()
        rows = [pool[bt[s // 64], s % 64].double().tolist() for s in sel]
        q = inp["q"][l][t].float().double().tolist()
        res.append(_brute_attention(q, rows, cfg.Dl, cfg.sm_scale))
    return scores, sel + [-1] * (cfg.k - len(sel)), res


def composition_inputs():
    """Tiny CPU input sets: a 2-layer fp32 group with dense and sparse rows, a 2-layer
    bf16 group, and a prefill chunk whose tokens belong to two requests."""
    import torch
    import dsa_inputs as I
    tiny = I.CONFIGS["tiny_fp32"]
    sets = []
    g1 = I.shrink(tiny, batch=3, ctx_range=(70, 300), extra_dense=(50,), identity_pages=False, layers=2)
    sets.append(I.make_inputs(g1))
    g2 = I.shrink(tiny, dtype=torch.bfloat16, batch=2, ctx_range=(100, 260), extra_dense=(33,),
                  identity_pages=False, layers=2)
    sets.append(I.make_inputs(g2))
    base = I.shrink(tiny, batch=2, ctx=300, identity_pages=False)
    pre = I.make_inputs(base)
    T = 6
    gen = torch.Generator().manual_seed(11)
    pre["q_row"] = torch.tensor([0, 1, 0, 1, 1, 0], dtype=torch.int32)
    pre["q_pos"] = torch.tensor([299, 10, 63, 64, 200, 150], dtype=torch.int32)
    pre["q_idx"] = torch.randint(-3, 4, (T, 4, 32), generator=gen).float()
    pre["w"] = torch.randint(0, 3, (T, 4), generator=gen).float()
    pre["q"] = [torch.randn(T, 8, 80, generator=gen)]
    pre["cfg"] = I.shrink(base, prefill_tokens=T)
    sets.append(pre)
    return sets


def check_composition(impl, inputs=None):
    """oracle/run.py's expected_token, run with impl's visibility rule and group
    composition, against _brute_token on every token of the tiny input sets."""
    from oracle import run as R
    saved = (O.visible_count, O.group_token)
    O.visible_count, O.group_token = impl.visible_count, impl.group_token
    try:
        for inp in (inputs or composition_inputs()):
            cfg = inp["cfg"]
            layers = list(range(cfg.layers))
            for t in range(inp["q_idx"].shape[0]):
                got = R.expected_token(inp, t)
                scores, idx, res = _brute_token(inp, t, layers)
                assert got["n"] == len(scores)
                assert [int(v) for v in got["scores"].tolist()] == scores, (cfg.name, t)
                assert got["idx"].tolist() == idx, (cfg.name, t)
                for (o, l), (bo, bl) in zip(zip(got["out"], got["lse"]), res):
                    assert np.allclose(o, bo, rtol=1e-12, atol=1e-12), (cfg.name, t)
                    assert np.allclose(l, bl, rtol=1e-12, atol=1e-12), (cfg.name, t)
    finally:
        O.visible_count, O.group_token = saved


ALL_CHECKS += [check_bf16_decode, check_composition]


# ------------------------------------------------------------------ MHA mode

def check_mha(impl, seed=5):
    """MHA mode against a pure-Python brute force, and against MQA mode through the
    absorption identity: with q' = [w_uk[h] @ q_nope[h], q_rope[h]] the absorbed attention
    over [latent, rope] rows gives the latent-space output o, and o @ w_uv[h] is MHA mode's
    output (the logits and the softmax are the same numbers), exactly in float64."""
    rng = np.random.default_rng(seed)
    for (H, dl, dn, dr, dv, S) in [(2, 6, 3, 2, 4, 5), (3, 16, 8, 4, 8, 33), (2, 8, 4, 4, 2, 1)]:
        qn = rng.standard_normal((H, dn))
        qr = rng.standard_normal((H, dr))
        lat = rng.standard_normal((S, dl))
        rp = rng.standard_normal((S, dr))
        wuk = rng.standard_normal((H, dl, dn)) / np.sqrt(dl)
        wuv = rng.standard_normal((H, dl, dv)) / np.sqrt(dl)
        sc = 1.0 / np.sqrt(dn + dr)
        out, lse = impl.mla_mha(qn, qr, lat, rp, wuk, wuv, sc)
        assert out.shape == (H, dv) and lse.shape == (H,)
        # brute force, per head, in Python floats
        for h in range(H):
            k = [[sum(lat[s][c] * wuk[h][c][j] for c in range(dl)) for j in range(dn)] + list(rp[s]) for s in range(S)]
            v = [[sum(lat[s][c] * wuv[h][c][j] for c in range(dl)) for j in range(dv)] for s in range(S)]
            q = list(qn[h]) + list(qr[h])
            lg = [sc * sum(a * b for a, b in zip(q, k[s])) for s in range(S)]
            m = max(lg)
            e = [math.exp(x - m) for x in lg]
            z = sum(e)
            want = [sum(e[s] * v[s][j] for s in range(S)) / z for j in range(dv)]
            assert np.allclose(out[h], want, rtol=1e-11, atol=1e-11)
            assert abs(lse[h] - (m + math.log(z))) < 1e-11
        # absorption identity: MQA mode over the latent rows, then the value up-projection
        rows = np.concatenate([lat, rp], axis=1)
        qabs = np.stack([np.concatenate([wuk[h] @ qn[h], qr[h]]) for h in range(H)])
        o_lat, lse_abs = O.mla_absorbed(qabs, rows, dl, sc)
        mqa = np.stack([o_lat[h] @ wuv[h] for h in range(H)])
        assert np.allclose(out, mqa, rtol=1e-11, atol=1e-11)
        assert np.allclose(lse, lse_abs, rtol=1e-11, atol=1e-11)
    # closed form: no NoPE weights and a zero rope query -> uniform weights, the mean of V
    lat = rng.standard_normal((7, 6))
    wuv = rng.standard_normal((2, 6, 3))
    out, lse = impl.mla_mha(rng.standard_normal((2, 3)), np.zeros((2, 2)), lat, rng.standard_normal((7, 2)),
                            np.zeros((2, 6, 3)), wuv, 0.7)
    assert np.allclose(out, np.stack([lat.mean(0) @ wuv[h] for h in range(2)]), atol=1e-12)
    assert np.allclose(lse, math.log(7), atol=1e-12)


ALL_CHECKS += [check_mha]


# ------------------------------------------------------------------ MHA-mode composition used by the GPU tests

def mha_composition_inputs():
    """Tiny CPU prefill chunks drawn with MHA-mode inputs (2 heads of 192 + 64 query-key and
    128 value dims over 512 + 64 latent rows): one whose tokens select 64 of ~300 positions,
    one whose tokens see fewer positions than k (dense)."""
    import torch
    import dsa_inputs as I
    base = I.shrink(I.CONFIGS["prefill_4096_at_128k"], ctx=300, prefill_tokens=5, Hi=4, Di=32, idx_range=3,
                    w_max=2, H=2, identity_pages=False, mha=True, sm_scale=1.0 / 16)
    return [I.make_inputs(I.shrink(base, k=64)), I.make_inputs(I.shrink(base, seed=13, k=512))]


def check_mha_composition(impl=None, inputs=None):
    """oracle/run.py's expected_token_mha against a from-scratch composition on every token:
    the selection of _brute_token, then per head the up-projected keys [latent . w_uk[h],
    rope] and values latent . w_uv[h] of each selected row (row by row), Python-float
    logits with the query's first 192 dims on the NoPE part and last 64 on the rope part, and
    a Python softmax."""
    from oracle import run as R
    for inp in (inputs or mha_composition_inputs()):
        cfg = inp["cfg"]
        wuk = inp["w_uk"].float().double().numpy()
        wuv = inp["w_uv"].float().double().numpy()
        pool = inp["kv_pools"][0].float()
        for t in range(inp["q_idx"].shape[0]):
            got = R.expected_token_mha(inp, t)
            _, idx, _ = _brute_token(inp, t, [])
            assert got["idx"].tolist() == idx, (cfg.name, t)
            sel = [s for s in idx if s >= 0]
            bt = inp["block_table"][int(inp["q_row"][t])].tolist()
            rows = [pool[bt[s // 64], s % 64].double().numpy() for s in sel]
            q = inp["q_mha"][t].float().double().tolist()
            for h in range(cfg.H):
                lg, vs = [], []
                for r in rows:
                    lat, rope = r[:cfg.Dl], r[cfg.Dl:]
                    key = [float(lat @ wuk[h][:, j]) for j in range(wuk.shape[2])] + [float(x) for x in rope]
                    vs.append([float(lat @ wuv[h][:, j]) for j in range(wuv.shape[2])])
                    lg.append(cfg.sm_scale * sum(a * b for a, b in zip(q[h], key)))
                m = max(lg)
                e = [math.exp(x - m) for x in lg]
                z = sum(e)
                want = [sum(e[i] * vs[i][j] for i in range(len(e))) / z for j in range(len(vs[0]))]
                assert np.allclose(got["out"][h], want, rtol=1e-10, atol=1e-10), (cfg.name, t, h)
                assert abs(got["lse"][h] - (m + math.log(z))) < 1e-10, (cfg.name, t, h)


ALL_CHECKS += [check_mha_composition]



# ------------------------------------------------------------------ HBM working set (LRU)

def _brute_lru(S, steps):
    """The working set from its plain definition: every slot carries the time it was last
    used, (step, rank of its position in that step's ascending selection), a free slot
    (-1, slot index); a step's misses, in ascending position order, take the non-hit slots
    with the oldest times.  Yields (slots, loads, evicted, order) per step."""
    last = {s: (-1, s) for s in range(S)}
    holds = {}                       # slot -> position
    where = {}                       # position -> slot
    for t, sel in enumerate(steps):
        hits = {where[p] for p in sel if p in where}
        misses = [p for p in sel if p not in where]
        free = sorted((s for s in range(S) if s not in hits), key=lambda s: last[s])
        if len(misses) > len(free):
            raise ValueError("too small")
        loads, evicted = [], []
        for p, s in zip(misses, free):
            if s in holds:
                evicted.append(holds[s])
                del where[holds[s]]
            holds[s] = p
            where[p] = s
            loads.append((p, s))
        for r, p in enumerate(sel):
            last[where[p]] = (t, r)
        yield [where[p] for p in sel], loads, evicted, sorted(range(S), key=lambda s: last[s])


def _lru_sequences(rng):
    """Selection sequences over a small universe with a drift between steps (some positions
    kept, some new), including repeats, empty steps and full-size selections."""
    cases = []
    for S, size, universe, steps in [(4, 3, 9, 12), (7, 7, 20, 10), (64, 40, 300, 15), (16, 5, 16, 20)]:
        seq, prev = [], []
        for _ in range(steps):
            n = int(rng.integers(0, size + 1))
            keep = [p for p in prev if rng.random() < 0.6][:n]
            new = [int(p) for p in rng.permutation(universe)[:n] if p not in keep][:n - len(keep)]
            cur = sorted(set(keep + new))
            seq.append(cur)
            prev = cur
        seq.append(list(seq[-1]))            # the same selection twice
        cases.append((S, seq))
    return cases


def check_working_set(impl, seed=7):
    rng = np.random.default_rng(seed)
    for S, seq in _lru_sequences(rng):
        st = impl.working_set_init(S)
        for sel, (b_slots, b_loads, b_evicted, b_order) in zip(seq, _brute_lru(S, seq)):
            before = dict(st["slot_of"])
            slots, loads, evicted = impl.working_set_step(st, sel)
            assert slots == b_slots and loads == b_loads and evicted == b_evicted, (S, sel)
            assert st["order"] == b_order, (S, sel)
            # invariants: every selected position resident; the maps are inverse; loads are
            # exactly the selected positions that were not resident; evictions are unselected
            assert all(p in st["slot_of"] for p in sel)
            assert sorted(st["order"]) == list(range(S))
            assert all(st["pos_of"][s] == p for p, s in st["slot_of"].items())
            assert sum(1 for p in st["pos_of"] if p >= 0) == len(st["slot_of"]) <= S
            assert [p for p, _ in loads] == [p for p in sel if p not in before]
            assert not set(evicted) & set(sel)
        # the repeated last selection loaded nothing
        assert loads == []
    # special cases: a history that fits never evicts; disjoint full-size selections evict
    # everything every step; a selection larger than the working set is refused
    st = impl.working_set_init(10)
    for sel in ([0, 1, 2], [3, 4], [0, 5, 6, 7, 8, 9], [1, 2, 3]):
        _, _, ev = impl.working_set_step(st, sel)
        assert ev == []
    st = impl.working_set_init(3)
    impl.working_set_step(st, [0, 1, 2])
    for base in (10, 20, 30):
        _, loads, ev = impl.working_set_step(st, [base, base + 1, base + 2])
        assert len(loads) == 3 and len(ev) == 3
    try:
        impl.working_set_step(impl.working_set_init(2), [1, 2, 3])
        raise AssertionError("a selection larger than the working set was accepted")
    except ValueError:
        pass


def check_working_set_exact(impl, seed=8):
    """The working set changes where rows live, not what attention computes: rows copied
    into device slots by each step's loads, read back through the step's slot list, are the
    selected rows, and attention over them equals attention over the full cache, bit for
    bit, step after step."""
    rng = np.random.default_rng(seed)
    n, D, Dl, S, k = 200, 12, 8, 24, 16
    cache = rng.standard_normal((n, D))           # the history, in host memory
    q = rng.standard_normal((3, D))
    device = np.full((S, D), np.nan)              # slots start with nothing valid
    st = impl.working_set_init(S)
    prev = []
    for _ in range(12):
        keep = [p for p in prev if rng.random() < 0.7]
        sel = sorted(set(keep) | set(int(p) for p in rng.permutation(n)[:k - len(keep)]))[:k]
        slots, loads, _ = impl.working_set_step(st, sel)
        for p, s in loads:
            device[s] = cache[p]
        got = impl.mla_absorbed(q, device[slots], Dl, 0.3)
        want = impl.mla_absorbed(q, cache[sel], Dl, 0.3)
        assert all(np.array_equal(a, b) for a, b in zip(got, want))
        prev = sel


ALL_CHECKS += [check_working_set, check_working_set_exact]
