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
                                 decode_token=O.decode_token)


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
