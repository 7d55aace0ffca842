"""Drive the CPU oracle over a set of generated inputs.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU-baseline leg).

Inputs arrive as the torch tensors produced by `dsa_inputs.make_inputs` (on any
device); torch is used here only to copy exact values to the host.  bfloat16 tensors
are copied as raw bits and decoded by the oracle's own bit shift.
"""
from __future__ import annotations

import numpy as np
import torch

from . import dsa_oracle as O


def to_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(t.view(torch.int16).numpy())
    return t.double().numpy()


def request_rows(pool: torch.Tensor, block_table_row: np.ndarray, n: int) -> np.ndarray:
    """Logical rows 0..n-1 of one request.

    Only the blocks the request owns are copied to the host (pools can be many GB); the
    page translation itself is the oracle's `logical_rows` over that copied sub-pool."""
    nb = (n + O.BLOCK - 1) // O.BLOCK
    phys = np.asarray(block_table_row[:nb], dtype=np.int64)
    sub = to_f64(pool[torch.as_tensor(phys, device=pool.device)])       # [nb][64][D]
    return O.logical_rows(sub, np.arange(nb), n)


def selected_rows(pool: torch.Tensor, block_table_row: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Rows of the given logical positions: the oracle maps each position to its
    (block, slot); only those rows are copied to the host."""
    blk, slot = O.page_slots(block_table_row, positions)
    dev = pool.device
    return to_f64(pool[torch.as_tensor(blk, device=dev), torch.as_tensor(slot, device=dev)])


def expected_token(inp: dict, t: int, layers=None, key_cache: dict = None) -> dict:
    """Oracle results for query token t of an input set (decode or prefill).

    The token belongs to request q_row[t] and sees O.visible_count(q_pos[t]) positions;
    O.group_token runs the indexer and top-k once and every listed layer attends over
    that selection with its own q and latent pool (layer 0 alone is plain DSA).
    key_cache (optional) keeps each request's logical key rows between calls.
    Returns dict(scores f32 [n], idx int32 [k], out list of f64 [H][Dl], lse list [H], n)."""
    cfg = inp["cfg"]
    layers = range(cfg.layers) if layers is None else layers
    b = int(inp["q_row"][t])
    n = O.visible_count(int(inp["q_pos"][t]))
    bt = inp["block_table"][b].cpu().numpy()
    if key_cache is not None and b in key_cache and key_cache[b].shape[0] >= n:
        keys = key_cache[b]
    else:
        keys = request_rows(inp["k_pool"], bt, n)
        if key_cache is not None:
            key_cache[b] = keys
    per_layer = [(to_f64(inp["q"][l][t]),
                  (lambda pos, pool=inp["kv_pools"][l]: selected_rows(pool, bt, pos)))
                 for l in layers]
    scores, idx, res = O.group_token(to_f64(inp["q_idx"][t]), to_f64(inp["w"][t]), keys, n, cfg.k,
                                     per_layer, cfg.Dl, cfg.sm_scale)
    return dict(scores=scores, idx=idx, out=[o for o, _ in res], lse=[s for _, s in res], n=n)


def expected_topk(scores: np.ndarray, n_valid: np.ndarray, k: int) -> np.ndarray:
    """Top-k of every row of a score matrix [rows][ld] (fp32)."""
    return np.stack([O.topk_positions(scores[r], int(n_valid[r]), k) for r in range(scores.shape[0])])


def expected_token_mha(inp: dict, t: int, heads=None) -> dict:
    """Oracle MHA-mode output of query token t of an input set drawn with cfg.mha: the
    token's selection (indexer scores, stable-sort top-k, dense below k) and dsa_oracle.mla_mha
    over those rows of layer 0's latent pool with the input set's up-projection weights,
    for the listed heads (all by default).
    Returns dict(out f64 [heads][128], lse [heads], idx, n)."""
    cfg = inp["cfg"]
    b = int(inp["q_row"][t])
    n = O.visible_count(int(inp["q_pos"][t]))
    bt = inp["block_table"][b].cpu().numpy()
    keys = request_rows(inp["k_pool"], bt, n)
    scores = O.indexer_scores(to_f64(inp["q_idx"][t]), to_f64(inp["w"][t]), keys)
    idx = O.topk_positions(scores, n, cfg.k)
    rows = selected_rows(inp["kv_pools"][0], bt, idx[idx >= 0])
    heads = list(range(cfg.H)) if heads is None else list(heads)
    q = to_f64(inp["q_mha"][t])[heads]
    dn = inp["w_uk"].shape[2]
    out, lse = O.mla_mha(q[:, :dn], q[:, dn:], rows[:, :cfg.Dl], rows[:, cfg.Dl:], to_f64(inp["w_uk"][heads]),
                         to_f64(inp["w_uv"][heads]), cfg.sm_scale)
    return dict(out=out, lse=lse, idx=idx, n=n)
