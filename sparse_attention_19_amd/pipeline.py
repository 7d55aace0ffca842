"""One step of the DSA hot path through the C ABI: indexer -> top-k -> sparse MLA, with
the IndexShare reuse of the first layer's selection by the following layers of a group.

(SemiAnalysis, "Inside GLM-5.3: How Sparse Attention Affects DRAM Memory TAM",
§Lightning Indexer, §Sparse MLA, §IndexShare.)

Buffers are allocated once with torch (device memory only) and reused every step; the
step itself only enqueues library calls on the current stream.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

from . import (DSA_OP_MLA, DSA_OP_TOPK, IndexCache, dsa_indexer_scores, dsa_sparse_mla_decode,
               dsa_sparse_mla_prefill, dsa_topk, workspace)


@dataclasses.dataclass
class StepBuffers:
    scores: torch.Tensor            # [T][ld] fp32
    idx: torch.Tensor               # [T][k] int32 (also the IndexShare cache)
    outs: List[torch.Tensor]        # per layer [T][H][Dl]
    lses: List[torch.Tensor]        # per layer [T][H] fp32
    ws_topk: Optional[torch.Tensor]
    ws_mla: Optional[torch.Tensor]
    cache: Optional[IndexCache]
    n_valid: Optional[torch.Tensor] = None   # prefill: q_pos (n = q_pos + 1)


def alloc_buffers(T: int, ld: int, k: int, H: int, Dl: int, layers: int, dtype, device,
                  group: int = 4) -> StepBuffers:
    idx = torch.empty((T, k), dtype=torch.int32, device=device)
    return StepBuffers(
        scores=torch.empty((T, ld), dtype=torch.float32, device=device),
        idx=idx,
        outs=[torch.empty((T, H, Dl), dtype=dtype, device=device) for _ in range(layers)],
        lses=[torch.empty((T, H), dtype=torch.float32, device=device) for _ in range(layers)],
        ws_topk=workspace(DSA_OP_TOPK, T, ld, k, H, Dl, device),
        ws_mla=workspace(DSA_OP_MLA, T, 0, k, H, Dl, device),
        cache=IndexCache(idx, k, group=max(group, 2)) if layers > 1 else None,
    )


def decode_step(q_idx, w, k_pool, kv_pools, qs, block_table, seq_len, k, sm_scale, buf: StepBuffers,
                step: int = 0) -> None:
    """One decode token per request through len(kv_pools) DSA layers sharing one indexer."""
    dsa_indexer_scores(q_idx, w, k_pool, block_table, seq_len, buf.scores)
    dsa_topk(buf.scores, seq_len, k, buf.idx, n_add=0, ws=buf.ws_topk)
    if buf.cache is not None:
        buf.cache.publish(step)
    for layer, (kv, q) in enumerate(zip(kv_pools, qs)):
        idx = buf.idx if layer == 0 else buf.cache.get(step, layer)
        dsa_sparse_mla_decode(q, kv, block_table, seq_len, idx, k, sm_scale, buf.outs[layer],
                              buf.lses[layer], ws=buf.ws_mla)


def prefill_step(q_idx, w, k_pool, kv_pools, qs, block_table, seq_len, q_row, q_pos, k, sm_scale,
                 buf: StepBuffers, step: int = 0) -> None:
    """A causal prefill chunk: token t of request q_row[t] at position q_pos[t]."""
    dsa_indexer_scores(q_idx, w, k_pool, block_table, seq_len, buf.scores, q_row=q_row, q_pos=q_pos)
    dsa_topk(buf.scores, q_pos, k, buf.idx, n_add=1, ws=buf.ws_topk)
    if buf.cache is not None:
        buf.cache.publish(step)
    for layer, (kv, q) in enumerate(zip(kv_pools, qs)):
        idx = buf.idx if layer == 0 else buf.cache.get(step, layer)
        dsa_sparse_mla_prefill(q, kv, block_table, seq_len, q_row, q_pos, idx, k, sm_scale,
                               buf.outs[layer], buf.lses[layer], ws=buf.ws_mla)


def run_inputs(inp: dict, buf: Optional[StepBuffers] = None, step: int = 0) -> StepBuffers:
    """Run one step on an input set from dsa_inputs.make_inputs (tensors on the GPU)."""
    cfg = inp["cfg"]
    T = inp["q_idx"].shape[0]
    ld = inp["block_table"].shape[1] * 64
    if buf is None:
        buf = alloc_buffers(T, ld, cfg.k, cfg.H, cfg.Dl, cfg.layers, cfg.dtype, inp["q_idx"].device)
    if cfg.prefill_tokens:
        prefill_step(inp["q_idx"], inp["w"], inp["k_pool"], inp["kv_pools"], inp["q"], inp["block_table"],
                     inp["seq_len"], inp["q_row"], inp["q_pos"], cfg.k, cfg.sm_scale, buf, step)
    else:
        decode_step(inp["q_idx"], inp["w"], inp["k_pool"], inp["kv_pools"], inp["q"], inp["block_table"],
                    inp["seq_len"], cfg.k, cfg.sm_scale, buf, step)
    return buf
