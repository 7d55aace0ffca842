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

from . import (DSA_OP_MLA, DSA_OP_TOPK, Chunk, IndexCache, PageTable, WorkingSet, dsa_indexer_scores,
               dsa_sparse_mla_decode, dsa_sparse_mla_prefill, dsa_topk, dsa_working_set_fetch,
               dsa_working_set_plan, workspace)


@dataclasses.dataclass
class StepBuffers:
    scores: torch.Tensor            # [T][ld] fp32
    idx: torch.Tensor               # [T][k] int32 (also the IndexShare cache)
    outs: List[torch.Tensor]        # per layer [T][H][Dl]
    lses: List[torch.Tensor]        # per layer [T][H] fp32
    ws_topk: Optional[torch.Tensor]
    ws_mla: Optional[torch.Tensor]
    cache: Optional[IndexCache]


def alloc_buffers(T: int, ld: int, k: int, H: int, Dl: int, layers: int, dtype, device,
                  group: int = 4, share: bool = True) -> StepBuffers:
    idx = torch.empty((T, k), dtype=torch.int32, device=device)
    return StepBuffers(
        scores=torch.empty((T, ld), dtype=torch.float32, device=device),
        idx=idx,
        outs=[torch.empty((T, H, Dl), dtype=dtype, device=device) for _ in range(layers)],
        lses=[torch.empty((T, H), dtype=torch.float32, device=device) for _ in range(layers)],
        ws_topk=workspace(DSA_OP_TOPK, T, ld, k, H, Dl, device),
        ws_mla=workspace(DSA_OP_MLA, T, 0, k, H, Dl, device),
        cache=IndexCache(idx, k, group=max(group, 2)) if layers > 1 and share else None,
    )


def decode_step(q_idx, w, k_pool, kv_pools, qs, pt: PageTable, k, sm_scale, buf: StepBuffers,
                step: int = 0, share: bool = True) -> None:
    """One decode token per request through len(kv_pools) DSA layers sharing one indexer
    (share=False: every layer runs the indexer and top-k itself, as DSA without IndexShare)."""
    if not share:
        for kv, q, out, lse in zip(kv_pools, qs, buf.outs, buf.lses):
            dsa_indexer_scores(q_idx, w, k_pool, pt, buf.scores)
            dsa_topk(buf.scores, pt.seq_len, pt.seq_len_host, k, buf.idx, n_add=0, ws=buf.ws_topk)
            dsa_sparse_mla_decode(q, kv, pt, buf.idx, k, sm_scale, out, lse, ws=buf.ws_mla)
        return
    dsa_indexer_scores(q_idx, w, k_pool, pt, buf.scores)
    dsa_topk(buf.scores, pt.seq_len, pt.seq_len_host, k, buf.idx, n_add=0, ws=buf.ws_topk)
    if buf.cache is not None:
        buf.cache.publish(step)
    for layer, (kv, q) in enumerate(zip(kv_pools, qs)):
        idx = buf.idx if layer == 0 else buf.cache.get(step, layer)
        dsa_sparse_mla_decode(q, kv, pt, idx, k, sm_scale, buf.outs[layer], buf.lses[layer], ws=buf.ws_mla)


def prefill_step(q_idx, w, k_pool, kv_pools, qs, pt: PageTable, chunk: Chunk, k, sm_scale,
                 buf: StepBuffers, step: int = 0) -> None:
    """A causal prefill chunk: token t of request q_row[t] at position q_pos[t]."""
    dsa_indexer_scores(q_idx, w, k_pool, pt, buf.scores, chunk=chunk)
    dsa_topk(buf.scores, chunk.q_pos, chunk.q_pos_host, k, buf.idx, n_add=1, ws=buf.ws_topk)
    if buf.cache is not None:
        buf.cache.publish(step)
    for layer, (kv, q) in enumerate(zip(kv_pools, qs)):
        idx = buf.idx if layer == 0 else buf.cache.get(step, layer)
        dsa_sparse_mla_prefill(q, kv, pt, chunk, idx, k, sm_scale, buf.outs[layer], buf.lses[layer],
                               ws=buf.ws_mla)


@dataclasses.dataclass
class WorkingSetBuffers:
    """Decode through an HBM working set of latent rows (remio.ai GLM-5.3 explainer,
    §HiSparse): the selection's rows are loaded from each layer's history in pinned host
    memory into that layer's working-set pool, then attended to there."""
    ws: WorkingSet
    pt: PageTable                   # the working set's page table (request b's slots)
    slot_idx: torch.Tensor          # [T][k] int32, the MLA's index list into the slots
    loads: torch.Tensor             # [T][k][2] int32 (position, slot) to load
    load_count: torch.Tensor        # [T] int32
    dev_pools: List[torch.Tensor]   # per layer [T * slots / 64][64][row_dim]
    fetch_stream: Optional[torch.cuda.Stream]   # None: loads and attention in one stream
    fetched: List[torch.cuda.Event]


def alloc_working_set(batch: int, slots: int, max_len: int, k: int, layers: int, row_dim: int, dtype, device,
                      overlap: bool = True) -> WorkingSetBuffers:
    ws = WorkingSet(batch, slots, max_len, device)
    return WorkingSetBuffers(
        ws=ws, pt=ws.page_table(),
        slot_idx=torch.empty((batch, k), dtype=torch.int32, device=device),
        loads=torch.empty((batch, k, 2), dtype=torch.int32, device=device),
        load_count=torch.empty((batch,), dtype=torch.int32, device=device),
        dev_pools=[torch.empty((batch * slots // 64, 64, row_dim), dtype=dtype, device=device)
                   for _ in range(layers)],
        fetch_stream=torch.cuda.Stream(device=device) if overlap else None,   # default priority
        fetched=[torch.cuda.Event() for _ in range(layers)],
    )


def decode_step_working_set(q_idx, w, k_pool, host_pools, qs, pt: PageTable, k, sm_scale, buf: StepBuffers,
                            wb: WorkingSetBuffers) -> None:
    """One decode token per request through the layers of an IndexShare group whose latent
    caches live in pinned host memory (host_pools): the indexer and top-k over the device
    key cache, one working-set plan for the group's shared selection, then per layer the
    loads of its missing rows and its attention over the working set.  With a fetch stream
    the loads of layer l + 1 run while layer l attends (SemiAnalysis, introduction: the
    layer-wise overlap HiSparse takes from HiCache)."""
    dsa_indexer_scores(q_idx, w, k_pool, pt, buf.scores)
    dsa_topk(buf.scores, pt.seq_len, pt.seq_len_host, k, buf.idx, n_add=0, ws=buf.ws_topk)
    dsa_working_set_plan(wb.ws, buf.idx, k, wb.slot_idx, wb.loads, wb.load_count)
    cur = torch.cuda.current_stream(q_idx.device)
    if wb.fetch_stream is None:
        for layer, (host, q) in enumerate(zip(host_pools, qs)):
            dsa_working_set_fetch(wb.ws, host, pt, wb.loads, wb.load_count, k, wb.dev_pools[layer])
            dsa_sparse_mla_decode(q, wb.dev_pools[layer], wb.pt, wb.slot_idx, k, sm_scale, buf.outs[layer],
                                  buf.lses[layer], ws=buf.ws_mla)
        return
    planned = torch.cuda.Event()
    planned.record(cur)
    wb.fetch_stream.wait_event(planned)
    for layer, host in enumerate(host_pools):
        dsa_working_set_fetch(wb.ws, host, pt, wb.loads, wb.load_count, k, wb.dev_pools[layer],
                              stream=wb.fetch_stream)
        wb.fetched[layer].record(wb.fetch_stream)
    for layer, q in enumerate(qs):
        cur.wait_event(wb.fetched[layer])
        dsa_sparse_mla_decode(q, wb.dev_pools[layer], wb.pt, wb.slot_idx, k, sm_scale, buf.outs[layer],
                              buf.lses[layer], ws=buf.ws_mla)


def page_table(inp: dict) -> PageTable:
    """The page table of an input set from dsa_inputs.make_inputs."""
    return PageTable(inp["block_table"], inp["seq_len"], inp["seq_len_host"])


def chunk(inp: dict) -> Chunk:
    """The query-token positions of a prefill input set."""
    return Chunk(inp["q_row"], inp["q_pos"], inp["q_row_host"], inp["q_pos_host"])


def run_inputs(inp: dict, buf: Optional[StepBuffers] = None, step: int = 0, pt: Optional[PageTable] = None,
               ch: Optional[Chunk] = None) -> StepBuffers:
    """Run one step on an input set from dsa_inputs.make_inputs (tensors on the GPU).
    pt / ch: the input set's PageTable and Chunk when the caller keeps them (else built
    here from the set)."""
    cfg = inp["cfg"]
    T = inp["q_idx"].shape[0]
    ld = inp["block_table"].shape[1] * 64
    if buf is None:
        buf = alloc_buffers(T, ld, cfg.k, cfg.H, cfg.Dl, cfg.layers, cfg.dtype, inp["q_idx"].device,
                            share=cfg.index_share)
    pt = pt or page_table(inp)
    if cfg.prefill_tokens:
        prefill_step(inp["q_idx"], inp["w"], inp["k_pool"], inp["kv_pools"], inp["q"], pt, ch or chunk(inp),
                     cfg.k, cfg.sm_scale, buf, step)
    else:
        decode_step(inp["q_idx"], inp["w"], inp["k_pool"], inp["kv_pools"], inp["q"], pt, cfg.k, cfg.sm_scale,
                    buf, step, share=cfg.index_share)
    return buf


class StepGraph:
    """One whole step of an input set captured once as a HIP graph (torch.cuda.CUDAGraph
    records a HIP graph on ROCm) and replayed with a single launch call: the indexer, the
    top-k and every layer's sparse MLA (and split combine) as graph nodes, with no per-kernel
    host work at replay time.

    The library enqueues kernel launches only (no memset, copy or allocation nodes), on
    torch's current stream, which is the capture stream inside torch.cuda.graph.  What the
    host does per call happens once, at capture: argument checks, kernel and split choices
    from the host lengths, and the IndexShare cache's step stamp.  A replay therefore
    repeats the captured step over the same buffers: new inputs are written into those
    tensors in place, with the same lengths and page layout (the host lengths decide the
    launch shapes)."""

    def __init__(self, inp: dict, buf: StepBuffers, step: int = 0, pt: Optional[PageTable] = None,
                 ch: Optional[Chunk] = None):
        self.inp, self.buf = inp, buf
        self.pt = pt or page_table(inp)
        self.ch = ch if ch is not None or not inp["cfg"].prefill_tokens else chunk(inp)
        # one eager step on a side stream first (torch's capture recipe: whatever is set up
        # lazily on first use happens outside the capture)
        side = torch.cuda.Stream(device=inp["q_idx"].device)   # default priority
        side.wait_stream(torch.cuda.current_stream(inp["q_idx"].device))
        with torch.cuda.stream(side):
            run_inputs(inp, buf, step, self.pt, self.ch)
        torch.cuda.current_stream(inp["q_idx"].device).wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            run_inputs(inp, buf, step, self.pt, self.ch)

    def replay(self) -> StepBuffers:
        self.graph.replay()
        return self.buf
