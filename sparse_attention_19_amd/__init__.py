"""MI355X (gfx950) DeepSeek Sparse Attention hot path: Python binding of libdsa.so.

The functions below carry the names of the C entry points in include/dsa.h and only
marshal arguments: tensors become device pointers and sizes, the stream defaults to
torch's current stream.  Callers allocate every output and workspace (torch is used for
device memory and streams only).  Importing the package without the built library
raises ImportError; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import (DSA_BF16, DSA_BLOCK, DSA_ERR_INVALID, DSA_F32, DSA_MAX_K, DSA_OP_MLA, DSA_OP_MLA_HEADS,
                   DSA_OP_MLA_MHA, DSA_OP_TOPK, LIB,
                   LIB_PATH, DsaChunk, DsaError, DsaIndexCache, DsaPageTable, DsaPool, DsaWorkingSet, check)

__all__ = [
    "dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_decode", "dsa_sparse_mla_decode_noalloc",
    "dsa_sparse_mla_prefill", "dsa_mla_up_project", "dsa_mla_absorb_q", "dsa_mla_unabsorb_o",
    "dsa_sparse_mla_prefill_mha", "dsa_mla_prefill_heads", "DSA_OP_MLA_MHA", "DSA_OP_MLA_HEADS",
    "IndexCache", "PageTable", "Chunk", "dsa_workspace_bytes", "workspace", "DsaError", "LIB_PATH",
    "DSA_OP_TOPK", "DSA_OP_MLA",
    "dsa_timing_start", "dsa_timing_collect", "dsa_probe_row_gather",
    "WorkingSet", "dsa_working_set_reset", "dsa_working_set_plan", "dsa_working_set_fetch",
]

_DT = {torch.float32: DSA_F32, torch.bfloat16: DSA_BF16}


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _opt(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    return None if t is None else _dev(t, name, dtype)


def _stream(stream, ref: torch.Tensor) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(ref.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _pool(pool: torch.Tensor, name: str) -> DsaPool:
    if pool.dim() != 3 or pool.shape[1] != DSA_BLOCK:
        raise ValueError(f"{name} must be [num_blocks][{DSA_BLOCK}][row_dim]")
    if pool.dtype not in _DT:
        raise ValueError(f"{name}: dtype {pool.dtype} not supported")
    return DsaPool(_dev(pool, name), pool.shape[0], DSA_BLOCK, pool.shape[2], _DT[pool.dtype])


def _host(t: torch.Tensor, name: str) -> int:
    """Host pointer of a CPU int32 tensor (the host copy of a device length array)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 host (CPU) tensor")
    return t.data_ptr()


class PageTable:
    """dsa_page_table: block_table [B][max_blocks] and seq_len [B] on the device, and the
    host copy seq_len_host [B] (CPU int32, the same values) that the library checks."""

    def __init__(self, block_table: torch.Tensor, seq_len: torch.Tensor, seq_len_host: torch.Tensor):
        if block_table.dim() != 2 or seq_len.dim() != 1 or seq_len.shape[0] != block_table.shape[0]:
            raise ValueError("block_table must be [B][max_blocks] and seq_len [B]")
        if seq_len_host.shape != seq_len.shape:
            raise ValueError("seq_len_host must have the shape of seq_len")
        self.tensors = (block_table, seq_len, seq_len_host)   # kept alive with the struct
        self.c = DsaPageTable(_dev(block_table, "block_table", torch.int32), _dev(seq_len, "seq_len", torch.int32),
                              _host(seq_len_host, "seq_len_host"), block_table.shape[0], block_table.shape[1])

    @property
    def batch(self) -> int:
        return self.c.batch

    @property
    def seq_len(self) -> torch.Tensor:
        return self.tensors[1]

    @property
    def seq_len_host(self) -> torch.Tensor:
        return self.tensors[2]


class Chunk:
    """dsa_chunk: the request q_row [T] and position q_pos [T] of each query token of a
    prefill chunk on the device, and their host copies (CPU int32, the same values)."""

    def __init__(self, q_row: torch.Tensor, q_pos: torch.Tensor, q_row_host: torch.Tensor,
                 q_pos_host: torch.Tensor):
        T = q_row.shape[0]
        if any(x.dim() != 1 or x.shape[0] != T for x in (q_pos, q_row_host, q_pos_host)):
            raise ValueError("q_row, q_pos and their host copies must all be [T]")
        self.tensors = (q_row, q_pos, q_row_host, q_pos_host)
        self.T = T
        self.q_pos, self.q_pos_host = q_pos, q_pos_host
        self.c = DsaChunk(_dev(q_row, "q_row", torch.int32), _dev(q_pos, "q_pos", torch.int32),
                          _host(q_row_host, "q_row_host"), _host(q_pos_host, "q_pos_host"))


def dsa_workspace_bytes(op: int, rows: int, max_len: int, k: int, H: int, Dl: int) -> int:
    return int(LIB.dsa_workspace_bytes(op, rows, max_len, k, H, Dl))


def workspace(op: int, rows: int, max_len: int, k: int, H: int, Dl: int, device) -> Optional[torch.Tensor]:
    """Allocate (with torch) the workspace an operation needs, or None."""
    n = dsa_workspace_bytes(op, rows, max_len, k, H, Dl)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _ws(ws):
    return (_opt(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size())


def dsa_indexer_scores(q_idx, w, k_pool, pt: PageTable, scores, chunk: Optional[Chunk] = None, stream=None):
    """scores[t][s] for s < n_t (see dsa_indexer_scores in include/dsa.h).
    q_idx [T][Hi][Di], w [T][Hi] fp32, k_pool [nblk][64][Di], scores [T][ld] fp32;
    chunk None = decode (one token per request)."""
    T, Hi, Di = q_idx.shape
    pool = _pool(k_pool, "k_pool")
    check(LIB.dsa_indexer_scores(_dev(q_idx, "q_idx", k_pool.dtype), _dev(w, "w", torch.float32),
                                 ctypes.byref(pool), ctypes.byref(pt.c),
                                 None if chunk is None else ctypes.byref(chunk.c), T, Hi, Di,
                                 _dev(scores, "scores", torch.float32), scores.shape[1],
                                 _stream(stream, scores)))


def dsa_topk(scores, n_valid, n_valid_host, k, idx, n_add=0, ws=None, stream=None):
    """idx[r] = top-k positions of scores[r][:n_valid[r] + n_add] (ascending, -1 padded);
    n_valid_host is the CPU int32 copy of n_valid."""
    rows, ld = scores.shape
    if n_valid_host.shape != n_valid.shape:
        raise ValueError("n_valid_host must have the shape of n_valid")
    check(LIB.dsa_topk(_dev(scores, "scores", torch.float32), ld, _dev(n_valid, "n_valid", torch.int32),
                       _host(n_valid_host, "n_valid_host"), n_add, rows, k, _dev(idx, "idx", torch.int32),
                       idx.shape[1], *_ws(ws), _stream(stream, scores)))


def dsa_sparse_mla_decode(q, kv_pool, pt: PageTable, idx, k, sm_scale, out, lse=None, ws=None, stream=None):
    """Absorbed-mode sparse MLA for one decode token per request.
    q [B][H][Dl+Dr], kv_pool [nblk][64][Dl+Dr], idx [B][>=k] int32, out [B][H][Dl]."""
    B, H, D = q.shape
    Dl = out.shape[2]
    pool = _pool(kv_pool, "kv_pool")
    check(LIB.dsa_sparse_mla_decode(_dev(q, "q", kv_pool.dtype), ctypes.byref(pool), ctypes.byref(pt.c),
                                    _dev(idx, "idx", torch.int32), idx.shape[1], k, H, Dl, D - Dl,
                                    float(sm_scale), _dev(out, "out", kv_pool.dtype),
                                    _opt(lse, "lse", torch.float32), *_ws(ws), _stream(stream, q)))


def dsa_sparse_mla_decode_noalloc(q, kv_pool, pt: PageTable, idx, k, sm_scale, out, lse=None, stream=None):
    """dsa_sparse_mla_decode with the split partials in the library's own device array:
    no workspace argument, no allocation (calls that overlap on one GPU race)."""
    B, H, D = q.shape
    Dl = out.shape[2]
    pool = _pool(kv_pool, "kv_pool")
    check(LIB.dsa_sparse_mla_decode_noalloc(_dev(q, "q", kv_pool.dtype), ctypes.byref(pool), ctypes.byref(pt.c),
                                            _dev(idx, "idx", torch.int32), idx.shape[1], k, H, Dl, D - Dl,
                                            float(sm_scale), _dev(out, "out", kv_pool.dtype),
                                            _opt(lse, "lse", torch.float32), _stream(stream, q)))


def dsa_sparse_mla_prefill(q, kv_pool, pt: PageTable, chunk: Chunk, idx, k, sm_scale, out, lse=None, ws=None,
                           stream=None):
    """Absorbed-mode sparse MLA for a causal prefill chunk of T tokens."""
    T, H, D = q.shape
    Dl = out.shape[2]
    pool = _pool(kv_pool, "kv_pool")
    check(LIB.dsa_sparse_mla_prefill(_dev(q, "q", kv_pool.dtype), ctypes.byref(pool), ctypes.byref(pt.c),
                                     ctypes.byref(chunk.c), _dev(idx, "idx", torch.int32), idx.shape[1], T, k,
                                     H, Dl, D - Dl, float(sm_scale), _dev(out, "out", kv_pool.dtype),
                                     _opt(lse, "lse", torch.float32), *_ws(ws), _stream(stream, q)))


def dsa_mla_up_project(kv_pool, w_kv, kv_mha, stream=None):
    """kv_mha [num_blocks * 64][H][320] = per-head NoPE keys and values of every latent row."""
    H = w_kv.shape[0]
    pool = _pool(kv_pool, "kv_pool")
    if kv_mha.numel() != kv_pool.shape[0] * kv_pool.shape[1] * H * 320:
        raise ValueError("kv_mha must hold num_blocks * 64 x H x 320 elements")
    check(LIB.dsa_mla_up_project(ctypes.byref(pool), _dev(w_kv, "w_kv", torch.bfloat16), H,
                                 _dev(kv_mha, "kv_mha", torch.bfloat16), _stream(stream, kv_mha)))


def dsa_mla_absorb_q(q_mha, w_uk, q_abs, stream=None):
    """q_abs [T][H][576] = [W_UK_h . q_nope, q_rope] (MQA mode's query)."""
    T, H, _ = q_mha.shape
    check(LIB.dsa_mla_absorb_q(_dev(q_mha, "q_mha", torch.bfloat16), _dev(w_uk, "w_uk", torch.bfloat16), T, H,
                               _dev(q_abs, "q_abs", torch.bfloat16), _stream(stream, q_abs)))


def dsa_mla_unabsorb_o(o_lat, w_kv, o, stream=None):
    """o [T][H][128] = o_lat [T][H][512] . W_UV_h (MQA mode's output to the value space)."""
    T, H, _ = o_lat.shape
    check(LIB.dsa_mla_unabsorb_o(_dev(o_lat, "o_lat", torch.bfloat16), _dev(w_kv, "w_kv", torch.bfloat16), T, H,
                                 _dev(o, "o", torch.bfloat16), _stream(stream, o)))


def dsa_sparse_mla_prefill_mha(q_mha, kv_pool, kv_mha, pt: PageTable, chunk: Chunk, idx, k, sm_scale, out, lse=None,
                               ws=None, stream=None):
    """MHA-mode attention of a prefill chunk: q_mha [T][H][256] -> out [T][H][128]."""
    T, H, _ = q_mha.shape
    pool = _pool(kv_pool, "kv_pool")
    check(LIB.dsa_sparse_mla_prefill_mha(_dev(q_mha, "q_mha", torch.bfloat16), ctypes.byref(pool),
                                         _dev(kv_mha, "kv_mha", torch.bfloat16), ctypes.byref(pt.c),
                                         ctypes.byref(chunk.c), _dev(idx, "idx", torch.int32), idx.shape[1], T, k, H,
                                         float(sm_scale), _dev(out, "out", torch.bfloat16),
                                         _opt(lse, "lse", torch.float32), *_ws(ws), _stream(stream, out)))


def dsa_mla_prefill_heads(q_mha, w_uk, w_kv, kv_pool, kv_mha, pt: PageTable, chunk: Chunk, idx, k, sm_scale,
                          mha_max_len, out, lse=None, ws=None, stream=None) -> int:
    """out [T][H][128] by MHA mode (no token sees more than mha_max_len positions and kv_mha
    is given) or MQA mode; returns 1 for MHA mode, 0 for MQA mode."""
    T, H, _ = q_mha.shape
    pool = _pool(kv_pool, "kv_pool")
    mode = ctypes.c_int32(-1)
    check(LIB.dsa_mla_prefill_heads(_dev(q_mha, "q_mha", torch.bfloat16), _dev(w_uk, "w_uk", torch.bfloat16),
                                    _dev(w_kv, "w_kv", torch.bfloat16), ctypes.byref(pool),
                                    _opt(kv_mha, "kv_mha", torch.bfloat16), ctypes.byref(pt.c), ctypes.byref(chunk.c),
                                    _dev(idx, "idx", torch.int32), idx.shape[1], T, k, H, float(sm_scale),
                                    int(mha_max_len), _dev(out, "out", torch.bfloat16),
                                    _opt(lse, "lse", torch.float32), ctypes.byref(mode), *_ws(ws),
                                    _stream(stream, out)))
    return mode.value


class IndexCache:
    """IndexShare top-k cache over a caller-owned idx tensor [rows][ld] (dsa_index_cache_*)."""

    def __init__(self, idx: torch.Tensor, k: int, group: int = 4):
        self.idx = idx
        self.c = DsaIndexCache()
        check(LIB.dsa_index_cache_init(ctypes.byref(self.c), _dev(idx, "idx", torch.int32), idx.shape[1],
                                       idx.shape[0], k, group))

    def publish(self, step: int) -> None:
        check(LIB.dsa_index_cache_publish(ctypes.byref(self.c), step))

    def get(self, step: int, layer_in_group: int) -> torch.Tensor:
        p = ctypes.c_void_p()
        check(LIB.dsa_index_cache_get(ctypes.byref(self.c), step, layer_in_group, ctypes.byref(p)))
        assert p.value == self.idx.data_ptr()
        return self.idx


class WorkingSet:
    """dsa_working_set: the HBM working set of `slots` latent rows per request, its state in
    three device int32 tensors allocated here with torch (slot_of [batch][max_len], pos_of and
    order [batch][slots]), emptied by dsa_working_set_reset on the current stream.

    page_table() is the table through which the sparse MLA reads the working-set pool:
    request b's slots are blocks b * slots / 64 .. and every slot is visible."""

    def __init__(self, batch: int, slots: int, max_len: int, device):
        self.slot_of = torch.empty((batch, max_len), dtype=torch.int32, device=device)
        self.pos_of = torch.empty((batch, slots), dtype=torch.int32, device=device)
        self.order = torch.empty((batch, slots), dtype=torch.int32, device=device)
        self.batch, self.slots, self.max_len = batch, slots, max_len
        self.c = DsaWorkingSet(self.slot_of.data_ptr(), self.pos_of.data_ptr(), self.order.data_ptr(), batch, slots,
                               max_len)
        dsa_working_set_reset(self)

    def page_table(self) -> PageTable:
        dev = self.slot_of.device
        nb = self.slots // DSA_BLOCK
        bt = (torch.arange(self.batch, dtype=torch.int32, device=dev)[:, None] * nb
              + torch.arange(nb, dtype=torch.int32, device=dev)[None, :]).contiguous()
        lens_host = torch.full((self.batch,), self.slots, dtype=torch.int32)
        return PageTable(bt, lens_host.to(dev), lens_host)


def dsa_working_set_reset(ws: WorkingSet, stream=None) -> None:
    check(LIB.dsa_working_set_reset(ctypes.byref(ws.c), _stream(stream, ws.slot_of)))


def dsa_working_set_plan(ws: WorkingSet, idx, k, slot_idx, loads, load_count, stream=None) -> None:
    """One decode step of the working set for selection idx [batch][>= k]: writes slot_idx
    [batch][>= k], loads [batch][k][2] and load_count [batch] (device int32)."""
    if loads.dim() != 3 or loads.shape[2] != 2 or loads.shape[0] != ws.batch or loads.shape[1] != k:
        raise ValueError("loads must be [batch][k][2]")
    if load_count.numel() != ws.batch or slot_idx.shape[0] != ws.batch or idx.shape[0] != ws.batch:
        raise ValueError("idx, slot_idx and load_count need one row per request")
    check(LIB.dsa_working_set_plan(ctypes.byref(ws.c), _dev(idx, "idx", torch.int32), idx.shape[1], k,
                                   _dev(slot_idx, "slot_idx", torch.int32), slot_idx.shape[1],
                                   _dev(loads, "loads", torch.int32), _dev(load_count, "load_count", torch.int32),
                                   _stream(stream, idx)))


def dsa_working_set_fetch(ws: WorkingSet, host_kv: torch.Tensor, pt: PageTable, loads, load_count, k,
                          dev_kv: torch.Tensor, stream=None) -> None:
    """Copy the planned rows of one layer from its history host_kv (a pinned CPU tensor
    [num_blocks][64][576] bf16) into dev_kv (device [batch * slots / 64][64][576] bf16)."""
    if not isinstance(host_kv, torch.Tensor) or host_kv.is_cuda or not host_kv.is_pinned():
        raise ValueError("host_kv must be a pinned host (CPU) tensor")
    if host_kv.dim() != 3 or host_kv.shape[1] != DSA_BLOCK or host_kv.dtype not in _DT or not host_kv.is_contiguous():
        raise ValueError(f"host_kv must be a contiguous [num_blocks][{DSA_BLOCK}][row_dim] tensor")
    if loads.dim() != 3 or loads.shape[0] != ws.batch or loads.shape[1] != k or loads.shape[2] != 2:
        raise ValueError("loads must be [batch][k][2]")
    hp = DsaPool(host_kv.data_ptr(), host_kv.shape[0], DSA_BLOCK, host_kv.shape[2], _DT[host_kv.dtype])
    check(LIB.dsa_working_set_fetch(ctypes.byref(ws.c), ctypes.byref(hp), ctypes.byref(pt.c),
                                    _dev(loads, "loads", torch.int32), _dev(load_count, "load_count", torch.int32), k,
                                    ctypes.byref(_pool(dev_kv, "dev_kv")), _stream(stream, dev_kv)))


def dsa_probe_row_gather(pool: torch.Tensor, rows: torch.Tensor, sink: Optional[torch.Tensor] = None,
                         lines: bool = False, stream=None) -> torch.Tensor:
    """Measurement aid: gather pool rows (1152-byte rows, [nrows][576] bf16) listed in rows
    with the sparse MLA's loads (or whole cache lines); returns the checksum sink
    (allocated here if not given)."""
    if pool.element_size() * pool.shape[-1] != 1152:
        raise ValueError("pool rows must be 1152 bytes")
    nrows = pool.numel() * pool.element_size() // 1152
    words = int(LIB.dsa_probe_row_gather_sink_words(rows.numel()))
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=pool.device)
    check(LIB.dsa_probe_row_gather(_dev(pool, "pool"), nrows, _dev(rows, "rows", torch.int32), rows.numel(),
                                   int(lines), _dev(sink, "sink", torch.int32), _stream(stream, pool)))
    return sink


def dsa_timing_start(capacity: int) -> None:
    """Time every kernel the library enqueues from now on (first `capacity` launches)."""
    check(LIB.dsa_timing_start(capacity))


def dsa_timing_collect(cap: int = 1 << 16):
    """Wait for the timed launches and return [(kernel name, ms)] in launch order."""
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = LIB.dsa_timing_collect(names, ms, cap)
    if n < 0:
        raise DsaError(DSA_ERR_INVALID, LIB.dsa_last_error().decode())
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]
