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

from ._lib import (DSA_BF16, DSA_BLOCK, DSA_ERR_INVALID, DSA_F32, DSA_MAX_K, DSA_OP_MLA, DSA_OP_TOPK, LIB,
                   LIB_PATH, DsaError, DsaIndexCache, DsaPageTable, DsaPool, check)

__all__ = [
    "dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill",
    "IndexCache", "dsa_workspace_bytes", "workspace", "DsaError", "LIB_PATH", "DSA_OP_TOPK", "DSA_OP_MLA",
    "dsa_timing_start", "dsa_timing_collect",
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


def _pt(block_table: torch.Tensor, seq_len: torch.Tensor) -> DsaPageTable:
    if block_table.dim() != 2 or seq_len.dim() != 1 or seq_len.shape[0] != block_table.shape[0]:
        raise ValueError("block_table must be [B][max_blocks] and seq_len [B]")
    return DsaPageTable(_dev(block_table, "block_table", torch.int32), _dev(seq_len, "seq_len", torch.int32),
                        block_table.shape[0], block_table.shape[1])


def dsa_workspace_bytes(op: int, rows: int, max_len: int, k: int, H: int, Dl: int) -> int:
    return int(LIB.dsa_workspace_bytes(op, rows, max_len, k, H, Dl))


def workspace(op: int, rows: int, max_len: int, k: int, H: int, Dl: int, device) -> Optional[torch.Tensor]:
    """Allocate (with torch) the workspace an operation needs, or None."""
    n = dsa_workspace_bytes(op, rows, max_len, k, H, Dl)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def dsa_indexer_scores(q_idx, w, k_pool, block_table, seq_len, scores, q_row=None, q_pos=None, stream=None):
    """scores[t][s] for s < n_t (see dsa_indexer_scores in include/dsa.h).
    q_idx [T][Hi][Di], w [T][Hi] fp32, k_pool [nblk][64][Di], scores [T][ld] fp32."""
    T, Hi, Di = q_idx.shape
    pool, pt = _pool(k_pool, "k_pool"), _pt(block_table, seq_len)
    check(LIB.dsa_indexer_scores(_dev(q_idx, "q_idx", k_pool.dtype), _dev(w, "w", torch.float32),
                                 ctypes.byref(pool), ctypes.byref(pt), _opt(q_row, "q_row", torch.int32),
                                 _opt(q_pos, "q_pos", torch.int32), T, Hi, Di,
                                 _dev(scores, "scores", torch.float32), scores.shape[1],
                                 _stream(stream, scores)))


def dsa_topk(scores, n_valid, k, idx, n_add=0, ws=None, stream=None):
    """idx[r] = top-k positions of scores[r][:n_valid[r] + n_add] (ascending, -1 padded)."""
    rows, ld = scores.shape
    check(LIB.dsa_topk(_dev(scores, "scores", torch.float32), ld, _dev(n_valid, "n_valid", torch.int32),
                       n_add, rows, k, _dev(idx, "idx", torch.int32), idx.shape[1],
                       _opt(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(),
                       _stream(stream, scores)))


def dsa_sparse_mla_decode(q, kv_pool, block_table, seq_len, idx, k, sm_scale, out, lse=None, ws=None,
                          stream=None):
    """Absorbed-mode sparse MLA for one decode token per request.
    q [B][H][Dl+Dr], kv_pool [nblk][64][Dl+Dr], idx [B][>=k] int32, out [B][H][Dl]."""
    B, H, D = q.shape
    Dl = out.shape[2]
    pool, pt = _pool(kv_pool, "kv_pool"), _pt(block_table, seq_len)
    check(LIB.dsa_sparse_mla_decode(_dev(q, "q", kv_pool.dtype), ctypes.byref(pool), ctypes.byref(pt),
                                    _dev(idx, "idx", torch.int32), idx.shape[1], k, H, Dl, D - Dl,
                                    float(sm_scale), _dev(out, "out", kv_pool.dtype),
                                    _opt(lse, "lse", torch.float32), _opt(ws, "ws"),
                                    0 if ws is None else ws.numel() * ws.element_size(), _stream(stream, q)))


def dsa_sparse_mla_prefill(q, kv_pool, block_table, seq_len, q_row, q_pos, idx, k, sm_scale, out, lse=None,
                           ws=None, stream=None):
    """Absorbed-mode sparse MLA for a causal prefill chunk of T tokens."""
    T, H, D = q.shape
    Dl = out.shape[2]
    pool, pt = _pool(kv_pool, "kv_pool"), _pt(block_table, seq_len)
    check(LIB.dsa_sparse_mla_prefill(_dev(q, "q", kv_pool.dtype), ctypes.byref(pool), ctypes.byref(pt),
                                     _dev(q_row, "q_row", torch.int32), _dev(q_pos, "q_pos", torch.int32),
                                     _dev(idx, "idx", torch.int32), idx.shape[1], T, k, H, Dl, D - Dl,
                                     float(sm_scale), _dev(out, "out", kv_pool.dtype),
                                     _opt(lse, "lse", torch.float32), _opt(ws, "ws"),
                                     0 if ws is None else ws.numel() * ws.element_size(), _stream(stream, q)))


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
