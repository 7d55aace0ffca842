"""ctypes binding of libdsa.so (the C ABI declared in include/dsa.h).

Argument marshalling only: torch tensors are turned into device pointers, sizes and the
current HIP stream; every computation happens in the library's kernels.  The library
must have been built (python sparse_attention_19_amd/build.py); importing this module
without it raises ImportError -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_STALE_INDEX, DSA_ERR_HIP = range(6)
DSA_F32, DSA_BF16 = 0, 1
DSA_OP_TOPK, DSA_OP_MLA, DSA_OP_MLA_MHA, DSA_OP_MLA_HEADS = 0, 1, 2, 3
DSA_BLOCK = 64
DSA_MAX_K = 2048
ABI_VERSION = b"dsa-gfx950 0.3.0"   # argument layout this binding marshals for

EXPORTS = [
    "dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_decode", "dsa_sparse_mla_decode_noalloc",
    "dsa_sparse_mla_prefill", "dsa_mla_up_project", "dsa_mla_absorb_q", "dsa_mla_unabsorb_o",
    "dsa_sparse_mla_prefill_mha", "dsa_mla_prefill_heads", "dsa_index_cache_init", "dsa_index_cache_publish", "dsa_index_cache_get",
    "dsa_workspace_bytes", "dsa_status_string", "dsa_last_error", "dsa_version",
    "dsa_timing_start", "dsa_timing_collect", "dsa_probe_row_gather", "dsa_probe_row_gather_sink_words",
    "dsa_working_set_reset", "dsa_working_set_plan", "dsa_working_set_fetch",
]


class DsaPool(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("num_blocks", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("row_dim", ctypes.c_int32), ("dtype", ctypes.c_int)]


class DsaPageTable(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
                ("seq_len_host", ctypes.c_void_p), ("batch", ctypes.c_int32), ("max_blocks", ctypes.c_int32)]


class DsaChunk(ctypes.Structure):
    _fields_ = [("q_row", ctypes.c_void_p), ("q_pos", ctypes.c_void_p),
                ("q_row_host", ctypes.c_void_p), ("q_pos_host", ctypes.c_void_p)]


class DsaWorkingSet(ctypes.Structure):
    _fields_ = [("slot_of", ctypes.c_void_p), ("pos_of", ctypes.c_void_p), ("order", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("slots", ctypes.c_int32), ("max_len", ctypes.c_int64)]


class DsaIndexCache(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("ld", ctypes.c_int64), ("rows", ctypes.c_int32),
                ("k", ctypes.c_int32), ("group", ctypes.c_int32), ("valid", ctypes.c_int32),
                ("step", ctypes.c_uint64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python sparse_attention_19_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    pool_p, pt_p, cache_p = ctypes.POINTER(DsaPool), ctypes.POINTER(DsaPageTable), ctypes.POINTER(DsaIndexCache)
    chunk_p, ws_p = ctypes.POINTER(DsaChunk), ctypes.POINTER(DsaWorkingSet)
    sig = {
        "dsa_indexer_scores": [P, P, pool_p, pt_p, chunk_p, I32, I32, I32, P, I64, P],
        "dsa_topk": [P, I64, P, P, I32, I32, I32, P, I64, P, SZ, P],
        "dsa_sparse_mla_decode": [P, pool_p, pt_p, P, I64, I32, I32, I32, I32, F, P, P, P, SZ, P],
        "dsa_sparse_mla_decode_noalloc": [P, pool_p, pt_p, P, I64, I32, I32, I32, I32, F, P, P, P],
        "dsa_sparse_mla_prefill": [P, pool_p, pt_p, chunk_p, P, I64, I32, I32, I32, I32, I32, F, P, P, P, SZ,
                                   P],
        "dsa_mla_up_project": [pool_p, P, I32, P, P],
        "dsa_mla_absorb_q": [P, P, I32, I32, P, P],
        "dsa_mla_unabsorb_o": [P, P, I32, I32, P, P],
        "dsa_sparse_mla_prefill_mha": [P, pool_p, P, pt_p, chunk_p, P, I64, I32, I32, I32, F, P, P, P, SZ, P],
        "dsa_mla_prefill_heads": [P, P, P, pool_p, P, pt_p, chunk_p, P, I64, I32, I32, I32, F, I64, P, P,
                                  ctypes.POINTER(I32), P, SZ, P],
        "dsa_index_cache_init": [cache_p, P, I64, I32, I32, I32],
        "dsa_index_cache_publish": [cache_p, ctypes.c_uint64],
        "dsa_index_cache_get": [cache_p, ctypes.c_uint64, I32, ctypes.POINTER(ctypes.c_void_p)],
        "dsa_workspace_bytes": [I32, I32, I64, I32, I32, I32],
        "dsa_status_string": [ctypes.c_int],
        "dsa_last_error": [],
        "dsa_version": [],
        "dsa_timing_start": [I32],
        "dsa_timing_collect": [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(F), I32],
        "dsa_probe_row_gather": [P, I64, P, I64, I32, P, P],
        "dsa_probe_row_gather_sink_words": [I64],
        "dsa_working_set_reset": [ws_p, P],
        "dsa_working_set_plan": [ws_p, P, I64, I32, P, I64, P, P, P],
        "dsa_working_set_fetch": [ws_p, pool_p, pt_p, P, P, I32, pool_p, P],
    }
    missing = [n for n in sig if not hasattr(lib, n)]
    if missing:
        raise ImportError(f"{LIB_PATH} is stale (no {', '.join(missing)}): rebuild it with "
                          f"`python sparse_attention_19_amd/build.py`")
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.dsa_workspace_bytes.restype = ctypes.c_size_t
    lib.dsa_probe_row_gather_sink_words.restype = ctypes.c_size_t
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_version.restype = ctypes.c_char_p
    if lib.dsa_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} is stale ({lib.dsa_version().decode()}, this binding expects "
                          f"{ABI_VERSION.decode()}): rebuild it with `python sparse_attention_19_amd/build.py`")
    return lib


LIB = _load()


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{LIB.dsa_status_string(status).decode()}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != DSA_OK:
        raise DsaError(status, LIB.dsa_last_error().decode())
