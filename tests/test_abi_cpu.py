"""The C ABI on a host without a GPU: the library loads, exports every entry point that
include/dsa.h declares, and rejects invalid arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

from sparse_attention_19_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # 16-byte aligned, never dereferenced: every call below is rejected
FAKE2 = 0x20000
ACCEPTED = "accepted"   # lengths that pass every check (see test_topk_rejects)


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 24
    assert sorted(L.EXPORTS) == names
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert L.LIB.dsa_status_string(L.DSA_OK) == b"DSA_OK"
    assert L.LIB.dsa_status_string(L.DSA_ERR_STALE_INDEX) == b"DSA_ERR_STALE_INDEX"
    assert L.LIB.dsa_status_string(99) == b"DSA_ERR_UNKNOWN"
    assert L.LIB.dsa_version().startswith(b"dsa-gfx950")


def pool(dtype=L.DSA_BF16, row=128, nblk=10, data=FAKE, bs=64):
    return L.DsaPool(data, nblk, bs, row, dtype)


_KEEP = []   # host arrays referenced by structs built below


def host_i32(values):
    arr = (ctypes.c_int32 * max(1, len(values)))(*values)
    _KEEP.append(arr)
    return ctypes.cast(arr, ctypes.c_void_p).value


def pt(batch=2, max_blocks=4, lens=None, seq_len_host=True):
    lens = [max_blocks * 64 - 1] * batch if lens is None else lens
    return L.DsaPageTable(FAKE, FAKE2, host_i32(lens) if seq_len_host else None, batch, max_blocks)


def chunk(rows, poss, host=True):
    return L.DsaChunk(FAKE, FAKE2, host_i32(rows) if host else None, host_i32(poss) if host else None)


def idx_call(**kw):
    a = dict(q_idx=FAKE, w=FAKE, pool=pool(), pt=pt(), chunk=None, T=2, Hi=64, Di=128, scores=FAKE, ld=256)
    a.update(kw)
    return L.LIB.dsa_indexer_scores(a["q_idx"], a["w"], ctypes.byref(a["pool"]) if a["pool"] else None,
                                    ctypes.byref(a["pt"]) if a["pt"] else None,
                                    ctypes.byref(a["chunk"]) if a["chunk"] else None,
                                    a["T"], a["Hi"], a["Di"], a["scores"], a["ld"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q_idx=None), L.DSA_ERR_INVALID),
    (dict(w=None), L.DSA_ERR_INVALID),
    (dict(scores=None), L.DSA_ERR_INVALID),
    (dict(pool=None), L.DSA_ERR_INVALID),
    (dict(pt=None), L.DSA_ERR_INVALID),
    (dict(pool=pool(data=None)), L.DSA_ERR_INVALID),
    (dict(pool=pool(bs=32)), L.DSA_ERR_UNSUPPORTED),
    (dict(pool=pool(nblk=0)), L.DSA_ERR_INVALID),
    (dict(pool=pool(row=64)), L.DSA_ERR_INVALID),
    (dict(pool=pool(dtype=7)), L.DSA_ERR_UNSUPPORTED),
    (dict(pool=pool(data=FAKE + 4)), L.DSA_ERR_INVALID),
    (dict(T=3), L.DSA_ERR_INVALID),                       # decode: T must equal batch
    (dict(ld=255), L.DSA_ERR_INVALID),                    # ld < max_blocks * 64
    (dict(pt=pt(seq_len_host=False)), L.DSA_ERR_INVALID),            # no host lengths
    (dict(pt=pt(lens=[256, 257])), L.DSA_ERR_INVALID),               # seq_len > max_blocks * 64
    (dict(pt=pt(lens=[-1, 5])), L.DSA_ERR_INVALID),                  # negative length
    (dict(pt=pt(lens=[256, 0])), L.DSA_OK),                          # both ends of the range
    (dict(chunk=chunk([0, 1], [5, 5], host=False)), L.DSA_ERR_INVALID),   # chunk without host copies
    (dict(chunk=chunk([0, 2], [5, 5])), L.DSA_ERR_INVALID),          # q_row outside the batch
    (dict(chunk=chunk([0, -1], [5, 5])), L.DSA_ERR_INVALID),
    (dict(chunk=chunk([0, 1], [5, 255])), L.DSA_ERR_INVALID),        # q_pos >= seq_len (255)
    (dict(chunk=chunk([0, 1], [-1, 5])), L.DSA_ERR_INVALID),         # negative position
    (dict(Hi=32), L.DSA_ERR_UNSUPPORTED),                 # bf16 instance is 64 x 128
    (dict(Hi=8, Di=32, pool=pool(L.DSA_F32, row=32)), L.DSA_OK),   # fp32 small dims are fine ...
    (dict(Hi=8, Di=30, pool=pool(L.DSA_F32, row=30)), L.DSA_ERR_UNSUPPORTED),
    (dict(Hi=65, Di=32, pool=pool(L.DSA_F32, row=32)), L.DSA_ERR_UNSUPPORTED),
    (dict(pt=L.DsaPageTable(None, FAKE2, 2, 4)), L.DSA_ERR_INVALID),
    (dict(pt=L.DsaPageTable(FAKE, FAKE2, 0, 4)), L.DSA_ERR_INVALID),
    (dict(pt=L.DsaPageTable(FAKE, FAKE2, 2, 0)), L.DSA_ERR_INVALID),
])
def test_indexer_rejects(kw, status):
    if status == L.DSA_OK:
        # valid shape: only check it is not rejected for shape reasons -- with T = 0 no launch
        kw = dict(kw, T=0, chunk=chunk([], []))
    got = idx_call(**kw)
    assert got == status, L.LIB.dsa_last_error()
    if status != L.DSA_OK:
        assert L.LIB.dsa_last_error()


def topk_call(**kw):
    a = dict(scores=FAKE, ld=1000, n_valid=FAKE2, nvh=[1000, 10, 0], n_add=0, rows=3, k=64, idx=FAKE,
             ld_idx=64, ws=None, wsb=0)
    a.update(kw)
    nvh = host_i32(a["nvh"]) if a["nvh"] is not None else None
    return L.LIB.dsa_topk(a["scores"], a["ld"], a["n_valid"], nvh, a["n_add"], a["rows"], a["k"], a["idx"],
                          a["ld_idx"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(scores=None), L.DSA_ERR_INVALID),
    (dict(n_valid=None), L.DSA_ERR_INVALID),
    (dict(idx=None), L.DSA_ERR_INVALID),
    (dict(k=0), L.DSA_ERR_UNSUPPORTED),
    (dict(k=2049, ld_idx=4096), L.DSA_ERR_UNSUPPORTED),
    (dict(ld_idx=63), L.DSA_ERR_INVALID),
    (dict(ld=0), L.DSA_ERR_INVALID),
    (dict(n_add=2), L.DSA_ERR_INVALID),
    (dict(rows=-1), L.DSA_ERR_INVALID),
    (dict(rows=0), L.DSA_OK),                             # empty: nothing enqueued
    (dict(rows=0, scores=None, idx=None, nvh=None), L.DSA_OK),   # ... and may pass NULL data
    (dict(ld=40000), L.DSA_ERR_WORKSPACE),                # long rows need the prune workspace
    (dict(nvh=None), L.DSA_ERR_INVALID),                  # no host copy of the lengths
    (dict(nvh=[1001, 10, 0]), L.DSA_ERR_INVALID),         # a row longer than ld
    (dict(nvh=[1000, 10, 0], n_add=1), L.DSA_ERR_INVALID),   # n_valid + n_add > ld
    (dict(nvh=[999, 10, -1], n_add=1), ACCEPTED),    # -1 + 1 = 0 positions: valid
    (dict(nvh=[5, -1, 0]), L.DSA_ERR_INVALID),            # negative length
])
def test_topk_rejects(kw, status):
    if status == ACCEPTED:
        # valid lengths: accepted by every check; rows=0 afterwards keeps the call launch-free
        # (the same host array is re-validated with rows=3 up to the workspace check)
        assert topk_call(**dict(kw, ld=40000)) == L.DSA_ERR_WORKSPACE
        return
    assert topk_call(**kw) == status


def mla_call(prefill=False, **kw):
    a = dict(q=FAKE, pool=pool(row=576), pt=pt(), idx=FAKE, ld_idx=2048, k=2048, H=64, Dl=512, Dr=64,
             scale=0.04, out=FAKE, lse=None, ws=FAKE2, wsb=1 << 40, chunk=chunk([0, 1], [3, 4]), T=2)
    a.update(kw)
    pp = ctypes.byref(a["pool"]) if a["pool"] else None
    tp = ctypes.byref(a["pt"]) if a["pt"] else None
    if prefill:
        cp = ctypes.byref(a["chunk"]) if a["chunk"] else None
        return L.LIB.dsa_sparse_mla_prefill(a["q"], pp, tp, cp, a["idx"], a["ld_idx"],
                                            a["T"], a["k"], a["H"], a["Dl"], a["Dr"], a["scale"], a["out"],
                                            a["lse"], a["ws"], a["wsb"], None)
    return L.LIB.dsa_sparse_mla_decode(a["q"], pp, tp, a["idx"], a["ld_idx"], a["k"], a["H"], a["Dl"],
                                       a["Dr"], a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("prefill", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), L.DSA_ERR_INVALID),
    (dict(out=None), L.DSA_ERR_INVALID),
    (dict(idx=None), L.DSA_ERR_INVALID),
    (dict(pool=None), L.DSA_ERR_INVALID),
    (dict(pt=None), L.DSA_ERR_INVALID),
    (dict(pool=pool(row=512)), L.DSA_ERR_INVALID),
    (dict(H=32), L.DSA_ERR_UNSUPPORTED),
    (dict(H=96), L.DSA_ERR_UNSUPPORTED),                  # bf16: 64 or 128 heads
    (dict(H=192), L.DSA_ERR_UNSUPPORTED),
    (dict(H=128, Dl=256, Dr=320), L.DSA_ERR_UNSUPPORTED),
    (dict(Dl=256, Dr=320), L.DSA_ERR_UNSUPPORTED),
    (dict(k=4096, ld_idx=4096), L.DSA_ERR_UNSUPPORTED),
    (dict(ld_idx=100), L.DSA_ERR_INVALID),
    (dict(scale=float("inf")), L.DSA_ERR_INVALID),
    (dict(ws=None), L.DSA_ERR_WORKSPACE),
    (dict(wsb=16), L.DSA_ERR_WORKSPACE),
    (dict(out=FAKE + 2), L.DSA_ERR_INVALID),
    (dict(pool=pool(L.DSA_F32, row=80), H=65, Dl=64, Dr=16), L.DSA_ERR_UNSUPPORTED),
    (dict(pool=pool(L.DSA_F32, row=1028), H=8, Dl=1024, Dr=4), L.DSA_ERR_UNSUPPORTED),
    (dict(pt=pt(seq_len_host=False)), L.DSA_ERR_INVALID),            # no host lengths
    (dict(pt=pt(lens=[100, 257])), L.DSA_ERR_INVALID),               # seq_len > max_blocks * 64
])
def test_mla_rejects(prefill, kw, status):
    assert mla_call(prefill, **kw) == status


@pytest.mark.parametrize("ch", [
    chunk([0, 1], [3, 4], host=False),      # no host copies of the positions
    chunk([0, 2], [3, 4]),                  # q_row outside the batch
    chunk([0, 1], [3, 255]),                # q_pos >= seq_len
    chunk([0, 1], [-1, 4]),                 # negative position
])
def test_mla_prefill_rejects_positions(ch):
    assert mla_call(True, chunk=ch) == L.DSA_ERR_INVALID


def test_mla_f32_small_dims_accepted_without_workspace():
    # an empty prefill chunk passes every check and enqueues nothing
    assert mla_call(True, T=0, pool=pool(L.DSA_F32, row=80), H=8, Dl=64, Dr=16, k=64, ld_idx=64,
                    ws=None, wsb=0, chunk=None) == L.DSA_OK


def test_prefill_requires_positions():
    assert mla_call(True, chunk=None) == L.DSA_ERR_INVALID
    assert mla_call(True, T=-1) == L.DSA_ERR_INVALID


def test_workspace_sizes():
    # decode of 1 token splits the 2048-entry list 32 ways; a 4096-token prefill does not split.
    # Per (token, split, head): 512 bf16 of normalized partial O and fp32 (max, sum)
    per = 512 * 2 + 2 * 4
    one = L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, 1, 0, 2048, 64, 512)
    assert one == 32 * 64 * per
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, 4096, 0, 2048, 64, 512) == 0
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, 0, 0, 2048, 64, 512) == 0
    # 128 heads below 64 tokens run as two 64-head workgroups per (token, split): one token
    # still splits 32 ways (64 workgroups), 32 tokens 4 ways; from 64 tokens on one workgroup
    # per (token, split) serves all 128 heads, splits = 256 / tokens: 64 tokens split 4 ways,
    # 128 tokens 2 ways, 256 tokens do not split
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, 1, 0, 2048, 128, 512) == 32 * 128 * per
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, 32, 0, 2048, 128, 512) == 32 * 4 * 128 * per
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, 63, 0, 2048, 128, 512) == 63 * 2 * 128 * per
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, 64, 0, 2048, 128, 512) == 64 * 4 * 128 * per
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, 64, 0, 2048, 64, 512) == 64 * 4 * 64 * per
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, 128, 0, 2048, 128, 512) == 128 * 2 * 128 * per
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, 256, 0, 2048, 128, 512) == 0
    # rows of at most 32768 positions are selected in one workgroup: no workspace
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_TOPK, 64, 32768, 2048, 0, 0) == 0
    # longer rows, G = min(ceil(2048 / rows), blocks of 4096, 1024) prune workgroups per
    # row: tau per row (padded to 4 words), the largest key of each prune wave (4 per
    # workgroup), a candidate count per workgroup (padded) and 8192 (key, position) pairs
    # per workgroup; with G = 1 (2048 rows or more) one workgroup per row prunes and
    # selects, its candidates in LDS: no workspace
    def words(rows, G):
        pad4 = lambda x: -(-x // 4) * 4
        return pad4(rows) + rows * G * 4 + pad4(rows * G) + rows * G * 8192 * 2
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_TOPK, 1, 40000, 2048, 0, 0) == words(1, 10) * 4
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_TOPK, 40, 131072, 2048, 0, 0) == words(40, 32) * 4
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_TOPK, 2047, 131072, 2048, 0, 0) == words(2047, 2) * 4
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_TOPK, 2048, 131072, 2048, 0, 0) == 0
    assert L.LIB.dsa_workspace_bytes(L.DSA_OP_TOPK, 4096, 131072, 2048, 0, 0) == 0


def test_index_cache_host_logic():
    c = L.DsaIndexCache()
    lib = L.LIB
    assert lib.dsa_index_cache_init(ctypes.byref(c), FAKE, 2048, 40, 2048, 4) == L.DSA_OK
    out = ctypes.c_void_p()
    assert lib.dsa_index_cache_get(ctypes.byref(c), 0, 1, ctypes.byref(out)) == L.DSA_ERR_STALE_INDEX
    assert lib.dsa_index_cache_publish(ctypes.byref(c), 7) == L.DSA_OK
    for layer in (1, 2, 3):
        out = ctypes.c_void_p()
        assert lib.dsa_index_cache_get(ctypes.byref(c), 7, layer, ctypes.byref(out)) == L.DSA_OK
        assert out.value == FAKE
    assert lib.dsa_index_cache_get(ctypes.byref(c), 7, 0, ctypes.byref(out)) == L.DSA_ERR_STALE_INDEX
    assert lib.dsa_index_cache_get(ctypes.byref(c), 7, 4, ctypes.byref(out)) == L.DSA_ERR_STALE_INDEX
    assert lib.dsa_index_cache_get(ctypes.byref(c), 8, 1, ctypes.byref(out)) == L.DSA_ERR_STALE_INDEX
    assert lib.dsa_index_cache_publish(ctypes.byref(c), 8) == L.DSA_OK
    assert lib.dsa_index_cache_get(ctypes.byref(c), 7, 1, ctypes.byref(out)) == L.DSA_ERR_STALE_INDEX
    assert lib.dsa_index_cache_init(ctypes.byref(c), FAKE, 100, 40, 2048, 4) == L.DSA_ERR_INVALID
    assert lib.dsa_index_cache_init(ctypes.byref(c), FAKE, 2048, 40, 2048, 1) == L.DSA_ERR_INVALID
    assert lib.dsa_index_cache_init(ctypes.byref(c), None, 2048, 40, 2048, 4) == L.DSA_ERR_INVALID


def test_timing_rejects_before_any_hip_call():
    assert L.LIB.dsa_timing_start(0) == L.DSA_ERR_INVALID
    assert L.LIB.dsa_timing_start((1 << 20) + 1) == L.DSA_ERR_INVALID
    # never started: collect reports -1 and says why
    assert L.LIB.dsa_timing_collect(None, None, 0) == -1
    assert b"off" in L.LIB.dsa_last_error()


def noalloc_call(**kw):
    a = dict(q=FAKE, pool=pool(row=576), pt=pt(), idx=FAKE, ld_idx=2048, k=2048, H=64, Dl=512, Dr=64,
             scale=0.04, out=FAKE, lse=None)
    a.update(kw)
    pp = ctypes.byref(a["pool"]) if a["pool"] else None
    tp = ctypes.byref(a["pt"]) if a["pt"] else None
    return L.LIB.dsa_sparse_mla_decode_noalloc(a["q"], pp, tp, a["idx"], a["ld_idx"], a["k"], a["H"], a["Dl"],
                                               a["Dr"], a["scale"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), L.DSA_ERR_INVALID),
    (dict(pt=None), L.DSA_ERR_INVALID),
    (dict(pt=pt(seq_len_host=False)), L.DSA_ERR_INVALID),
    (dict(pt=pt(lens=[100, 257])), L.DSA_ERR_INVALID),
    (dict(H=96), L.DSA_ERR_UNSUPPORTED),
    (dict(k=4096, ld_idx=4096), L.DSA_ERR_UNSUPPORTED),
    (dict(out=FAKE + 2), L.DSA_ERR_INVALID),
])
def test_noalloc_decode_rejects(kw, status):
    assert noalloc_call(**kw) == status


def test_noalloc_scratch_holds_every_workspace():
    # the library's scratch array (33,816,576 bytes: 256 work items of 128 heads) covers the
    # split partials of every batch size, head count and list width the bf16 decode accepts
    scratch = 256 * 128 * (512 * 2 + 2 * 4)
    for H in (64, 128):
        for k in (1, 31, 32, 33, 500, 2047, 2048):
            for T in list(range(1, 300)) + [511, 512, 1000, 4096, 100000]:
                assert L.LIB.dsa_workspace_bytes(L.DSA_OP_MLA, T, 0, k, H, 512) <= scratch, (H, k, T)


def test_probe_rejects():
    assert L.LIB.dsa_probe_row_gather(None, 10, FAKE, 100, 0, FAKE2, None) == L.DSA_ERR_INVALID
    assert L.LIB.dsa_probe_row_gather(FAKE, 0, FAKE, 100, 0, FAKE2, None) == L.DSA_ERR_INVALID
    assert L.LIB.dsa_probe_row_gather(FAKE, 10, FAKE, 0, 0, FAKE2, None) == L.DSA_ERR_INVALID
    assert L.LIB.dsa_probe_row_gather(FAKE + 8, 10, FAKE, 100, 0, FAKE2, None) == L.DSA_ERR_INVALID
    assert L.LIB.dsa_probe_row_gather(FAKE, 10, FAKE, 100, 2, FAKE2, None) == L.DSA_ERR_INVALID
    assert L.LIB.dsa_probe_row_gather_sink_words(4097) == 3 * 256


def _heads_call(fn="mha", **kw):
    a = dict(q=FAKE, pool=pool(row=576), kv_mha=FAKE2, pt=pt(lens=[200, 255]), chunk=chunk([0, 0], [3, 4]),
             idx=FAKE, ld_idx=2048, T=2, k=2048, H=64, scale=0.0625, out=FAKE, lse=None, ws=FAKE2, wsb=1 << 40,
             thr=1 << 20)
    a.update(kw)
    pp = ctypes.byref(a["pool"]) if a["pool"] else None
    tp = ctypes.byref(a["pt"]) if a["pt"] else None
    cp = ctypes.byref(a["chunk"]) if a["chunk"] else None
    if fn == "mha":
        return L.LIB.dsa_sparse_mla_prefill_mha(a["q"], pp, a["kv_mha"], tp, cp, a["idx"], a["ld_idx"], a["T"], a["k"],
                                                a["H"], a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)
    mode = ctypes.c_int32(-1)
    return L.LIB.dsa_mla_prefill_heads(a["q"], FAKE, FAKE2, pp, a["kv_mha"], tp, cp, a["idx"], a["ld_idx"], a["T"],
                                       a["k"], a["H"], a["scale"], a["thr"], a["out"], a["lse"], ctypes.byref(mode),
                                       a["ws"], a["wsb"], None)


@pytest.mark.parametrize("fn", ["mha", "heads"])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), L.DSA_ERR_INVALID),
    (dict(pool=pool(L.DSA_F32, row=576)), L.DSA_ERR_UNSUPPORTED),      # bf16 only
    (dict(pool=pool(row=512)), L.DSA_ERR_INVALID),                     # latent rows are 512 + 64
    (dict(H=0), L.DSA_ERR_UNSUPPORTED),
    (dict(H=129), L.DSA_ERR_UNSUPPORTED),
    (dict(chunk=chunk([0, 1], [3, 255])), L.DSA_ERR_INVALID),          # q_pos beyond its request
    (dict(k=4096, ld_idx=4096), L.DSA_ERR_UNSUPPORTED),
    (dict(ws=None), L.DSA_ERR_WORKSPACE),
    (dict(out=FAKE + 2), L.DSA_ERR_INVALID),
    (dict(pt=pt(seq_len_host=False)), L.DSA_ERR_INVALID),
])
def test_mla_modes_reject(fn, kw, status):
    assert _heads_call(fn, **kw) == status


def test_mha_mode_limits():
    # a 128-token tile mixing two requests, and a token seeing more than 65536 positions
    mixed = chunk([0] * 100 + [1] * 100, [5] * 200)
    assert _heads_call("mha", T=200, chunk=mixed) == L.DSA_ERR_UNSUPPORTED
    big = pt(max_blocks=2048, lens=[70000, 10])
    assert _heads_call("mha", pt=big, chunk=chunk([0, 1], [69999, 3])) == L.DSA_ERR_UNSUPPORTED
    assert _heads_call("mha", kv_mha=None) == L.DSA_ERR_INVALID
    # the switch takes MQA mode there instead: H = 32 is not an MQA-mode instance
    assert _heads_call("heads", H=32, thr=0) == L.DSA_ERR_UNSUPPORTED
    assert _heads_call("heads", T=200, chunk=mixed, thr=0, H=32) == L.DSA_ERR_UNSUPPORTED


def test_projection_rejects():
    lib = L.LIB
    assert lib.dsa_mla_up_project(ctypes.byref(pool(L.DSA_F32, row=576)), FAKE, 64, FAKE2, None) == L.DSA_ERR_UNSUPPORTED
    assert lib.dsa_mla_up_project(ctypes.byref(pool(row=576)), None, 64, FAKE2, None) == L.DSA_ERR_INVALID
    assert lib.dsa_mla_up_project(ctypes.byref(pool(row=576)), FAKE, 0, FAKE2, None) == L.DSA_ERR_UNSUPPORTED
    assert lib.dsa_mla_absorb_q(FAKE, FAKE2, -1, 64, FAKE, None) == L.DSA_ERR_INVALID
    assert lib.dsa_mla_absorb_q(FAKE, None, 4, 64, FAKE, None) == L.DSA_ERR_INVALID
    assert lib.dsa_mla_absorb_q(None, None, 0, 64, None, None) == L.DSA_OK      # empty: nothing enqueued
    assert lib.dsa_mla_unabsorb_o(FAKE + 2, FAKE2, 4, 64, FAKE, None) == L.DSA_ERR_INVALID
    assert lib.dsa_mla_unabsorb_o(FAKE, FAKE2, 4, 200, FAKE, None) == L.DSA_ERR_UNSUPPORTED
    # workspace sizes: one 64-bit mask word per token and 64 positions; MQA mode's q_abs and
    # latent output
    assert lib.dsa_workspace_bytes(L.DSA_OP_MLA_MHA, 2048, 5120, 2048, 64, 512) == 2048 * 80 * 8
    mqa = 2048 * 64 * 576 * 2 + 2048 * 64 * 512 * 2
    assert lib.dsa_workspace_bytes(L.DSA_OP_MLA_HEADS, 2048, 5120, 2048, 64, 512) == mqa


# ---- HBM working set

FAKE3 = 0x30000


def wset(batch=2, slots=4096, max_len=256, arrays=True):
    return L.DsaWorkingSet(FAKE if arrays else None, FAKE2, FAKE3, batch, slots, max_len)


def plan_call(**kw):
    a = dict(ws=wset(), idx=FAKE, ld_idx=2048, k=2048, slot_idx=FAKE2, ld_slot=2048, loads=FAKE3, load_count=FAKE)
    a.update(kw)
    return L.LIB.dsa_working_set_plan(ctypes.byref(a["ws"]) if a["ws"] else None, a["idx"], a["ld_idx"], a["k"],
                                      a["slot_idx"], a["ld_slot"], a["loads"], a["load_count"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), L.DSA_ERR_INVALID),
    (dict(ws=wset(arrays=False)), L.DSA_ERR_INVALID),
    (dict(ws=wset(batch=0)), L.DSA_ERR_UNSUPPORTED),
    (dict(ws=wset(batch=70000)), L.DSA_ERR_UNSUPPORTED),
    (dict(ws=wset(slots=4000)), L.DSA_ERR_UNSUPPORTED),
    (dict(ws=wset(slots=32768)), L.DSA_ERR_UNSUPPORTED),
    (dict(ws=wset(slots=2048)), L.DSA_ERR_UNSUPPORTED),          # slots must exceed k
    (dict(ws=wset(max_len=0)), L.DSA_ERR_INVALID),
    (dict(k=0), L.DSA_ERR_UNSUPPORTED),
    (dict(k=4096), L.DSA_ERR_UNSUPPORTED),
    (dict(idx=None), L.DSA_ERR_INVALID),
    (dict(slot_idx=None), L.DSA_ERR_INVALID),
    (dict(loads=None), L.DSA_ERR_INVALID),
    (dict(load_count=None), L.DSA_ERR_INVALID),
    (dict(ld_idx=100), L.DSA_ERR_INVALID),
    (dict(ld_slot=100), L.DSA_ERR_INVALID),
    (dict(loads=FAKE3 + 4), L.DSA_ERR_INVALID),
])
def test_working_set_plan_rejects(kw, status):
    assert plan_call(**kw) == status


def test_working_set_reset_rejects():
    assert L.LIB.dsa_working_set_reset(None, None) == L.DSA_ERR_INVALID
    assert L.LIB.dsa_working_set_reset(ctypes.byref(wset(slots=100)), None) == L.DSA_ERR_UNSUPPORTED


def fetch_call(**kw):
    a = dict(ws=wset(batch=2, max_len=256), host=pool(row=576, nblk=100), pt=pt(batch=2, max_blocks=4), loads=FAKE3,
             load_count=FAKE, k=2048, dev=pool(row=576, nblk=128, data=FAKE2))
    a.update(kw)
    ref = lambda x: ctypes.byref(x) if x is not None else None   # noqa: E731
    return L.LIB.dsa_working_set_fetch(ref(a["ws"]), ref(a["host"]), ref(a["pt"]), a["loads"], a["load_count"], a["k"],
                                       ref(a["dev"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), L.DSA_ERR_INVALID),
    (dict(k=4096), L.DSA_ERR_UNSUPPORTED),
    (dict(host=None), L.DSA_ERR_INVALID),
    (dict(host=pool(row=512, nblk=100)), L.DSA_ERR_INVALID),
    (dict(host=pool(row=576, nblk=100, dtype=L.DSA_F32)), L.DSA_ERR_UNSUPPORTED),
    (dict(dev=None), L.DSA_ERR_INVALID),
    (dict(dev=pool(row=576, nblk=127, data=FAKE2)), L.DSA_ERR_INVALID),     # fewer than batch * slots rows
    (dict(pt=None), L.DSA_ERR_INVALID),
    (dict(pt=pt(batch=3, max_blocks=4)), L.DSA_ERR_INVALID),               # batch differs from the working set
    (dict(pt=pt(batch=2, max_blocks=5)), L.DSA_ERR_INVALID),               # covers other positions than max_len
    (dict(pt=pt(batch=2, max_blocks=4, lens=[300, 10])), L.DSA_ERR_INVALID),
    (dict(loads=None), L.DSA_ERR_INVALID),
    (dict(load_count=None), L.DSA_ERR_INVALID),
    (dict(loads=FAKE3 + 4), L.DSA_ERR_INVALID),
    (dict(), L.DSA_ERR_INVALID),     # every size is right, but the history is not pinned host memory
])
def test_working_set_fetch_rejects(kw, status):
    assert fetch_call(**kw) == status

