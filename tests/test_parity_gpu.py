"""HIP path vs the CPU oracle, element by element, through the C ABI.

Bars: indexer scores and top-k index sets bit-exact; attention outputs within the
normwise relative error 1e-5 (fp32) / 2e-2 (bf16) per (token, head) row:
max_c |out - ref| / max_c |ref|; lse within 1e-5 relative (fp32) / 2e-3 absolute (bf16).
Small cases and the full-size decode workloads (the launch configuration the benchmark
times) check every token; the full-size prefill chunks check 64 tokens spread over the
chunk (its first and last, both sides of its midpoint, and evenly spaced ones), each
computed one by one by the oracle.
"""
import numpy as np
import pytest
import torch

import dsa_inputs as I
from oracle import run as R

pytestmark = pytest.mark.gpu

import sparse_attention_19_amd as D  # noqa: E402  (fails loudly if the library is missing)
from sparse_attention_19_amd import pipeline as P  # noqa: E402

DEV = "cuda"
OUT_TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def log(msg):
    print(msg, flush=True)


def rel_rows(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max())


def check_token(inp, buf, t, layers=None, key_cache=None, check_scores=True):
    cfg = inp["cfg"]
    exp = R.expected_token(inp, t, layers, key_cache)
    n = exp["n"]
    if check_scores:
        got = buf.scores[t, :n].cpu().numpy()
        bad = np.nonzero(got.view(np.int32) != exp["scores"].view(np.int32))[0]
        assert bad.size == 0, f"token {t}: {bad.size} score mismatches, first at {bad[:5]}"
    gidx = buf.idx[t].cpu().numpy()
    assert np.array_equal(gidx, exp["idx"]), f"token {t}: top-k differs (n={n})"
    layers = range(cfg.layers) if layers is None else layers
    for li, l in enumerate(layers):
        out = R.to_f64(buf.outs[l][t])
        e = rel_rows(out, exp["out"][li])
        assert e <= OUT_TOL[cfg.dtype], f"token {t} layer {l}: out rel err {e:.3g}"
        lse = buf.lses[l][t].cpu().double().numpy()
        if cfg.dtype == torch.float32:
            assert np.allclose(lse, exp["lse"][li], rtol=1e-5, atol=1e-5)
        else:
            assert np.abs(lse - exp["lse"][li]).max() <= 2e-3, np.abs(lse - exp["lse"][li]).max()
    return exp


def set_lengths(inp, seq_len=None, q_row=None, q_pos=None):
    """Replace an input set's lengths / token positions (device tensors and host copies)."""
    for name, v in (("seq_len", seq_len), ("q_row", q_row), ("q_pos", q_pos)):
        if v is not None:
            host = torch.as_tensor(v, dtype=torch.int32).cpu().contiguous()
            inp[name + "_host"] = host
            inp[name] = host.to(DEV)


def run_cfg(cfg, **over):
    if over:
        cfg = I.shrink(cfg, **over)
    log(f"[gpu] inputs {cfg.name} {over}")
    inp = I.make_inputs(cfg, DEV)
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    return inp, buf


# ------------------------------------------------------------------ small cases, every token

def test_tiny_fp32_full_path():
    inp, buf = run_cfg(I.CONFIGS["tiny_fp32"])
    check_token(inp, buf, 0)


def test_tiny_fp32_dense_and_ragged():
    # several requests, lengths around k = 64 and not multiples of the page size
    cfg = I.shrink(I.CONFIGS["tiny_fp32"], batch=7, ctx_range=(1, 300), identity_pages=False)
    inp = I.make_inputs(cfg, DEV)
    lens = inp["seq_len"].tolist()
    log(f"[gpu] tiny ragged lens {lens}")
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    for t in range(len(lens)):
        check_token(inp, buf, t)


def test_bf16_decode_ragged_batch():
    # lengths straddle k = 2048 (dense and sparse rows), ragged last pages, random pages
    cfg = I.shrink(I.CONFIGS["decode_b64_paged"], batch=6, ctx_range=(1, 6000))
    inp = I.make_inputs(cfg, DEV)
    lens = inp["seq_len"].tolist()
    log(f"[gpu] bf16 ragged lens {lens}")
    assert min(lens) <= 2048 < max(lens)
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    for t in range(len(lens)):
        check_token(inp, buf, t)


def test_bf16_decode_h128_split():
    # 128 MLA heads (two 64-head workgroups per token and split); few tokens: split partials
    # and the combine; lengths straddle k (dense and sparse rows)
    cfg = I.shrink(I.CONFIGS["decode_b64_paged_h128"], batch=8, ctx_range=(1, 6000))
    inp = I.make_inputs(cfg, DEV)
    lens = inp["seq_len"].tolist()
    log(f"[gpu] h128 split lens {lens}")
    assert inp["q"][0].shape[1] == 128 and min(lens) <= 2048 < max(lens)
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    for t in range(len(lens)):
        check_token(inp, buf, t)


def test_bf16_decode_h128_one_gather_split():
    # 120 tokens: one workgroup per (token, split) for all 128 heads, 2 splits merged by the
    # combine kernel
    cfg = I.shrink(I.CONFIGS["decode_b64_paged_h128"], batch=120, ctx_range=(1500, 5000))
    inp = I.make_inputs(cfg, DEV)
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    for t in (0, 1, 64, 65, 118, 119):
        check_token(inp, buf, t)


def test_bf16_decode_h128_one_gather():
    # 130 tokens: one workgroup per token for all 128 heads, no split (normalized output)
    cfg = I.shrink(I.CONFIGS["decode_b64_paged_h128"], batch=130, ctx_range=(1500, 5000))
    inp = I.make_inputs(cfg, DEV)
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    for t in (0, 1, 64, 65, 128, 129):
        check_token(inp, buf, t)


def test_bf16_prefill_h128():
    cfg = I.shrink(I.CONFIGS["prefill_4096_at_128k"], ctx=2100, prefill_tokens=40, H=128)
    inp = I.make_inputs(cfg, DEV)
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    kc = {}
    for t in (0, 13, 26, 39):
        check_token(inp, buf, t, key_cache=kc)


def test_bf16_prefill_h128_unsplit():
    # 200 tokens x 128 heads: one workgroup per token serves both 64-head groups from one
    # gather.  The chunk crosses n = k (dense rows ending mid-tile, then top-k rows)
    cfg = I.shrink(I.CONFIGS["prefill_4096_at_128k"], ctx=2200, prefill_tokens=200, H=128)
    inp, buf = run_cfg(cfg)
    kc = {}
    for t in list(range(0, 200, 9)) + [47, 48, 151, 152, 199]:
        check_token(inp, buf, t, key_cache=kc)


def _scale_second_halves(inp, lens, factor):
    """Scales the latent rows of the pages holding the second half of every context."""
    bt = inp["block_table"].cpu()
    phys = sorted({int(bt[b, j]) for b, n in enumerate(lens) for j in range((n // 2) // 64 + 1, (n + 63) // 64)})
    sel = torch.tensor(phys, dtype=torch.long, device=DEV)
    for pool in inp["kv_pools"]:
        pool[sel] = (pool[sel].float() * factor).to(pool.dtype)
    return len(phys)


def test_mla_h128_running_max_moves_late():
    # the late-max case of the 64-head test for the one-gather 128-head kernel (130
    # tokens): logits rise by far more than 32 (log2 units) after the first tiles, and the
    # workgroup runs its second pass
    cfg = I.shrink(I.CONFIGS["decode_b64_paged_h128"], batch=130, ctx_range=(3000, 9000))
    inp = I.make_inputs(cfg, DEV)
    lens = inp["seq_len"].tolist()
    npg = _scale_second_halves(inp, lens, 8)
    inp["q"] = [(q.float() * 4).to(q.dtype) for q in inp["q"]]
    log(f"[gpu] h128 late-max, {npg} scaled pages")
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    for t in (0, 1, 37, 64, 100, 129):
        check_token(inp, buf, t)


@pytest.mark.parametrize("k", [1, 17, 100, 333])
def test_mla_h128_one_gather_small_k(k):
    # the one-gather kernel with lists shorter than a tile or ending mid-tile, and with
    # splits (96 tokens: 2 splits where the list has 2 tiles or more): a 96-token chunk at
    # the end of a 1200-position context, every row sparse once n > k
    cfg = I.shrink(I.CONFIGS["prefill_4096_at_128k"], seed=500 + k, ctx=1200, prefill_tokens=96, H=128, k=k,
                   identity_pages=False)
    inp, buf = run_cfg(cfg)
    kc = {}
    for t in (0, 31, 64, 95):
        check_token(inp, buf, t, key_cache=kc)


@pytest.mark.parametrize("sm_scale", [-1.0 / 16, 0.0])
def test_mla_h128_negative_and_zero_scale(sm_scale):
    # the one-gather 128-head kernel takes its max over scaled logits: a negative scale
    # reverses which rows lead, a zero scale makes every selected row weigh the same
    cfg = I.shrink(I.CONFIGS["decode_b64_paged_h128"], batch=130, ctx_range=(1000, 4000), sm_scale=sm_scale)
    inp, buf = run_cfg(cfg)
    for t in (0, 63, 129):
        check_token(inp, buf, t)


def test_mla_h128_ignores_non_finite_rows_outside_the_selection():
    # NaN / Inf in a block no request references, 130 tokens x 128 heads (one-gather kernel):
    # the masked tail entries of short dense rows read zeros, not that block
    cfg = I.shrink(I.CONFIGS["decode_b64_paged_h128"], batch=130, ctx_range=(5, 3000))
    inp = I.make_inputs(cfg, DEV)
    pool = inp["k_pool"]
    inp["k_pool"] = torch.cat([torch.zeros_like(pool[:1]), pool]).contiguous()
    pools = []
    for pool in inp["kv_pools"]:
        junk = torch.full_like(pool[:1], float("nan"))
        junk[0, ::2] = float("inf")
        pools.append(torch.cat([junk, pool]).contiguous())
    inp["kv_pools"] = pools
    bt = inp["block_table"]
    inp["block_table"] = torch.where(bt >= 0, bt + 1, bt).contiguous()
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    assert torch.isfinite(buf.outs[0].float()).all()
    for t in (0, 5, 64, 77, 129):
        check_token(inp, buf, t)


def test_bf16_decode_edge_lengths():
    # n = 1, n = k, n = k + 1, n a multiple of 64, n = 64k + 1
    lens = [1, 2048, 2049, 4096, 4097, 63, 65, 2047]
    cfg = I.shrink(I.CONFIGS["decode_b64_paged"], batch=len(lens), ctx_range=None)
    inp = I.make_inputs(cfg, DEV)
    # override lengths: block tables are sized for cfg.ctx so any length <= ctx is valid
    set_lengths(inp, seq_len=lens, q_pos=[n - 1 for n in lens])
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    for t in range(len(lens)):
        check_token(inp, buf, t)


def test_bf16_prefill_small_multi_request():
    # a chunk whose tokens cross n = k, plus tokens of a second request in the same chunk
    cfg = I.shrink(I.CONFIGS["prefill_4096_at_128k"], ctx=2100, prefill_tokens=100)
    inp = I.make_inputs(cfg, DEV)
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    kc = {}
    for t in list(range(0, 100, 7)) + [47, 48, 49, 99]:
        check_token(inp, buf, t, key_cache=kc)
    # mixed requests: same pools, two requests with different page tables
    cfg2 = I.shrink(I.CONFIGS["decode_b64_paged"], batch=2, ctx_range=None, ctx=3000)
    inp2 = I.make_inputs(cfg2, DEV)
    T = 24
    set_lengths(inp2, q_row=[i % 2 for i in range(T)],
                q_pos=[2990 - 100 * i if i % 3 else 2000 + i for i in range(T)])
    inp2["q_idx"] = inp2["q_idx"][:1].repeat(T, 1, 1).contiguous()
    inp2["q_idx"] = (inp2["q_idx"] + torch.arange(T, device=DEV).view(T, 1, 1).remainder(3)
                     .to(inp2["q_idx"].dtype) - 1).contiguous()
    inp2["w"] = inp2["w"][:1].repeat(T, 1).contiguous()
    g = torch.Generator(device=DEV).manual_seed(7)
    inp2["q"] = [torch.randn(T, 64, 576, device=DEV, generator=g).to(torch.bfloat16)]
    inp2["cfg"] = I.shrink(cfg2, prefill_tokens=T)
    buf2 = P.run_inputs(inp2)
    torch.cuda.synchronize()
    for t in range(T):
        check_token(inp2, buf2, t)


def test_mla_alternative_scale():
    # the 1/16 = 1/sqrt(256) reading of the softmax scale (GLM-5 SDPA head dim)
    cfg = I.shrink(I.CONFIGS["decode_b64_paged"], batch=3, ctx_range=(1000, 9000), sm_scale=1.0 / 16)
    inp, buf = run_cfg(cfg)
    for t in range(3):
        check_token(inp, buf, t)


def test_mla_running_max_moves_late():
    # rows in the second half of every context are scaled up, so the logits of a split that
    # spans the boundary rise by far more than 32 (log2 units) after its first tiles: the
    # running max moves after O has started to accumulate and the split runs a second pass
    cfg = I.shrink(I.CONFIGS["decode_b64_paged"], batch=4, ctx_range=(3000, 9000))
    inp = I.make_inputs(cfg, DEV)
    lens = inp["seq_len"].tolist()
    bt = inp["block_table"].cpu()
    phys = sorted({int(bt[b, j]) for b, n in enumerate(lens) for j in range((n // 2) // 64 + 1, (n + 63) // 64)})
    sel = torch.tensor(phys, dtype=torch.long, device=DEV)
    for pool in inp["kv_pools"]:
        pool[sel] = (pool[sel].float() * 8).to(pool.dtype)
    inp["q"] = [(q.float() * 4).to(q.dtype) for q in inp["q"]]
    log(f"[gpu] late-max lens {lens}, {len(phys)} scaled pages")
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    for t in range(len(lens)):
        check_token(inp, buf, t)


def test_mla_splits_repeat_bitwise():
    # 40 tokens -> 6 splits per token and a combine: a second call on the same buffers and
    # workspace reproduces the first bit for bit (no state carried between calls)
    cfg = I.shrink(I.CONFIGS["decode_b64_paged"], batch=40, ctx_range=(2500, 9000))
    inp = I.make_inputs(cfg, DEV)
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    first, first_lse = buf.outs[0].clone(), buf.lses[0].clone()
    P.run_inputs(inp, buf, step=1)
    torch.cuda.synchronize()
    assert torch.equal(buf.outs[0], first) and torch.equal(buf.lses[0], first_lse)
    for t in (0, 17, 39):
        check_token(inp, buf, t)


# ------------------------------------------------------------------ top-k in isolation

def _topk_case(scores: np.ndarray, n_valid, k):
    rows, ld = scores.shape
    s = torch.from_numpy(scores.astype(np.float32)).to(DEV)
    nv = torch.tensor(n_valid, dtype=torch.int32, device=DEV)
    idx = torch.empty((rows, k), dtype=torch.int32, device=DEV)
    D.dsa_topk(s, nv, nv.cpu(), k, idx, ws=D.workspace(D.DSA_OP_TOPK, rows, ld, k, 0, 0, DEV))
    torch.cuda.synchronize()
    exp = R.expected_topk(scores.astype(np.float32), np.array(n_valid), k)
    got = idx.cpu().numpy()
    for r in range(rows):
        assert np.array_equal(got[r], exp[r]), f"row {r} n={n_valid[r]} k={k}"


@pytest.mark.parametrize("k", [1, 7, 64, 2048])
def test_topk_adversarial(k):
    rng = np.random.default_rng(k)
    ld = 40000
    rows = []
    nv = []
    rows.append(np.full(ld, 3.0)); nv.append(ld)                                  # all equal
    rows.append(rng.integers(0, 2, ld).astype(np.float64)); nv.append(ld)         # two values
    r = rng.standard_normal(ld); r[rng.integers(0, ld, 500)] = 0.0
    r[rng.integers(0, ld, 500)] = -0.0; nv.append(ld); rows.append(r)             # signed zeros
    rows.append(rng.integers(-3, 4, ld).astype(np.float64)); nv.append(k)        # n = k
    rows.append(rng.integers(-3, 4, ld).astype(np.float64)); nv.append(k + 1)    # n = k + 1
    rows.append(rng.integers(-3, 4, ld).astype(np.float64)); nv.append(max(0, k - 1))
    rows.append(rng.integers(-3, 4, ld).astype(np.float64)); nv.append(0)         # empty
    rows.append(rng.integers(0, 50, ld).astype(np.float64)); nv.append(32768)    # cache edge
    rows.append(rng.integers(0, 50, ld).astype(np.float64)); nv.append(32769)
    rows.append(rng.integers(0, 50, ld).astype(np.float64)); nv.append(8192)     # largest direct row
    rows.append(rng.integers(0, 50, ld).astype(np.float64)); nv.append(8193)     # smallest pruned row
    rows.append(rng.standard_normal(ld)); nv.append(ld)                          # pruned, distinct
    rows.append(-np.abs(rng.standard_normal(ld)) * 1e30); nv.append(ld)          # huge negatives
    rows.append(np.where(np.arange(ld) > ld - k - 3, 5.0, 1.0)); nv.append(ld)   # winners at the end
    _topk_case(np.stack(rows), nv, k)


@pytest.mark.parametrize("rows,ld", [(300, 20000), (300, 40000), (2500, 40000)])
def test_topk_many_rows(rows, ld):
    # relu-weighted sums like indexer scores, ragged lengths across the direct / pruned
    # boundaries; ld <= 32768 selects in one kernel, otherwise 300 rows prune with several
    # workgroups per row (candidate lists in memory) and 2500 with one workgroup per row
    # that prunes and selects (candidate list in LDS)
    rng = np.random.default_rng(rows + ld)
    sc = np.maximum(rng.standard_normal((rows, ld)), 0.0) + 0.5 * np.maximum(rng.standard_normal((rows, ld)), 0.0)
    nv = rng.integers(0, ld + 1, rows)
    nv[:6] = [min(x, ld) for x in (ld, 8192, 8193, 2048, 32768, 32769)]
    _topk_case(sc, nv.tolist(), 2048)


def _sampled_heavy(rng, n, runs):
    """Values in [0, 1) except 10.0 on the first `runs` of the 512 sample runs (4 positions
    each, evenly spaced over the row): the sampled bound lands on 10.0 and lists
    4 * runs candidates, fewer than k = 2048 for runs < 512."""
    row = rng.random(n)
    for i in range(runs):
        p = 4 * ((i * (n // 4)) // 512)
        row[p:p + 4] = 10.0
    return row


def _spread_tens(rng, n, count):
    """Values in [0, 1) except 10.0 at `count` evenly spread positions: about a fifth of
    the samples are 10.0, so the sampled bound lands on 10.0 and lists exactly `count`
    candidates (8192 fills the candidate list, 8193 overflows it)."""
    row = rng.random(n)
    row[(np.arange(count) * n) // count] = 10.0
    return row


def _adversarial_rows(rng, ld, k):
    """Rows that defeat the sampled bound (ties, two values, winners at the end, too few or
    too many candidates) next to ordinary ones."""
    return [
        (_sampled_heavy(rng, ld, 300), ld),                                  # too few listed
        (_spread_tens(rng, ld, 8192), ld),                                   # list just full
        (_spread_tens(rng, ld, 8193), ld),                                   # one over
        (np.full(ld, 3.0), ld),                                               # all equal
        (rng.integers(0, 2, ld).astype(np.float64), ld),                     # two values
        (np.where(np.arange(ld) > ld - k - 3, 5.0, 1.0), ld),                # winners at the end
        (np.where(np.arange(ld) % 7 == 0, 2.0, 1.0), ld),                    # periodic ties
        (rng.standard_normal(ld), ld),                                       # distinct values
        (rng.integers(0, 50, ld).astype(np.float64), ld - 3),                # ragged length
    ]


@pytest.mark.parametrize("ld", [40000, 40001])
def test_topk_listed_rows_adversarial(ld):
    # 2048 rows: one workgroup per row prunes and selects, candidates listed in LDS; most
    # rows short (dense or direct), a few adversarial ones of full length.  ld = 40001
    # leaves the rows unaligned (scalar loads)
    rng = np.random.default_rng(ld)
    rows = 2048
    sc = rng.integers(0, 100, (rows, ld)).astype(np.float32)
    nv = rng.integers(0, 9000, rows)
    for i, (r, n) in enumerate(_adversarial_rows(rng, ld, 2048)):
        sc[100 * i + 7] = r
        nv[100 * i + 7] = n
    _topk_case(sc, nv.tolist(), 2048)


def test_topk_row_pass_block_edges():
    # 2048 rows (one workgroup per row streams it in 8192-position blocks): lengths at the
    # block edges -- one position into a block, whole blocks with no partial end, the 32768
    # edge, a ragged end -- next to short rows (dense, or selected without a bound)
    rng = np.random.default_rng(77)
    ld = 40000
    rows = 2048
    sc = rng.standard_normal((rows, ld)).astype(np.float32)
    sc[1::5] = rng.integers(0, 40, (len(range(1, rows, 5)), ld))   # heavy ties on some rows
    edges = [8193, 8200, 16383, 16384, 16385, 24576, 24577, 32767, 32768, 32769, 39999, 40000,
             2048, 2049, 8192, 0, 1]
    nv = [edges[i % len(edges)] for i in range(rows)]
    _topk_case(sc, nv, 2048)


@pytest.mark.parametrize("ld", [30001, 40001])
def test_topk_unaligned_rows(ld):
    # rows not 16-byte aligned: the one-pass kernel (ld <= 32768) and the prune with several
    # workgroups per row
    rng = np.random.default_rng(ld)
    cases = _adversarial_rows(rng, ld, 64)
    sc = np.stack([r for r, _ in cases] + [rng.integers(0, 1000, ld).astype(np.float64)])
    nv = [n for _, n in cases] + [ld - 1]
    _topk_case(sc, nv, 64)


def test_topk_long_rows_ties():
    rng = np.random.default_rng(5)
    ld = 131072
    sc = np.stack([rng.integers(0, 300, ld).astype(np.float64), np.full(ld, 1.0),
                   rng.integers(0, 4, ld) * 1000.0])
    _topk_case(sc, [ld, ld, 100000], 2048)


def test_topk_prefill_offset():
    # n_add = 1: row r considers q_pos[r] + 1 positions
    rng = np.random.default_rng(9)
    sc = rng.integers(0, 100, (5, 5000)).astype(np.float32)
    q_pos = [0, 99, 2047, 2048, 4999]
    s = torch.from_numpy(sc).to(DEV)
    idx = torch.empty((5, 2048), dtype=torch.int32, device=DEV)
    qp = torch.tensor(q_pos, dtype=torch.int32)
    D.dsa_topk(s, qp.to(DEV), qp, 2048, idx, n_add=1)
    exp = R.expected_topk(sc, np.array(q_pos) + 1, 2048)
    assert np.array_equal(idx.cpu().numpy(), exp)


# ------------------------------------------------------------------ layout and determinism

def test_paged_layout_invariance_and_determinism():
    cfg = I.shrink(I.CONFIGS["decode_b64_paged"], batch=4, ctx_range=(3000, 9000))
    inp = I.make_inputs(cfg, DEV)
    a = P.run_inputs(inp)
    torch.cuda.synchronize()
    snap = [a.scores.clone(), a.idx.clone(), a.outs[0].clone(), a.lses[0].clone()]
    b = P.run_inputs(inp)
    torch.cuda.synchronize()
    lens = inp["seq_len"].tolist()
    for t, n in enumerate(lens):           # run-to-run bit identical (scores past n are unwritten)
        assert torch.equal(snap[0][t, :n], b.scores[t, :n])
    for x, y in zip(snap[1:], [b.idx, b.outs[0], b.lses[0]]):
        assert torch.equal(x, y)
    # same logical rows laid out with an identity page table
    bt = inp["block_table"]
    ident = torch.full_like(bt, -1)
    kp = torch.empty_like(inp["k_pool"])
    kvp = torch.empty_like(inp["kv_pools"][0])
    off = 0
    for r, n in enumerate(lens):
        nb = (n + 63) // 64
        phys = bt[r, :nb].long()
        ident[r, :nb] = torch.arange(off, off + nb, dtype=torch.int32, device=DEV)
        kp[off:off + nb] = inp["k_pool"][phys]
        kvp[off:off + nb] = inp["kv_pools"][0][phys]
        off += nb
    inp2 = dict(inp, block_table=ident, k_pool=kp, kv_pools=[kvp])
    c = P.run_inputs(inp2)
    torch.cuda.synchronize()
    for t, n in enumerate(lens):
        assert torch.equal(c.scores[t, :n], snap[0][t, :n])
    assert torch.equal(c.idx, snap[1])
    assert torch.equal(c.outs[0], snap[2])
    assert torch.equal(c.lses[0], snap[3])


def test_indexshare_reuses_first_layer_selection():
    cfg = I.shrink(I.CONFIGS["indexshare_decode_4layer"], batch=3, ctx=5000, extra_dense=(1500, 700))
    inp, buf = run_cfg(cfg)
    for t in range(5):
        check_token(inp, buf, t)
    # the shared layers' outputs equal a plain decode of that layer with layer 0's idx
    cache = buf.cache
    with pytest.raises(D.DsaError):
        cache.get(step=1, layer_in_group=1)
    with pytest.raises(D.DsaError):
        cache.get(step=0, layer_in_group=4)
    idx = cache.get(0, 2)
    out = torch.empty_like(buf.outs[2])
    lse = torch.empty_like(buf.lses[2])
    ws = D.workspace(D.DSA_OP_MLA, 5, 0, cfg.k, cfg.H, cfg.Dl, DEV)
    D.dsa_sparse_mla_decode(inp["q"][2], inp["kv_pools"][2], P.page_table(inp), idx, cfg.k, cfg.sm_scale,
                            out, lse, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, buf.outs[2]) and torch.equal(lse, buf.lses[2])


def test_empty_prefill_chunk_is_a_noop():
    cfg = I.CONFIGS["decode_b1_32k"]
    z = torch.zeros((0,), dtype=torch.int32, device=DEV)
    zh = torch.zeros((0,), dtype=torch.int32)
    kv = torch.zeros((1, 64, 576), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    sl = torch.ones((1,), dtype=torch.int32, device=DEV)
    q = torch.zeros((0, 64, 576), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((0, 64, 512), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((0, 2048), dtype=torch.int32, device=DEV)
    D.dsa_sparse_mla_prefill(q, kv, D.PageTable(bt, sl, sl.cpu()), D.Chunk(z, z, zh, zh), idx, 2048,
                             cfg.sm_scale, out)


def test_lengths_rejected_before_launch():
    # a length beyond the page table's capacity, a prefill position beyond its request and a
    # top-k row longer than its stride are refused on the host; nothing is enqueued
    inp = I.make_inputs(I.shrink(I.CONFIGS["decode_b64_paged"], batch=2, ctx_range=None, ctx=3000), DEV)
    cap = inp["block_table"].shape[1] * 64
    bad = torch.tensor([3000, cap + 1], dtype=torch.int32)
    pt = D.PageTable(inp["block_table"], bad.to(DEV), bad)
    scores = torch.empty((2, cap), dtype=torch.float32, device=DEV)
    with pytest.raises(D.DsaError, match="seq_len"):
        D.dsa_indexer_scores(inp["q_idx"], inp["w"], inp["k_pool"], pt, scores)
    ch = D.Chunk(torch.zeros(2, dtype=torch.int32, device=DEV), torch.tensor([5, 3000], dtype=torch.int32,
                 device=DEV), torch.zeros(2, dtype=torch.int32), torch.tensor([5, 3000], dtype=torch.int32))
    with pytest.raises(D.DsaError, match="q_pos"):
        D.dsa_indexer_scores(inp["q_idx"], inp["w"], inp["k_pool"], P.page_table(inp), scores, chunk=ch)
    nv = torch.tensor([cap, cap + 1], dtype=torch.int32)
    idx = torch.empty((2, 2048), dtype=torch.int32, device=DEV)
    with pytest.raises(D.DsaError, match="positions"):
        D.dsa_topk(scores, nv.to(DEV), nv, 2048, idx)
    torch.cuda.synchronize()


def test_mla_ignores_non_finite_rows_outside_the_selection():
    # An unused block (physical 0, referenced by no request) full of NaN and Inf.  Rows whose
    # list ends mid-tile (dense rows of ragged length, split tails) must not pick it up: the
    # masked entries of a tile contribute nothing, not 0 * NaN.
    cfg = I.shrink(I.CONFIGS["decode_b64_paged"], batch=6, ctx_range=(5, 3000))
    inp = I.make_inputs(cfg, DEV)
    for name in ("k_pool",):
        pool = inp[name]
        inp[name] = torch.cat([torch.zeros_like(pool[:1]), pool]).contiguous()
    pools = []
    for pool in inp["kv_pools"]:
        junk = torch.full_like(pool[:1], float("nan"))
        junk[0, ::2] = float("inf")
        pools.append(torch.cat([junk, pool]).contiguous())
    inp["kv_pools"] = pools
    bt = inp["block_table"]
    inp["block_table"] = torch.where(bt >= 0, bt + 1, bt).contiguous()
    lens = inp["seq_len"].tolist()
    log(f"[gpu] non-finite unused block, lens {lens}")
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    assert torch.isfinite(buf.outs[0].float()).all()
    for t in range(len(lens)):
        check_token(inp, buf, t)


# ------------------------------------------------------------------ seeded shape sweep

def _sweep_shape(seed):
    """One seeded draw of the path's shape parameters: k (1, values off the 32-row tile,
    2048), 64 or 128 MLA heads, one or two layers of an IndexShare group, random pages."""
    rng = np.random.default_rng(7000 + seed)
    return dict(k=int(rng.choice([1, 17, 64, 100, 333, 2048])), H=int(rng.choice([64, 128])),
                layers=int(rng.choice([1, 2])), hi=int(rng.choice([300, 2500, 7000])),
                batch=int(rng.integers(1, 10)), T=int(rng.integers(1, 200)))


@pytest.mark.parametrize("seed", range(12))
def test_sweep_decode_shapes(seed):
    """Decode through the whole path on a seeded draw of shapes (lengths from 1, so rows on
    both sides of k): every token's scores, selection and outputs against the oracle."""
    sh = _sweep_shape(seed)
    cfg = I.shrink(I.CONFIGS["decode_b64_paged"], seed=300 + seed, batch=sh["batch"], ctx_range=(1, sh["hi"]),
                   H=sh["H"], k=sh["k"], layers=sh["layers"])
    inp = I.make_inputs(cfg, DEV)
    lens = inp["seq_len"].tolist()
    log(f"[gpu] sweep decode {sh} lens {lens}")
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    for t in range(len(lens)):
        check_token(inp, buf, t)


@pytest.mark.parametrize("seed", range(8))
def test_sweep_prefill_shapes(seed):
    """A causal prefill chunk of a seeded length at the end of a seeded context, shapes as
    for the decode sweep; spread tokens against the oracle."""
    sh = _sweep_shape(100 + seed)
    ctx = max(sh["T"], sh["hi"])
    cfg = I.shrink(I.CONFIGS["prefill_4096_at_128k"], seed=400 + seed, ctx=ctx, prefill_tokens=sh["T"], H=sh["H"],
                   k=sh["k"], layers=sh["layers"], identity_pages=False)
    inp = I.make_inputs(cfg, DEV)
    log(f"[gpu] sweep prefill {sh} ctx {ctx}")
    buf = P.run_inputs(inp)
    torch.cuda.synchronize()
    T = sh["T"]
    for t in sorted({0, T - 1} | set(np.linspace(0, T - 1, min(T, 12)).round().astype(int).tolist())):
        check_token(inp, buf, t)


# ------------------------------------------------------------------ full-size workloads

def test_full_decode_b1_32k():
    inp, buf = run_cfg(I.CONFIGS["decode_b1_32k"])
    check_token(inp, buf, 0)


def test_full_decode_b64_paged_every_token():
    inp, buf = run_cfg(I.CONFIGS["decode_b64_paged"])
    lens = inp["seq_len"].tolist()
    for t in range(len(lens)):
        log(f"[gpu] decode_b64 token {t} n={lens[t]}")
        check_token(inp, buf, t)


def test_full_decode_b64_paged_h128_every_token():
    # 128 MLA heads at full size: 64 tokens, one workgroup per (token, split) for all heads,
    # 4 splits
    inp, buf = run_cfg(I.CONFIGS["decode_b64_paged_h128"])
    lens = inp["seq_len"].tolist()
    for t in range(len(lens)):
        log(f"[gpu] decode_b64_h128 token {t} n={lens[t]}")
        check_token(inp, buf, t)


def test_full_indexshare_every_token():
    inp, buf = run_cfg(I.CONFIGS["indexshare_decode_4layer"])
    for t in range(inp["q_idx"].shape[0]):
        log(f"[gpu] indexshare token {t} n={int(inp['seq_len_host'][t])}")
        check_token(inp, buf, t)


def prefill_tokens_checked(T):
    """64 tokens of a T-token chunk: the first two, the last two, both sides of the
    midpoint and evenly spaced others."""
    fixed = {0, 1, T // 2 - 1, T // 2, T - 2, T - 1}
    spread = set(np.linspace(0, T - 1, 64 - len(fixed) + 2).round().astype(int).tolist())
    pick = sorted(fixed | spread)
    return pick[:64] if len(pick) >= 64 else pick


def test_full_prefill_h128_spread():
    inp, buf = run_cfg(I.CONFIGS["prefill_4096_at_128k_h128"])
    kc = {}
    for t in prefill_tokens_checked(inp["q_idx"].shape[0]):
        log(f"[gpu] prefill h128 token {t}")
        check_token(inp, buf, t, key_cache=kc)


def test_full_prefill_spread():
    inp, buf = run_cfg(I.CONFIGS["prefill_4096_at_128k"])
    kc = {}
    for t in prefill_tokens_checked(inp["q_idx"].shape[0]):
        log(f"[gpu] prefill token {t}")
        check_token(inp, buf, t, key_cache=kc)
