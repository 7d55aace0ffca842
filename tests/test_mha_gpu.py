"""MLA's MHA mode and the switch between the two modes, through the C ABI, against the
oracle (dsa_oracle.mla_mha over each token's selection).

Bars as for the other attention outputs: normwise 2e-2 per (token, head) row for the bf16
outputs, lse within 2e-3.  The oracle up-projects the selected rows per head in float64, so
every token is checked on two heads and a few tokens on all heads."""
import dataclasses

import numpy as np
import pytest
import torch

import dsa_inputs as I
from oracle import run as R

pytestmark = pytest.mark.gpu

import sparse_attention_19_amd as D  # noqa: E402
from sparse_attention_19_amd import pipeline as P  # noqa: E402

DEV = "cuda"


def log(msg):
    print(msg, flush=True)


def rel_rows(got, ref):
    return float((np.abs(got - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)).max())


def mha_inputs(ctx, T, H=64, batch=1, seed=21):
    """A prefill chunk of T tokens at the end of a ctx-position context (random pages); with
    batch 2 the chunk's 128-token tiles alternate between the two requests."""
    base = I.shrink(I.CONFIGS["decode_b64_paged"], seed=seed, batch=batch, ctx_range=None, ctx=ctx, H=H, mha=True,
                    sm_scale=1.0 / 16, prefill_tokens=T)
    inp = I.make_inputs(base, DEV)
    rows = [(t // 128) % batch for t in range(T)]
    pos = [ctx - T + t for t in range(T)]
    for name, v in (("q_row", rows), ("q_pos", pos)):
        host = torch.tensor(v, dtype=torch.int32)
        inp[name + "_host"] = host
        inp[name] = host.to(DEV)
    return inp


def select(inp):
    """Indexer scores and top-k of the chunk through the library (the path's own selection)."""
    cfg = inp["cfg"]
    T = inp["q_idx"].shape[0]
    ld = inp["block_table"].shape[1] * 64
    pt, ch = P.page_table(inp), P.chunk(inp)
    scores = torch.empty((T, ld), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=DEV)
    D.dsa_indexer_scores(inp["q_idx"], inp["w"], inp["k_pool"], pt, scores, chunk=ch)
    D.dsa_topk(scores, ch.q_pos, ch.q_pos_host, cfg.k, idx, n_add=1, ws=D.workspace(D.DSA_OP_TOPK, T, ld, cfg.k, 0, 0, DEV))
    return pt, ch, idx


def up_projected(inp):
    pool = inp["kv_pools"][0]
    H = inp["cfg"].H
    kv_mha = torch.empty((pool.shape[0] * 64, H, 320), dtype=torch.bfloat16, device=DEV)
    D.dsa_mla_up_project(pool, inp["w_kv"], kv_mha)
    return kv_mha


def check(inp, out, lse, tokens, heads, idx=None):
    for t in tokens:
        exp = R.expected_token_mha(inp, t, heads)
        if idx is not None:
            assert np.array_equal(idx[t].cpu().numpy(), exp["idx"]), f"token {t}: selection differs"
        got = R.to_f64(out[t][heads])
        e = rel_rows(got, exp["out"])
        assert e <= 2e-2, f"token {t}: rel err {e:.3g}"
        d = np.abs(lse[t][heads].cpu().double().numpy() - exp["lse"]).max()
        assert d <= 2e-3, f"token {t}: lse diff {d:.3g}"


def poison_page_tails(inp, value=float("nan")):
    """Fill the unused slots of each request's last page (positions >= its length) of the
    latent pool with a non-finite value: a cache leaves them unwritten."""
    pool = inp["kv_pools"][0]
    for b, n in enumerate(inp["seq_len_host"].tolist()):
        if n % 64:
            phys = int(inp["block_table"][b, n // 64])
            pool[phys, n % 64:] = value


def test_mha_mode_against_oracle():
    # tokens on both sides of k (dense up to position 2047), three 128-token tiles, the last
    # one partial; NaN in the unused tail of the request's last page
    inp = mha_inputs(ctx=2400, T=330)
    poison_page_tails(inp)
    T, H = 330, 64
    pt, ch, idx = select(inp)
    kv_mha = up_projected(inp)
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = D.workspace(D.DSA_OP_MLA_MHA, T, 2400, 2048, H, 512, DEV)
    D.dsa_sparse_mla_prefill_mha(inp["q_mha"], inp["kv_pools"][0], kv_mha, pt, ch, idx, 2048, 1.0 / 16, out, lse, ws=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    log("[gpu] MHA mode: every token on heads 0 and 63")
    check(inp, out, lse, range(T), [0, 63], idx)
    log("[gpu] MHA mode: all heads of a few tokens")
    check(inp, out, lse, [0, 127, 128, 329], list(range(H)))


def test_mha_mode_two_requests_and_small_heads():
    # 128-token tiles of two requests with different page tables; 8 heads
    inp = mha_inputs(ctx=3100, T=256, H=8, batch=2, seed=22)
    T, H = 256, 8
    pt, ch, idx = select(inp)
    kv_mha = up_projected(inp)
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = D.workspace(D.DSA_OP_MLA_MHA, T, 3100, 2048, H, 512, DEV)
    D.dsa_sparse_mla_prefill_mha(inp["q_mha"], inp["kv_pools"][0], kv_mha, pt, ch, idx, 2048, 1.0 / 16, out, lse, ws=ws)
    torch.cuda.synchronize()
    check(inp, out, lse, range(0, T, 5), list(range(H)), idx)


def test_mha_mode_odd_head_count():
    """Five heads: the grid pads the head count to a multiple of 8 (one head per XCD in
    turn), and the padding workgroups have nothing to do; a ragged 200-token chunk."""
    inp = mha_inputs(ctx=2600, T=200, H=5, seed=29)
    T, H = 200, 5
    pt, ch, idx = select(inp)
    kv_mha = up_projected(inp)
    out = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = D.workspace(D.DSA_OP_MLA_MHA, T, 2600, 2048, H, 512, DEV)
    D.dsa_sparse_mla_prefill_mha(inp["q_mha"], inp["kv_pools"][0], kv_mha, pt, ch, idx, 2048, 1.0 / 16, out, lse,
                                 ws=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    log("[gpu] MHA mode, 5 heads")
    check(inp, out, lse, range(0, T, 7), list(range(H)), idx)


@pytest.mark.parametrize("sm_scale", [-1.0 / 16, 0.0])
def test_mha_mode_negative_and_zero_scale(sm_scale):
    """The kernel runs a negative scale as a positive one on -Q, and a zero scale as the
    smallest normal one (every valid p = 1: the mean of the selected values, lse = log |S|)."""
    inp = mha_inputs(ctx=2300, T=140, H=8, seed=28)
    T, H = 140, 8
    inp["cfg"] = dataclasses.replace(inp["cfg"], sm_scale=sm_scale)
    pt, ch, idx = select(inp)
    kv_mha = up_projected(inp)
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = D.workspace(D.DSA_OP_MLA_MHA, T, 2300, 2048, H, 512, DEV)
    D.dsa_sparse_mla_prefill_mha(inp["q_mha"], inp["kv_pools"][0], kv_mha, pt, ch, idx, 2048, sm_scale, out, lse,
                                 ws=ws)
    torch.cuda.synchronize()
    log(f"[gpu] MHA mode, sm_scale {sm_scale}")
    check(inp, out, lse, range(0, T, 3), list(range(H)), idx)


def test_switch_runs_either_mode_to_the_same_result():
    inp = mha_inputs(ctx=2600, T=256, seed=23)
    T, H = 256, 64
    pt, ch, idx = select(inp)
    kv_mha = up_projected(inp)
    ws = D.workspace(D.DSA_OP_MLA_HEADS, T, 2600, 2048, H, 512, DEV)
    outs = {}
    for thr, want in ((2600, 1), (2599, 0), (0, 0)):
        out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
        mode = D.dsa_mla_prefill_heads(inp["q_mha"], inp["w_uk"], inp["w_kv"], inp["kv_pools"][0], kv_mha, pt, ch,
                                       idx, 2048, 1.0 / 16, thr, out, lse, ws=ws)
        torch.cuda.synchronize()
        assert mode == want, (thr, mode)
        outs[thr] = (out, lse)
        log(f"[gpu] switch at {thr}: mode {mode}")
        check(inp, out, lse, [0, 100, 255], list(range(0, H, 9)))
    # MQA mode without an MHA cache
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    assert D.dsa_mla_prefill_heads(inp["q_mha"], inp["w_uk"], inp["w_kv"], inp["kv_pools"][0], None, pt, ch, idx,
                                   2048, 1.0 / 16, 1 << 20, out, ws=ws) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, outs[0][0])
    # the two modes agree with each other to the same bar
    a, b = R.to_f64(outs[2600][0].reshape(-1, 128)), R.to_f64(outs[0][0].reshape(-1, 128))
    assert rel_rows(a, b) <= 2e-2


def test_projections_against_float64():
    g = torch.Generator(device=DEV).manual_seed(5)
    T, H = 37, 64
    q_mha = torch.randn((T, H, 256), generator=g, device=DEV).to(torch.bfloat16)
    w_uk = (torch.randn((H, 512, 192), generator=g, device=DEV) / 512 ** 0.5).to(torch.bfloat16)
    w_uv = (torch.randn((H, 512, 128), generator=g, device=DEV) / 512 ** 0.5).to(torch.bfloat16)
    w_kv = torch.cat([w_uk.transpose(1, 2), w_uv.transpose(1, 2)], dim=1).contiguous()
    q_abs = torch.empty((T, H, 576), dtype=torch.bfloat16, device=DEV)
    D.dsa_mla_absorb_q(q_mha, w_uk, q_abs)
    o_lat = torch.randn((T, H, 512), generator=g, device=DEV).to(torch.bfloat16)
    o = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    D.dsa_mla_unabsorb_o(o_lat, w_kv, o)
    pool = torch.randn((3, 64, 576), generator=g, device=DEV).to(torch.bfloat16)
    kv_mha = torch.empty((192, H, 320), dtype=torch.bfloat16, device=DEV)
    D.dsa_mla_up_project(pool, w_kv, kv_mha)
    torch.cuda.synchronize()
    f = lambda x: R.to_f64(x)  # noqa: E731
    wuk, wuv, qm, ol, lat = f(w_uk), f(w_uv), f(q_mha), f(o_lat), f(pool).reshape(192, 576)
    want_abs = np.concatenate([np.einsum("hcj,thj->thc", wuk, qm[:, :, :192]), qm[:, :, 192:]], axis=2)
    assert rel_rows(f(q_abs).reshape(-1, 576), want_abs.reshape(-1, 576)) <= 1e-2
    assert torch.equal(q_abs[:, :, 512:], q_mha[:, :, 192:])          # the rope dims are copied
    want_o = np.einsum("thc,hcv->thv", ol, wuv)
    assert rel_rows(f(o).reshape(-1, 128), want_o.reshape(-1, 128)) <= 1e-2
    want_kv = np.concatenate([np.einsum("rc,hcj->rhj", lat[:, :512], wuk), np.einsum("rc,hcv->rhv", lat[:, :512], wuv)],
                             axis=2)
    assert rel_rows(f(kv_mha).reshape(-1, 320), want_kv.reshape(-1, 320)) <= 1e-2


def test_128_heads_both_modes():
    """DeepSeek-V3.2's 128 heads: MHA mode and MQA mode (two 64-head groups of the sparse
    MLA between the projections) against the oracle, and against each other."""
    inp = mha_inputs(ctx=2300, T=200, H=128, seed=24)
    T, H = 200, 128
    pt, ch, idx = select(inp)
    kv_mha = up_projected(inp)
    ws = D.workspace(D.DSA_OP_MLA_HEADS, T, 2300, 2048, H, 512, DEV)
    outs = {}
    for thr, want in ((1 << 20, 1), (0, 0)):
        out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
        mode = D.dsa_mla_prefill_heads(inp["q_mha"], inp["w_uk"], inp["w_kv"], inp["kv_pools"][0], kv_mha, pt, ch,
                                       idx, 2048, 1.0 / 16, thr, out, lse, ws=ws)
        torch.cuda.synchronize()
        assert mode == want
        log(f"[gpu] 128 heads, mode {mode}")
        check(inp, out, lse, [0, 63, 64, 127, 128, 199], [0, 1, 63, 64, 65, 127], idx)
        outs[mode] = out
    a, b = R.to_f64(outs[1].reshape(-1, 128)), R.to_f64(outs[0].reshape(-1, 128))
    assert rel_rows(a, b) <= 2e-2


def test_mha_mode_at_its_longest_context():
    """The longest context MHA mode takes (65536 positions, 1024 mask words per token): a
    128-token tile at the end of it, checked on a few tokens and heads."""
    inp = mha_inputs(ctx=65536, T=128, seed=25)
    T, H = 128, 64
    pt, ch, idx = select(inp)
    kv_mha = up_projected(inp)
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = D.workspace(D.DSA_OP_MLA_MHA, T, 65536, 2048, H, 512, DEV)
    D.dsa_sparse_mla_prefill_mha(inp["q_mha"], inp["kv_pools"][0], kv_mha, pt, ch, idx, 2048, 1.0 / 16, out, lse, ws=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    log("[gpu] MHA mode at 65536 positions")
    check(inp, out, lse, [0, 77, 127], [0, 31, 63], idx)


def test_mha_mode_reference_max_moves_late():
    """Latent rows of the context's second half scaled up 12x: a token's logits there (about
    60, log2 units) pass the reference max its first tile sets (about 5) by more than 32, so
    the kernel runs its second pass from each row's final max.  The up-projections are
    selection matrices (each NoPE key and value dim copies one latent dim), so the bf16
    per-head cache holds exactly the keys and values the oracle forms in float64: with logits
    this large, a rounded key would move p by several percent and the comparison would test
    the cache's rounding instead of the kernel."""
    inp = mha_inputs(ctx=3000, T=256, seed=26)
    T, H, ctx = 256, 64, 3000
    g = torch.Generator().manual_seed(27)
    wuk = torch.zeros((H, 512, 192))
    wuv = torch.zeros((H, 512, 128))
    for h in range(H):
        d = torch.randperm(512, generator=g)
        wuk[h, d[:192], torch.arange(192)] = 1.0
        wuv[h, d[192:320], torch.arange(128)] = 1.0
    inp["w_uk"] = wuk.to(torch.bfloat16).to(DEV)
    inp["w_uv"] = wuv.to(torch.bfloat16).to(DEV)
    inp["w_kv"] = torch.cat([inp["w_uk"].transpose(1, 2), inp["w_uv"].transpose(1, 2)], dim=1).contiguous()
    pool = inp["kv_pools"][0]
    bt = inp["block_table"].cpu()
    pages = sorted({int(bt[0, j]) for j in range((ctx // 2) // 64 + 1, (ctx + 63) // 64)})
    sel = torch.tensor(pages, dtype=torch.long, device=DEV)
    pool[sel] = (pool[sel].float() * 12).to(pool.dtype)
    pt, ch, idx = select(inp)
    # the case is real: token 0, head 0 (float64, from the inputs, over the oracle's
    # selection) -- its largest logit over the scaled pages against its largest over the
    # unscaled first half, which bounds the reference max its first tiles set
    lat = R.to_f64(pool).reshape(-1, 576)
    pos = np.asarray(R.expected_token_mha(inp, 0, [0])["idx"])
    rows = [int(bt[0, s // 64]) * 64 + s % 64 for s in pos.tolist()]
    k_nope = lat[rows, :512] @ R.to_f64(inp["w_uk"][0])
    q0 = R.to_f64(inp["q_mha"][0, 0])
    lg = (k_nope @ q0[:192] + lat[rows, 512:] @ q0[192:]) / 16 * np.log2(np.e)
    assert lg[pos >= (ctx // 2 // 64 + 1) * 64].max() > lg[pos < ctx // 2].max() + 32
    kv_mha = up_projected(inp)
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = D.workspace(D.DSA_OP_MLA_MHA, T, ctx, 2048, H, 512, DEV)
    D.dsa_sparse_mla_prefill_mha(inp["q_mha"], pool, kv_mha, pt, ch, idx, 2048, 1.0 / 16, out, lse, ws=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    log(f"[gpu] MHA mode, late max: {len(pages)} scaled pages")
    check(inp, out, lse, range(0, T, 3), [0, 17, 63], idx)
    check(inp, out, lse, [0, 129, 255], list(range(H)))
