"""dsa_sparse_mla_decode_noalloc (split partials in the library's own device array) against
dsa_sparse_mla_decode (caller workspace), through the C ABI: bit-identical outputs and lse
on two calls in a row, the second with a smaller batch, and against the oracle."""
import numpy as np
import pytest
import torch

import dsa_inputs as I
from oracle import run as R

pytestmark = pytest.mark.gpu

import sparse_attention_19_amd as D  # noqa: E402
from sparse_attention_19_amd import pipeline as P  # noqa: E402

DEV = "cuda"


def _case(cfg):
    print(f"[gpu] no-alloc case {cfg.name} batch {cfg.batch} H {cfg.H}", flush=True)
    inp = I.make_inputs(cfg, DEV)
    pt = P.page_table(inp)
    T = inp["q_idx"].shape[0]
    buf = P.run_inputs(inp, pt=pt)              # indexer, top-k, MLA with a caller workspace
    torch.cuda.synchronize()
    out = torch.full_like(buf.outs[0], float("nan"))
    lse = torch.full_like(buf.lses[0], float("nan"))
    D.dsa_sparse_mla_decode_noalloc(inp["q"][0], inp["kv_pools"][0], pt, buf.idx, cfg.k, cfg.sm_scale, out, lse)
    torch.cuda.synchronize()
    return inp, buf, out, lse, T


def test_noalloc_matches_workspace_entry_point_twice():
    big = I.shrink(I.CONFIGS["decode_b64_paged"], batch=40, ctx_range=(1000, 9000))   # 6 splits per token
    small = I.shrink(I.CONFIGS["decode_b64_paged"], seed=12, batch=3, ctx_range=(1500, 7000))   # 32 splits
    for cfg in (big, small):
        inp, buf, out, lse, T = _case(cfg)
        assert torch.equal(out, buf.outs[0]), cfg.batch
        assert torch.equal(lse, buf.lses[0]), cfg.batch
        for t in (0, T - 1):
            exp = R.expected_token(inp, t, layers=[0])
            got = R.to_f64(out[t])
            err = float((np.abs(got - exp["out"][0]).max(1) / np.abs(exp["out"][0]).max(1)).max())
            assert err <= 2e-2, (cfg.batch, t, err)


def test_noalloc_h128():
    # 5 tokens: two 64-head workgroups per (token, split); 64 tokens: one workgroup per
    # (token, split) for all 128 heads, 4 splits (the largest partials the array holds)
    for batch in (5, 64):
        cfg = I.shrink(I.CONFIGS["decode_b64_paged_h128"], batch=batch, ctx_range=(1000, 6000))
        inp, buf, out, lse, T = _case(cfg)
        assert torch.equal(out, buf.outs[0]) and torch.equal(lse, buf.lses[0]), batch
