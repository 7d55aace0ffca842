"""The figures the pages print, against the byte and FLOP accounting that bench.py uses
for its roofline (tests/golden/pages_figures.txt holds them with their sources)."""
import math
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import dsa_inputs as I  # noqa: E402


def _figures():
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", "pages_figures.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.rsplit("=", 1)
            parts = lhs.split()
            out[parts[0]] = (dict(p.split("=") for p in parts[1:]), float(rhs))
    return out


FIG = _figures()


def test_mla_arithmetic_intensity():
    params, expected = FIG["mla_flop_per_byte"]
    cfg = I.CONFIGS["decode_b1_32k"]
    assert (cfg.H, cfg.Dl, cfg.row_dim - cfg.Dl, cfg.dtype.itemsize) == \
        tuple(int(params[x]) for x in ("H", "d", "r", "b"))
    alg, _ = bench.algorithmic(cfg)
    flops = alg["mla_bf16_kernel"][1]
    rows = min(32768, cfg.k)           # one token, k selected rows
    per_row_flop = flops / rows
    per_row_bytes = cfg.row_dim * cfg.dtype.itemsize
    intensity = per_row_flop / per_row_bytes
    assert math.floor(intensity * 10) / 10 == pytest.approx(expected)


def test_indexshare_indexer_cut():
    params, expected = FIG["indexshare_indexer_cut"]
    cfg = I.CONFIGS["indexshare_decode_4layer"]
    assert cfg.layers == int(params["group"])
    _, shared = bench.algorithmic(cfg)                       # one indexer per 4 layers
    _, single = bench.algorithmic(I.shrink(cfg, layers=1))   # one layer, its own indexer
    # attention work grows with the layers, the indexer's does not
    assert shared["mla"] == pytest.approx(cfg.layers * single["mla"])
    cut = 1.0 - shared["indexer"] / (cfg.layers * single["indexer"])
    assert cut == pytest.approx(expected)


def test_mla_mode_ratios():
    params, expected = FIG["mha_memory_ratio"]
    H, dn, dr, dv, d = (int(params[x]) for x in ("H", "dn", "dr", "dv", "d"))
    r = bench.mla_mode_ratios(H=H, dl=d, dr=dr, dn=dn, dv=dv)
    assert math.floor(r["memory_ratio_rope_per_head"]) == expected
    params, expected = FIG["mqa_flop_ratio_max"]
    r = bench.mla_mode_ratios(dn=int(params["dn"]), dr=int(params["dr"]), dv=int(params["dv"]), dl=int(params["d"]))
    assert round(r["flop_ratio"], 1) == pytest.approx(expected)


def test_roofline_accounting_closed_forms():
    """bench.algorithmic() against the per-unit figures written out from the workloads'
    definitions: 2*Hi*Di FLOP and 2*Di bytes of key per (token, visible position) for the
    indexer; one (Dl + Dr)-wide bf16 row and 2*H*(2*Dl + Dr) FLOP per selected row for the
    MQA-mode MLA (SemiAnalysis, "Inside GLM-5.3", lightning indexer and MLA sections)."""
    pre = I.CONFIGS["prefill_4096_at_128k"]
    alg, _ = bench.algorithmic(pre)
    first = pre.ctx - pre.prefill_tokens            # 126976: the chunk's first position
    pairs = sum(p + 1 for p in range(first, pre.ctx))
    assert pairs == 528_484_352
    assert alg["indexer_prefill_kernel"][1] == 2 * 64 * 128 * pairs            # 8.659 TFLOP
    assert alg["mla_bf16_kernel"][1] == 4096 * 2048 * 2 * 64 * (2 * 512 + 64)   # 1.168 TFLOP
    assert alg["indexer_prefill_kernel"][2] == "mfma" and alg["mla_bf16_kernel"][2] == "mfma"

    dec = I.CONFIGS["indexshare_decode_4layer"]
    alg, step = bench.algorithmic(dec)
    n = [131072] * 32 + [1500] * 8
    keys = sum(n) * 128 * 2
    scores = sum(n) * 4
    q_w = 40 * (64 * 128 * 2 + 64 * 4)
    assert alg["indexer_decode_kernel"][0] == keys + scores + q_w              # 1094.3 MB
    sel = 32 * 2048 + 8 * 1500                                                 # dense rows keep all n
    rows = sel * 576 * 2
    assert rows == 32 * 2_359_296 + 8 * 1500 * 1152                            # 2.36 MB per token
    q = 40 * 64 * 576 * 2
    out = 40 * 64 * (512 * 2 + 4)
    assert alg["mla_bf16_kernel"][0] == rows + q + 40 * 2048 * 4 + out
    assert alg["mla_bf16_kernel"][1] == sel * 2 * 64 * (2 * 512 + 64)
    assert alg["mla_bf16_kernel"][2] == "hbm"
    # one indexer and one top-k per step, four layers of attention
    assert step["indexer"] == alg["indexer_decode_kernel"][0]
    assert step["mla"] == 4 * (rows + q + 40 * 2048 * 4 + out)
