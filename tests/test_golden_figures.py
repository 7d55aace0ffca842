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
