"""Seeded input generators: shapes, value ranges, determinism and page-table structure."""
import torch

import dsa_inputs as I


def test_configs_present():
    assert set(I.CONFIGS) == {"tiny_fp32", "decode_b1_32k", "decode_b64_paged",
                              "prefill_4096_at_128k", "indexshare_decode_4layer",
                              "decode_b64_paged_h128", "prefill_4096_at_128k_h128"}
    h = I.CONFIGS["decode_b64_paged_h128"]
    assert (h.H, h.Dl, h.Dr, h.Hi, h.Di, h.k) == (128, 512, 64, 64, 128, 2048)
    assert I.context_lengths(h)[0] >= 4096 and len(I.context_lengths(h)) == 64
    c = I.CONFIGS["decode_b64_paged"]
    lens = I.context_lengths(c)
    assert len(lens) == 64 and min(lens) >= 4096 and max(lens) <= 65536
    c5 = I.CONFIGS["indexshare_decode_4layer"]
    assert I.context_lengths(c5) == [131072] * 32 + [1500] * 8


def test_tiny_inputs_shape_range_determinism():
    c = I.CONFIGS["tiny_fp32"]
    a = I.make_inputs(c)
    b = I.make_inputs(c)
    for key in ("k_pool", "q_idx", "w"):
        assert torch.equal(a[key], b[key])
    assert torch.equal(a["kv_pools"][0], b["kv_pools"][0])
    assert a["k_pool"].shape == (4, 64, 32) and a["q_idx"].shape == (1, 4, 32)
    assert a["kv_pools"][0].shape == (4, 64, 80) and a["q"][0].shape == (1, 8, 80)
    assert a["k_pool"].abs().max() <= 3 and a["w"].min() >= 0 and a["w"].max() <= 2
    assert torch.equal(a["k_pool"], a["k_pool"].round())
    assert a["block_table"].tolist() == [[0, 1, 2, 3]]
    assert a["q_pos"].tolist() == [255]


def test_paged_table_is_a_permutation():
    c = I.shrink(I.CONFIGS["decode_b64_paged"], batch=5, ctx_range=(100, 700))
    lens = I.context_lengths(c)
    bt, total = I.page_table(c, lens)
    used = [int(x) for row, n in zip(bt.tolist(), lens) for x in row[:(n + 63) // 64]]
    assert sorted(used) == list(range(total))
    assert used != list(range(total))            # actually permuted


def test_prefill_positions():
    c = I.shrink(I.CONFIGS["prefill_4096_at_128k"], ctx=1000, prefill_tokens=64,
                 Hi=4, Di=32, H=8, Dl=64, Dr=16, k=64)
    a = I.make_inputs(c)
    assert a["q_pos"].tolist() == list(range(936, 1000))
    assert a["q_row"].tolist() == [0] * 64
