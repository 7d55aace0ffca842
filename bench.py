#!/usr/bin/env python3
"""Benchmark of the DSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode_b1_32k]

A step is one pass of the whole path (lightning indexer -> top-k -> sparse MLA, plus the
IndexShare reuse when the workload has a layer group) over one batch of synthetic
inputs already resident in HBM.  Consecutive steps rotate over several independent
copies of the inputs whose total size exceeds the 256 MB Infinity Cache, so every step
streams its key cache and latent rows from HBM as a multi-layer model would.

Prints one JSON line: tokens/s, the step's algorithmic HBM bandwidth, the roofline of
the dominant kernel (its launches timed with HIP events recorded on the kernel's own
stream by the library, dsa_timing_start/collect) and the CPU oracle timed on a bounded
sample of the same workload.

Two helper modes turn rocprofv3 output into the text summaries kept under profiles/:
    --copy-calibration MIB      only copies MIB MiB device-to-device (--steps times),
                                the reference for scaling FETCH_SIZE / WRITE_SIZE
    --summarize-trace DIR       per-kernel table of a --kernel-trace --stats run
    --summarize-traffic ...     HBM bytes per dispatch of one kernel from --pmc runs
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sqlite3
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "sparse_attention_19_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, 2.5 PFLOP/s
MALL_BYTES = 256 << 20
METRIC = "DSA decode tokens/s at 32K–128K ctx + achieved HBM GB/s fraction"

# kernel -> source file that defines it (its hash decides whether stored counters still apply)
KERNEL_SRC = {
    "indexer_decode_kernel": "indexer.hip", "indexer_prefill_kernel": "indexer.hip",
    "indexer_f32_kernel": "indexer.hip", "topk_prune_kernel": "topk.hip", "topk_select_kernel": "topk.hip",
    "topk_onepass_kernel": "topk.hip",
    "mla_bf16_kernel": "mla.hip", "mla_combine_kernel": "mla.hip", "mla_f32_kernel": "mla.hip",
}


def kernel_source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in (KERNEL_SRC[kernel], "common.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def workload_sizes(cfg):
    """Token-level sizes of a workload: (T, per-token visible n, unique keys read)."""
    import dsa_inputs as I
    lens = I.context_lengths(cfg)
    if cfg.prefill_tokens:
        T = cfg.prefill_tokens
        n_tok = [cfg.ctx - T + i + 1 for i in range(T)]
        uniq = cfg.ctx
    else:
        T = len(lens)
        n_tok = list(lens)
        uniq = sum(lens)
    return T, n_tok, uniq


def algorithmic(cfg, kernels_seen=()):
    """Algorithmic bytes (each input read once, each output written once) and FLOPs per
    launch of each kernel, and the bound that applies to it.

    indexer  keys 2*Di B per cached position (once), q_idx + w per token, fp32 score per
             visible (token, position) pair; 2*Hi*Di FLOP per pair
    top-k    the fp32 scores read (by the prune kernel when it runs), k int32 indices
             written per token (by the select kernel); both by the one-pass kernel
    MLA      2*(Dl+Dr) B per selected row per token (one layer per launch), q, idx, and
             out + lse per token; 2*H*(2*Dl+Dr) FLOP per selected row
    """
    T, n_tok, uniq = workload_sizes(cfg)
    eb = cfg.dtype.itemsize
    n_tot = sum(n_tok)
    sel = sum(min(n, cfg.k) for n in n_tok)
    prefill = bool(cfg.prefill_tokens)
    mfma_ok = eb == 2
    ix_b = uniq * cfg.Di * eb + n_tot * 4 + T * (cfg.Hi * cfg.Di * eb + cfg.Hi * 4)
    ix_f = 2 * n_tot * cfg.Hi * cfg.Di
    tk_in, tk_out = n_tot * 4, T * cfg.k * 4
    mla_in = sel * cfg.row_dim * eb + T * cfg.H * cfg.row_dim * eb + T * cfg.k * 4
    mla_out = T * cfg.H * (cfg.Dl * eb + 4)
    mla_f = 2 * sel * cfg.H * (cfg.row_dim + cfg.Dl)
    prune = "topk_prune_kernel" in kernels_seen
    combine = "mla_combine_kernel" in kernels_seen
    ix_bound = "mfma" if (prefill and mfma_ok) else "hbm"
    mla_bound = "mfma" if (prefill and mfma_ok) else "hbm"
    out = {
        "indexer_decode_kernel": (ix_b, ix_f, "hbm"),
        "indexer_prefill_kernel": (ix_b, ix_f, ix_bound),
        "indexer_f32_kernel": (ix_b, ix_f, "hbm"),
        "topk_prune_kernel": (tk_in, 0, "hbm"),
        "topk_select_kernel": (tk_out + (0 if prune else tk_in), 0, "hbm"),
        "topk_onepass_kernel": (tk_in + tk_out, 0, "hbm"),
        "mla_bf16_kernel": (mla_in + (0 if combine else mla_out), mla_f, mla_bound),
        "mla_combine_kernel": (mla_out, 0, "hbm"),
        "mla_f32_kernel": (mla_in + mla_out, mla_f, "hbm"),
    }
    # a step's HBM bytes: in prefill the tokens' selections overlap, and each latent row
    # is fetched from HBM once (later visits hit the caches), so count unique rows there
    rows_hbm = min(uniq, sel) if prefill else sel
    mla_step = rows_hbm * cfg.row_dim * eb + T * cfg.H * cfg.row_dim * eb + T * cfg.k * 4 + mla_out
    step = {"indexer": ix_b, "topk": tk_in + tk_out, "mla": cfg.layers * mla_step}
    return out, step


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed --pmc summary, if the kernel is unchanged."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("JSON "):
                rec = json.loads(line[5:])
                if rec.get("source_sha") == kernel_source_sha(kernel):
                    return rec["traffic_bytes_per_dispatch"]
    return None


def cpu_baseline(inp, budget_s=12.0):
    """The oracle (numpy float64) on whole tokens of the same workload, ~budget_s of CPU work."""
    from oracle import dsa_oracle as O
    from oracle import run as R
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = inp["cfg"]
    t = 0
    b = int(inp["q_row"][t])
    n = int(inp["q_pos"][t]) + 1
    bt = inp["block_table"][b].cpu().numpy()
    keys = R.request_rows(inp["k_pool"], bt, n)
    kv = [R.request_rows(p, bt, n) for p in inp["kv_pools"]]
    qi, w = R.to_f64(inp["q_idx"][t]), R.to_f64(inp["w"][t])
    qs = [R.to_f64(q[t]) for q in inp["q"]]
    done = 0
    t0 = time.perf_counter()
    while True:
        sc = O.indexer_scores(qi, w, keys)
        idx = O.topk_positions(sc, n, cfg.k)
        sel = idx[idx >= 0]
        for q, rows in zip(qs, kv):
            O.mla_absorbed(q, rows[sel], cfg.Dl, cfg.sm_scale)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= 10000:
            break
    kind = "prefill" if cfg.prefill_tokens else "decode"
    return {"value": done / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} whole {kind} tokens (token 0 of {cfg.name}, n={n}, {cfg.layers} "
                      f"layer(s): indexer, stable-sort top-k, attention) in {el:.1f} s; the oracle's "
                      f"work per token grows with its n"}


# --------------------------------------------------------------------------- benchmark

def run_bench(args):
    import torch
    import dsa_inputs as I
    import sparse_attention_19_amd as D
    from sparse_attention_19_amd import pipeline as P

    cfg = I.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, n_tok, _ = workload_sizes(cfg)
    _, step_parts = algorithmic(cfg)
    step_bytes = sum(step_parts.values())
    copies = args.copies or max(1, min(64, -(-2 * MALL_BYTES // step_bytes)))

    # copies: same lengths and page layout, new data
    inputs = [I.make_inputs(I.shrink(cfg, seed=cfg.seed + 1000 * c, layout_seed=cfg.seed), dev)
              for c in range(copies)]
    buf = P.run_inputs(inputs[0])
    torch.cuda.synchronize()

    def step(i):
        P.run_inputs(inputs[i % copies], buf, step=i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K whole steps back to back, no per-kernel instrumentation
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    # per-kernel durations: the library brackets each launch with HIP events on its stream
    K2 = max(20, min(args.steps, 100))
    D.dsa_timing_start(K2 * (8 + 2 * cfg.layers))
    for i in range(K2):
        step(args.warmup + args.steps + i)
    launches = D.dsa_timing_collect()
    per = {}
    for name, t in launches:
        c = per.setdefault(name, [0, 0.0])
        c[0] += 1
        c[1] += t
    kern = {n: {"launches_per_step": c[0] / K2, "avg_ms": c[1] / c[0], "ms_per_step": c[1] / K2}
            for n, c in per.items()}
    alg, _ = algorithmic(cfg, kernels_seen=set(per))
    dom = max(kern, key=lambda n: kern[n]["ms_per_step"])
    a_bytes, a_flops, bound = alg[dom]
    avg_s = kern[dom]["avg_ms"] * 1e-3
    if bound == "mfma":
        achieved, peak, unit = a_flops / avg_s / 1e12, MFMA_BF16_PEAK_TFS, "TFLOP/s"
    else:
        achieved, peak, unit = a_bytes / avg_s / 1e9, HBM_PEAK_GBS, "GB/s"
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": load_traffic(dom, cfg.name), "kernel": dom,
            "avg_launch_ms": round(kern[dom]["avg_ms"], 5),
            "algorithmic_bytes_per_launch": a_bytes, "algorithmic_flops_per_launch": a_flops}

    value = T / (ms * 1e-3)
    step_gbs = step_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype.itemsize == 2 else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "requests": len(I.context_lengths(cfg)), "ctx": cfg.ctx,
                   "query_tokens": T, "k": cfg.k, "indexer_heads_x_dim": f"{cfg.Hi}x{cfg.Di}",
                   "mla_heads_x_dim": f"{cfg.H}x({cfg.Dl}+{cfg.Dr})", "layers": cfg.layers,
                   "rotated_input_copies": copies},
        "step_hbm": {"algorithmic_bytes": step_bytes, "achieved_gbs": round(step_gbs, 1),
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "kernels": {n: {k: round(v, 5) for k, v in d.items()} for n, d in sorted(kern.items())},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inputs[0])
    print(json.dumps(res), flush=True)


def run_copy_calibration(args):
    """Device-to-device copies of a known size: FETCH_SIZE / WRITE_SIZE of these dispatches
    against the bytes moved give the scale factors applied to the path's kernels."""
    import torch
    n = args.copy_calibration << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": args.steps}), flush=True)


# --------------------------------------------------------------------------- rocprofv3 summaries

def _db(d):
    dbs = glob.glob(os.path.join(d, "**", "*results.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no rocprofv3 results database under {d}")
    return sqlite3.connect(dbs[0])


def _short(name):
    m = re.search(r"dsa::.*?(\w+_kernel)\b", name or "")
    return m.group(1) if m else (name or "")[:40]


def summarize_trace(args):
    c = _db(args.summarize_trace)
    rows = list(c.execute("select name, total_calls, average, total_duration, percentage from top_kernels"))
    print(f"# rocprofv3 kernel trace: {args.title}")
    print(f"# profiled with : {args.command}")
    print(f"# summarised by : python bench.py --summarize-trace <output dir>")
    print("# avg_us and total_ms are per-dispatch GPU durations; the path's kernels are dsa::*")
    print(f"{'kernel':40s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s} {'pct':>6s}")
    for name, calls, avg, total, pct in rows:
        print(f"{_short(name):40s} {calls:6d} {avg:10.3f} {total / 1000.0:10.3f} {pct:6.2f}")


def _counter_per_dispatch(d, counter, pick):
    c = _db(d)
    per = {}
    for kname, disp, cname, val in c.execute(
            "select kernel_name, dispatch_id, counter_name, value from counters_collection"):
        if cname != counter or not pick(kname or ""):
            continue
        per[disp] = per.get(disp, 0.0) + val
    if not per:
        raise SystemExit(f"{d}: no {counter} values for the selected kernel")
    return per


N_XCC = 8   # MI355X: 8 accelerator complex dies, each with its own GRBM


def summarize_counters(args):
    """Per-kernel averages of every counter of a --pmc run (the path's kernels only).
    The database stores one value per dispatch and counter, summed over the counter's
    dimensions; a GRBM counter is kept per XCC, so the per-die value is that sum / N_XCC.
    MfmaUtil, when collected, is rocprofv3's own derived counter
    sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMDs); otherwise it is
    computed the same way from the raw counters (1024 SIMDs)."""
    c = _db(args.summarize_counters)
    per = {}
    for kname, disp, cname, val in c.execute(
            "select kernel_name, dispatch_id, counter_name, value from counters_collection"):
        k = _short(kname or "")
        if not k.endswith("_kernel"):
            continue
        d = per.setdefault(k, {}).setdefault(cname, {})
        d[disp] = d.get(disp, 0.0) + val
    print(f"# rocprofv3 counters: {args.title}")
    print(f"# profiled with : {args.command}")
    print(f"# summarised by : python bench.py --summarize-counters <output dir>")
    print(f"# values per dispatch, summed over the counter's dimensions (GRBM_*: over {N_XCC} XCCs)")
    for k in sorted(per):
        print(k)
        avg = {cname: sum(d.values()) / len(d) for cname, d in per[k].items()}
        for cname, d in sorted(per[k].items()):
            print(f"   {cname:28s} {avg[cname]:18.1f}  per dispatch ({len(d)} dispatches)")
        if "MfmaUtil" not in avg and avg.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            util = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (avg["GRBM_GUI_ACTIVE"] / N_XCC * 1024)
            print(f"   {'MfmaUtil (computed)':28s} {100 * util:18.1f}  % (1024 SIMDs)")


def summarize_traffic(args):
    import dsa_inputs as I
    kernel, cfg = args.kernel, I.CONFIGS[args.workload]
    is_k = lambda n: _short(n) == kernel  # noqa: E731
    fetch = _counter_per_dispatch(args.fetch, "FETCH_SIZE", is_k)
    write = _counter_per_dispatch(args.write, "WRITE_SIZE", is_k)
    exp_kib = args.copy_mib * 1024.0
    big = lambda n: "copy" in n.lower() or "elementwise" in n.lower()  # noqa: E731
    cf = [v for v in _counter_per_dispatch(args.copy_fetch, "FETCH_SIZE", big).values() if v > 0.5 * exp_kib]
    cw = [v for v in _counter_per_dispatch(args.copy_write, "WRITE_SIZE", big).values() if v > 0.5 * exp_kib]
    if not cf or not cw:
        raise SystemExit("copy calibration dispatches not found")
    f_fac = exp_kib / (sum(cf) / len(cf))
    w_fac = exp_kib / (sum(cw) / len(cw))
    f_kib = sum(fetch.values()) / len(fetch)
    w_kib = sum(write.values()) / len(write)
    traffic = (f_kib * f_fac + w_kib * w_fac) * 1024.0
    seen = {"mla_combine_kernel"} if args.combine else set()
    # rows longer than 32768 positions (ld = the longest context) go through the prune kernel
    if -(-max(workload_sizes(cfg)[1]) // 64) * 64 > 32768:
        seen.add("topk_prune_kernel")
    alg, _ = algorithmic(cfg, kernels_seen=seen)
    rec = {"kernel": kernel, "workload": cfg.name, "source_sha": kernel_source_sha(kernel),
           "fetch_kib_per_dispatch": round(f_kib, 1), "write_kib_per_dispatch": round(w_kib, 1),
           "dispatches": len(fetch), "copy_fetch_factor": round(f_fac, 4), "copy_write_factor": round(w_fac, 4),
           "traffic_bytes_per_dispatch": int(traffic), "algorithmic_bytes_per_dispatch": alg[kernel][0]}
    print(f"# HBM traffic of {kernel} on {cfg.name} (rocprofv3 --pmc, one counter per pass)")
    print(f"# FETCH_SIZE pass : {args.fetch_command}")
    print(f"# WRITE_SIZE pass : {args.write_command}")
    print(f"# copy calibration: the same two passes over `python bench.py --copy-calibration {args.copy_mib}`")
    print(f"# summarised by   : python bench.py --summarize-traffic (arguments: the four output dirs)")
    print(f"FETCH_SIZE  {f_kib:14.1f} KiB/dispatch  x {f_fac:.4f} (copy of {args.copy_mib} MiB read "
          f"{sum(cf) / len(cf):.0f} KiB)")
    print(f"WRITE_SIZE  {w_kib:14.1f} KiB/dispatch  x {w_fac:.4f} (copy of {args.copy_mib} MiB wrote "
          f"{sum(cw) / len(cw):.0f} KiB)")
    print(f"traffic     {traffic / 1e6:14.3f} MB/dispatch; algorithmic {alg[kernel][0] / 1e6:.3f} MB "
          f"(ratio {traffic / max(1, alg[kernel][0]):.3f})")
    print("JSON " + json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_b1_32k")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-traffic", action="store_true")
    ap.add_argument("--summarize-counters", metavar="DIR")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="")
    ap.add_argument("--kernel")
    ap.add_argument("--workload")
    ap.add_argument("--combine", action="store_true", help="the MLA ran with its combine kernel")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--fetch-command", default="")
    ap.add_argument("--write-command", default="")
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_traffic:
        return summarize_traffic(args)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build measures "
              f"the path on one MI355X; how it would shard over several is described, not run.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        return run_copy_calibration(args)
    run_bench(args)


if __name__ == "__main__":
    main()
