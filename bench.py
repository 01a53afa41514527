#!/usr/bin/env python3
"""Benchmark of the retrieval-sparse attention hot path on one MI355X.

A step is one pass of the whole path over one batch: indexer scoring fused with exact top-k selection
(sa_select_topk), then sparse attention over sink + window + selected latent rows (sa_sparse_attn); for the
bucket workload the selection is the Flat bucket search (sa_bucket_select). Inputs are synthetic, seeded and
already resident in HBM; several independent copies of the caches rotate so that the measured traffic comes from
HBM rather than the 256 MB Infinity Cache.

Prints one JSON line. Default: the DSA-style decode at 128K (16 queries, L = 131072).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selected-attn queries/sec + indexer keys scored/sec; % of HBM/MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsa_decode_128k")
    ap.add_argument("--rotate-bytes", type=float, default=1.2e9, help="total bytes of rotated cache copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-queries", type=int, default=0, help="0 = pick by workload")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="the oracle baseline repeats its query sample until this much CPU time has passed")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference for the HBM counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (sharding the cache along the "
              "sequence is described in the design notes, not implemented). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_sparse_sa_amd as sa
    from sa_workloads import gen, get_workload, perf

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}))
        return
    sa.load()
    dev = "cuda"
    wl = get_workload(args.workload)
    torch.manual_seed(0)

    # ---------------- inputs, rotated copies of the caches --------------------------------------------------------
    base = gen.make_inputs(wl, device=dev)
    cache_keys = ["k_idx", "kv"]
    per_copy = sum(base[k].numel() * base[k].element_size() for k in cache_keys)
    n_copies = max(1, min(8, int(math.ceil(args.rotate_bytes / per_copy))))
    free = torch.cuda.mem_get_info()[0]
    while n_copies > 1 and per_copy * (n_copies - 1) > 0.6 * free:
        n_copies -= 1
    copies = [base] + [{**base, **{k: base[k].clone() for k in cache_keys}} for _ in range(n_copies - 1)]

    stream = torch.cuda.current_stream()
    t = base["t"]
    is_bucket = wl.kind == "bucket"
    if is_bucket:
        dirs = []
        build_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        build_ev[0].record()
        for c in copies:
            dirs.append(sa.sa_bucket_build(c["k_idx"], c["assign"], wl.n_buckets))
        build_ev[1].record()
        torch.cuda.synchronize()
        build_ms = build_ev[0].elapsed_time(build_ev[1]) / len(copies)
        cap = 8192
        idx_ld = cap
        bws = torch.empty(sa.api._lib.load().sa_bucket_select_workspace(wl.B, wl.n_buckets, wl.top_b),
                          dtype=torch.uint8, device=dev)
    else:
        idx_ld = wl.k_sparse
        qd = sa.api._dtype(base["q_idx"])
        sel_ws = torch.empty(sa.sa_select_topk_workspace(wl.L, wl.B, wl.H_I, wl.d_I, qd, qd, wl.k_sparse),
                             dtype=torch.uint8, device=dev)
    max_rows = wl.n_sink + wl.n_window + idx_ld
    attn_ws_bytes = sa.sa_sparse_attn_workspace(wl.B, wl.H, wl.d_qk, wl.d_v, max_rows, sa.api._dtype(base["q"]))
    attn_ws = torch.empty(max(attn_ws_bytes, 256), dtype=torch.uint8, device=dev)
    idx = torch.empty((wl.B, idx_ld), dtype=torch.int32, device=dev)
    n_sel = torch.empty((wl.B,), dtype=torch.int32, device=dev)
    out = torch.empty((wl.B, wl.H, wl.d_v), dtype=base["q"].dtype, device=dev)

    def select(i):
        c = copies[i % n_copies]
        if is_bucket:
            reps, offsets, members = dirs[i % n_copies]
            lib = sa.api._lib.load()
            st = lib.sa_bucket_select(c["q_idx"].data_ptr(), sa.api._dtype(c["q_idx"]), wl.B, wl.d_I,
                                      reps.data_ptr(), offsets.data_ptr(), members.data_ptr(), wl.n_buckets, wl.L,
                                      t.data_ptr(), wl.top_b, wl.n_sink, wl.n_window, idx.data_ptr(), cap,
                                      n_sel.data_ptr(), None, bws.data_ptr(), bws.numel(), stream.cuda_stream)
            sa.api._lib.check("sa_bucket_select", st)
        else:
            sa.sa_select_topk(c["q_idx"], c["w"], c["k_idx"], wl.k_sparse, wl.n_sink, wl.n_window, t=t, ws=sel_ws,
                              out=(idx, n_sel))

    def attend(i):
        c = copies[i % n_copies]
        sa.sa_sparse_attn(c["q"], c["kv"], idx, n_sel, wl.n_sink, wl.n_window, wl.softmax_scale, t=t, d_v=wl.d_v,
                          ws=attn_ws, out=out)

    # ---------------- warmup + timed steps ------------------------------------------------------------------------
    for i in range(args.warmup):
        select(i)
        attend(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        select(i)
        attend(i)
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t0
    ms_per_step = 1e3 * total_s / args.steps

    # ---------------- per-stage HIP events on the launch stream ---------------------------------------------------
    n_stage = max(10, min(args.steps, 50))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_stage)]
    for i in range(n_stage):
        ev[i][0].record(stream)
        select(i)
        ev[i][1].record(stream)
        attend(i)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    sel_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    att_ms = sorted(e[1].elapsed_time(e[2]) for e in ev)
    med = lambda v: v[len(v) // 2]
    t_sel, t_att = med(sel_ms) * 1e-3, med(att_ms) * 1e-3

    nsel = n_sel.cpu().tolist()
    rows_total = 0
    for b, tb in enumerate(wl.t_positions()):
        ns = min(wl.n_sink, tb + 1)
        w0 = max(ns, tb - wl.n_window + 1)
        rows_total += ns + max(0, tb + 1 - w0) + max(0, nsel[b])
    width = max(wl.d_qk, wl.d_v)
    a_bytes = perf.attn_bytes(rows_total, wl.B, wl.H, wl.d_qk, wl.d_v, width, wl.attn_dtype)
    a_flops = perf.attn_flops(rows_total, wl.H, wl.d_qk, wl.d_v)
    attn_gbps = a_bytes / t_att / 1e9
    # which kernels serve the workload (the same conditions the library applies)
    attn_mfma = wl.attn_dtype == "bf16" and wl.d_qk == 576 and wl.d_v in (512, 576) and wl.H % 64 == 0
    idx_mfma = wl.idx_dtype in ("bf16", "e4m3") and wl.d_I == 128 and wl.H_I in (32, 64)
    attn_roof = {"kernel": "sa_sparse_attn (" + ("gather + MFMA + split combine" if attn_mfma
                                                 else "fp32 VALU kernel, one block per head") + ")", "bound": "hbm",
                 "achieved": round(attn_gbps, 1), "peak": perf.PEAK_HBM_GBPS, "unit": "GB/s",
                 "frac": round(attn_gbps / perf.PEAK_HBM_GBPS, 4), "traffic": None,
                 "algorithmic_bytes_per_launch": a_bytes, "launch_ms": round(t_att * 1e3, 4),
                 "mfma_tflops": round(a_flops / t_att / 1e12, 1)}
    if is_bucket:
        n_keys = wl.B * wl.n_buckets
        sel_roof = {"kernel": "sa_bucket_select (rep scan + top-b + expand)", "bound": "hbm",
                    "achieved": round(wl.n_buckets * wl.d_I * 4 / t_sel / 1e9, 1), "peak": perf.PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(wl.n_buckets * wl.d_I * 4 / t_sel / 1e9 / perf.PEAK_HBM_GBPS, 4),
                    "traffic": None, "launch_ms": round(t_sel * 1e3, 4)}
        keys_per_s = n_keys / t_sel
    else:
        pairs = 0
        for tb in wl.t_positions():
            lo, hi = wl.n_sink, tb - wl.n_window
            pairs += max(0, hi - lo + 1)
        i_flops = perf.indexer_flops(pairs, wl.H_I, wl.d_I)
        i_bytes = perf.indexer_bytes(wl.L, wl.B, wl.H_I, wl.d_I, wl.idx_dtype)
        tf = i_flops / t_sel / 1e12
        peak = perf.PEAK_TFLOPS["bf16" if idx_mfma else "f32_vector"]
        sel_roof = {"kernel": "sa_select_topk (" + ("MFMA" if idx_mfma else "fp32 VALU") + " scoring + exact top-k)",
                    "bound": "mfma" if idx_mfma else "alu",
                    "achieved": round(tf, 1), "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                    "traffic": None, "algorithmic_flops_per_launch": i_flops, "launch_ms": round(t_sel * 1e3, 4),
                    "hbm_gbps": round(i_bytes / t_sel / 1e9, 1)}
        keys_per_s = pairs / t_sel
    traffic = measured_traffic(wl.name)
    if traffic:
        sel_roof["traffic"] = traffic.get("select")
        attn_roof["traffic"] = traffic.get("attn")
    dominant, other = (sel_roof, attn_roof) if t_sel >= t_att else (attn_roof, sel_roof)

    res = {
        "metric": METRIC, "value": round(wl.B / (ms_per_step * 1e-3), 1), "unit": "queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"e4m3": "e4m3 index / bf16 attn", "bf16": "bf16", "f32": "f32"}[wl.idx_dtype],
        "data": "synthetic (seeded N(0,1) queries, index keys and latent rows)",
        "config": {"workload": wl.name, "L": wl.L, "B": wl.B, "H_I": wl.H_I, "d_I": wl.d_I, "k_sparse": wl.k_sparse,
                   "n_buckets": wl.n_buckets, "top_b": wl.top_b, "n_sink": wl.n_sink, "n_window": wl.n_window,
                   "H": wl.H, "d_latent": width, "d_v": wl.d_v, "cache_copies_rotated": n_copies},
        "indexer_keys_scored_per_s": round(keys_per_s, 1),
        "selected_attn_queries_per_s": round(wl.B / t_att, 1),
        "stage_ms": {"select": round(t_sel * 1e3, 4), "attn": round(t_att * 1e3, 4)},
        "roofline": dominant, "roofline_other": other,
    }
    if is_bucket:
        res["bucket_build_ms_per_cache"] = round(build_ms, 3)

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, base, args.cpu_sample_queries, args.cpu_seconds)
    res["host"] = {"cpu": platform.processor() or platform.machine(), "nproc": os.cpu_count(),
                   "gpu": torch.cuda.get_device_name(0)}
    print(json.dumps(res))


def measured_traffic(workload: str):
    """HBM bytes per call of each stage from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this
    workload (scaled by the plain-copy calibration), or None when there is none or when the kernel sources no
    longer hash to the ones the counters were taken on."""
    import glob
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "long_context_sparse_sa_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    if h.hexdigest() != rec.get("source_sha256"):
        return None
    return {k: v["read_bytes"] + v["write_bytes"] for k, v in rec.items() if isinstance(v, dict)}


def cpu_baseline(wl, base, n_sample, min_seconds):
    """The oracle as it stands, timed on the host cores over a bounded sample of the same workload: the first
    n_sample queries, cycled until min_seconds have passed (at least one query)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import sa_oracle as O
    from tests.gpu_helpers import to_f64

    t0 = time.perf_counter()
    kv = to_f64(base["kv"])
    q = base["q"]
    if wl.kind == "bucket":
        kf = to_f64(base["k_idx"])
        reps, off, mem = O.bucket_build(kf, base["assign"].cpu().numpy(), wl.n_buckets)
        qi = base["q_idx"]
    else:
        kf = to_f64(base["k_idx"])
        qi, w = base["q_idx"], base["w"].double().cpu().numpy()
    prep = time.perf_counter() - t0
    ts = wl.t_positions()
    n = n_sample or (wl.B if wl.L <= 200_000 else 1)
    n = min(n, wl.B)
    qi64, q64 = {}, {}  # per-query inputs decoded to fp64 on first use, outside the timed part
    done = 0
    dt = 0.0
    while True:
        b = done % n
        if b not in q64:
            t1 = time.perf_counter()
            qi64[b], q64[b] = to_f64(qi[b]), to_f64(q[b])
            prep += time.perf_counter() - t1
        t0 = time.perf_counter()
        if wl.kind == "bucket":
            O.bucket_step(qi64[b], reps, off, mem, q64[b], kv, ts[b], wl.top_b, wl.n_sink, wl.n_window,
                          wl.softmax_scale, wl.d_qk, wl.d_v)
        else:
            O.dsa_step(qi64[b], w[b], kf, q64[b], kv, ts[b], wl.k_sparse, wl.n_sink, wl.n_window,
                       wl.softmax_scale, wl.d_qk, wl.d_v)
        done += 1
        dt += time.perf_counter() - t0
        if dt >= min_seconds:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    which = (f"queries 0..{done - 1} of {wl.name} ({wl.B} in all), each once" if done <= n else
             f"queries 0..{n - 1} of {wl.name}, cycled: {done} query evaluations")
    return {"value": round(done / dt, 3), "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{which}; full per-query path (score all candidates, exact top-k, attention), fp64 numpy; "
                      f"{prep:.1f} s input decode not counted",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
