#!/usr/bin/env python3
"""Benchmark of the retrieval-sparse attention hot path on one MI355X.

A step is one pass of the whole path over one batch: indexer scoring fused with exact top-k selection
(sa_select_topk), then sparse attention over sink + window + selected latent rows (sa_sparse_attn); for the
bucket workload the selection is the Flat bucket search (sa_bucket_select), for the coarse-to-fine workload the
two-stage page-then-token search (sa_hi_select; its mean keys are built once per cache, outside the step). Inputs are synthetic, seeded and
already resident in HBM; several independent copies of the caches rotate so that the measured traffic comes from
HBM rather than the 256 MB Infinity Cache.

Prints one JSON line. Default workload: the prefill chunk (the last 32768 queries of a causal 128K sequence), the
largest single-GPU workload; `--workload` selects another. Each kernel's duration is measured live with HIP events
that the library records on the launch stream right after each of its kernel launches (sa_set_stage_events).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selected-attn queries/sec + indexer keys scored/sec; % of HBM/MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_chunk_128k")
    ap.add_argument("--L", type=int, default=0, help="override the workload's cache length (positions)")
    ap.add_argument("--B", type=int, default=0, help="override the workload's number of queries")
    ap.add_argument("--rotate-bytes", type=float, default=1.2e9, help="total bytes of rotated cache copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="the oracle baseline repeats its query sample until this much CPU time has passed")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference for the HBM counters)")
    return ap.parse_args()


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model or "unknown", "nproc": usable}


def copy_bandwidth_gbps(torch, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of nbytes, timed with events: (read + write) bytes / median time."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * nbytes / sorted(ts)[len(ts) // 2] / 1e9, 1)


def bf16_gemm_tflops(torch, n=8192, reps=5):
    """The library's dense bf16 GEMM (n x n x n, N(0,1) operands, hipBLASLt through torch.mm), timed with events:
    the box's reachable matrix-core rate on random data, beside the spec peak the rooflines divide by."""
    g = torch.Generator(device="cuda").manual_seed(1)
    a = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    c = torch.mm(a, b)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.mm(a, b, out=c)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del a, b, c
    torch.cuda.empty_cache()
    return round(2.0 * n ** 3 / sorted(ts)[len(ts) // 2] / 1e12, 1)


class StageTimer:
    """Per-kernel durations of library calls from events the library records after each of its launches."""

    def __init__(self, torch, lib, n=32):
        self.torch, self.lib, self.n = torch, lib, n
        self.begin = torch.cuda.Event(enable_timing=True)
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in [self.begin] + self.ev:  # events are created on their first record
            e.record()
        torch.cuda.synchronize()
        self.handles = (ctypes.c_void_p * n)(*[e.cuda_event for e in self.ev])

    def run(self, fn, stream):
        """Runs fn() once and returns the durations (ms) of the kernels it launched, in launch order. A spin kernel
        keeps the GPU busy while the host enqueues the call, so no kernel waits for its own launch."""
        self.torch.cuda._sleep(2_000_000)
        self.begin.record(stream)
        self.lib.sa_set_stage_events(self.handles, self.n)
        try:
            fn()
        finally:
            used = self.lib.sa_stage_events_used()
            self.lib.sa_set_stage_events(None, 0)
        self.torch.cuda.synchronize()
        out, prev = [], self.begin
        for e in self.ev[:used]:
            out.append(prev.elapsed_time(e))
            prev = e
        return out


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
    lib = sa.load()
    dev = "cuda"
    over = {k: v for k, v in (("L", args.L), ("B", args.B)) if v}
    wl = get_workload(args.workload, **over)
    torch.manual_seed(0)
    copy_gbps = copy_bandwidth_gbps(torch)
    gemm_tflops = bf16_gemm_tflops(torch)

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
    is_hi = wl.kind == "hi"
    is_blocks = wl.kind in ("qsa", "msa")
    # attention queries: MSA reads one set per (query, group), each group's query heads forming one attention query
    G_att = wl.groups if wl.kind == "msa" else 1
    B_att, H_att = wl.B * G_att, wl.H // G_att
    t_attq = t.repeat_interleave(G_att) if G_att > 1 else t
    if wl.kind == "qsa":
        pooled = [sa.sa_qsa_pool(c["k_idx"], wl.block) for c in copies]
        idx_ld = wl.k_blocks * wl.block + wl.block - 1
        blk_ws = torch.empty(lib.sa_qsa_select_workspace(wl.L, wl.B, wl.H_I, wl.d_I, wl.block, wl.k_blocks),
                             dtype=torch.uint8, device=dev)
    elif wl.kind == "msa":
        idx_ld = wl.k_blocks * wl.block
        blk_ws = torch.empty(lib.sa_msa_select_workspace(wl.L, wl.B, wl.groups, wl.block, wl.k_blocks),
                             dtype=torch.uint8, device=dev)
    elif is_hi:
        build_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        build_ev[0].record()
        hi_means = [sa.sa_hi_build(c["k_idx"], wl.sub_block) for c in copies]
        build_ev[1].record()
        torch.cuda.synchronize()
        build_ms = build_ev[0].elapsed_time(build_ev[1]) / len(copies)
        idx_ld = wl.k_sparse
        hi_ws = torch.empty(sa.sa_hi_select_workspace(wl.L, wl.B, wl.sub_block, wl.page_len, wl.n_pages_keep,
                                                      wl.k_sparse), dtype=torch.uint8, device=dev)
    elif is_bucket:
        dirs = []
        build_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        build_ev[0].record()
        is_tree = wl.tree_fan > 0
        tree_levels = []
        for c in copies:
            dirs.append(sa.sa_bucket_build(c["k_idx"], c["assign"], wl.n_buckets))
        build_ev[1].record()
        torch.cuda.synchronize()
        for c in copies:
            if is_tree:  # one parent level: parent of bucket c = c // fan (siblings numbered contiguously)
                n_top = (wl.n_buckets + wl.tree_fan - 1) // wl.tree_fan
                parent = torch.arange(wl.n_buckets, device=dev, dtype=torch.int32) // wl.tree_fan
                top_reps, _, _ = sa.sa_bucket_build(c["k_idx"], parent[c["assign"].long()], n_top)
                child_off = torch.clamp(torch.arange(n_top + 1, device=dev, dtype=torch.int32) * wl.tree_fan,
                                        max=wl.n_buckets).to(torch.int32)
                tree_levels.append([(top_reps, child_off, wl.tree_keep)])
        torch.cuda.synchronize()
        build_ms = build_ev[0].elapsed_time(build_ev[1]) / len(copies)
        cap = 8192
        idx_ld = cap
        bws = torch.empty(lib.sa_bucket_select_workspace(wl.B, wl.n_buckets, wl.top_b), dtype=torch.uint8,
                          device=dev)
        if is_tree:
            import ctypes
            n_top = tree_levels[0][0][0].shape[0]
            tree_ws = torch.empty(lib.sa_bucket_tree_select_workspace(
                wl.B, 1, (ctypes.c_int32 * 1)(n_top), (ctypes.c_int32 * 1)(wl.tree_keep), wl.n_buckets),
                dtype=torch.uint8, device=dev)
    else:
        idx_ld = wl.k_sparse
        qd = sa.api._dtype(base["q_idx"])
        sel_ws = torch.empty(sa.sa_select_topk_workspace(wl.L, wl.B, wl.H_I, wl.d_I, qd, qd, wl.k_sparse),
                             dtype=torch.uint8, device=dev)
    max_rows = wl.n_sink + wl.n_window + idx_ld
    attn_ws_bytes = sa.sa_sparse_attn_workspace(B_att, H_att, wl.d_qk, wl.d_v, max_rows, sa.api._dtype(base["q"]))
    attn_ws = torch.empty(max(attn_ws_bytes, 256), dtype=torch.uint8, device=dev)
    idx = torch.empty((B_att, idx_ld), dtype=torch.int32, device=dev)
    n_sel = torch.empty((B_att,), dtype=torch.int32, device=dev)
    out = torch.empty((B_att, H_att, wl.d_v), dtype=base["q"].dtype, device=dev)

    def select(i):
        c = copies[i % n_copies]
        if is_bucket and is_tree:
            reps, offsets, members = dirs[i % n_copies]
            sa.sa_bucket_tree_select(c["q_idx"], tree_levels[i % n_copies], reps, offsets, members, wl.L, wl.top_b,
                                     wl.n_sink, wl.n_window, t=t, cap=cap, ws=tree_ws, out=(idx, n_sel))
        elif is_bucket:
            reps, offsets, members = dirs[i % n_copies]
            st = lib.sa_bucket_select(c["q_idx"].data_ptr(), sa.api._dtype(c["q_idx"]), wl.B, wl.d_I,
                                      reps.data_ptr(), offsets.data_ptr(), members.data_ptr(), wl.n_buckets, wl.L,
                                      t.data_ptr(), wl.top_b, wl.n_sink, wl.n_window, idx.data_ptr(), cap,
                                      n_sel.data_ptr(), None, bws.data_ptr(), bws.numel(), stream.cuda_stream)
            sa.api._lib.check("sa_bucket_select", st)
        elif wl.kind == "qsa":
            sa.sa_qsa_select(c["q_idx"], c["w"], pooled[i % n_copies], wl.L, wl.block, wl.k_blocks, t=t, ws=blk_ws,
                             out=(idx, n_sel))
        elif wl.kind == "msa":
            sa.sa_msa_select(c["q_idx"], c["w"], c["k_idx"], wl.groups, wl.block, wl.k_blocks, t=t, ws=blk_ws,
                             out=(idx, n_sel))
        elif is_hi:
            sa.sa_hi_select(c["q_idx"], c["w"], c["k_idx"], hi_means[i % n_copies], wl.sub_block, wl.page_len,
                            wl.n_pages_keep, wl.k_sparse, wl.n_sink, wl.n_window, t=t, ws=hi_ws, out=(idx, n_sel))
        else:
            sa.sa_select_topk(c["q_idx"], c["w"], c["k_idx"], wl.k_sparse, wl.n_sink, wl.n_window, t=t, ws=sel_ws,
                              out=(idx, n_sel))

    def attend(i):
        c = copies[i % n_copies]
        q_att = c["q"].view(B_att, H_att, wl.d_qk) if G_att > 1 else c["q"]
        sa.sa_sparse_attn(q_att, c["kv"], idx, n_sel, wl.n_sink, wl.n_window, wl.softmax_scale, t=t_attq,
                          d_v=wl.d_v, ws=attn_ws, out=out)

    # ---------------- warmup + timed steps ------------------------------------------------------------------------
    for i in range(args.warmup):
        select(i)
        attend(i)
    torch.cuda.synchronize()
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_ev[i][0].record(stream)
        select(i)
        attend(i)
        step_ev[i][1].record(stream)
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t0
    ms_per_step = 1e3 * total_s / args.steps
    step_ms = sorted(a.elapsed_time(b) for a, b in step_ev)
    pct = lambda v, p: v[min(len(v) - 1, int(round(p * (len(v) - 1))))]

    # hot cache: every step on the same copy, whose caches then stay in the 256 MB Infinity Cache when they fit
    # (the timed steps above rotate copies so that each step reads them from HBM)
    hot = None
    if n_copies > 1 and per_copy < (256 << 20):
        hot_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
        select(0)
        attend(0)
        for i in range(args.steps):
            hot_ev[i][0].record(stream)
            select(0)
            attend(0)
            hot_ev[i][1].record(stream)
        torch.cuda.synchronize()
        hot_ms = sorted(a.elapsed_time(b) for a, b in hot_ev)[len(hot_ev) // 2]
        hot = {"ms_per_step": round(hot_ms, 4), "value": round(wl.B / (hot_ms * 1e-3), 1), "unit": "queries/s",
               "cache_bytes": per_copy}

    # ---------------- per-call and per-kernel HIP events on the launch stream -------------------------------------
    # entry points: one event before and one after each call; kernels: the library's stage events (which add a
    # little time between kernels, so the call durations come from the first loop)
    med = lambda v: sorted(v)[len(v) // 2]
    n_stage = max(10, min(args.steps, 30))
    call_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_stage)]
    for i in range(n_stage):
        torch.cuda._sleep(2_000_000)
        call_ev[i][0].record(stream)
        select(i)
        call_ev[i][1].record(stream)
        attend(i)
        call_ev[i][2].record(stream)
        torch.cuda.synchronize()
    t_sel = med([e[0].elapsed_time(e[1]) for e in call_ev]) * 1e-3
    t_att = med([e[1].elapsed_time(e[2]) for e in call_ev]) * 1e-3
    timer = StageTimer(torch, lib)
    sel_k, att_k = [], []
    for i in range(n_stage):
        sel_k.append(timer.run(lambda: select(i), stream))
        att_k.append(timer.run(lambda: attend(i), stream))
    sel_kernels = [med([r[j] for r in sel_k]) for j in range(len(sel_k[0]))]
    att_kernels = [med([r[j] for r in att_k]) for j in range(len(att_k[0]))]

    nsel = n_sel.cpu().tolist()
    rows_total = 0
    for b, tb in enumerate([tt for tt in wl.t_positions() for _ in range(G_att)]):
        ns = min(wl.n_sink, tb + 1)
        w0 = max(ns, tb - wl.n_window + 1)
        rows_total += ns + max(0, tb + 1 - w0) + max(0, nsel[b])
    width = max(wl.d_qk, wl.d_v)
    a_bytes = perf.attn_bytes(rows_total, B_att, H_att, wl.d_qk, wl.d_v, width, wl.attn_dtype)
    a_flops = perf.attn_flops(rows_total, H_att, wl.d_qk, wl.d_v)
    # which kernels serve the workload (the same conditions the library applies)
    attn_mfma = wl.attn_dtype == "bf16" and wl.d_qk == 576 and wl.d_v in (512, 576) and H_att % 64 == 0
    idx_mfma = wl.idx_dtype in ("bf16", "e4m3") and wl.d_I == 128 and wl.H_I in (32, 64)
    t_att_k = att_kernels[0] * 1e-3  # the gather kernel (a split combine, if any, follows it)
    att_name = ("k_attn_mfma" if attn_mfma else "k_attn_generic")
    attn_roof = {"kernel": att_name, "bound": "hbm", "achieved": round(a_bytes / t_att_k / 1e9, 1),
                 "peak": perf.PEAK_HBM_GBPS, "unit": "GB/s",
                 "frac": round(a_bytes / t_att_k / 1e9 / perf.PEAK_HBM_GBPS, 4), "traffic": None,
                 "algorithmic_bytes_per_launch": a_bytes, "launch_ms": round(t_att_k * 1e3, 4),
                 "mfma_tflops": round(a_flops / t_att_k / 1e12, 1),
                 "entry_point": {"name": "sa_sparse_attn", "ms": round(t_att * 1e3, 4),
                                 "hbm_frac": round(a_bytes / t_att / 1e9 / perf.PEAK_HBM_GBPS, 4),
                                 "kernel_ms": [round(x, 4) for x in att_kernels]}}
    if is_bucket and is_tree:
        # representatives read: every root node once (shared by the queries), and each query's kept nodes'
        # children; the longest kernel of the call is reported
        n_top = tree_levels[0][0][0].shape[0]
        rep_bytes = (n_top + wl.B * wl.tree_keep * wl.tree_fan) * wl.d_I * 4
        n_keys = wl.B * (n_top + wl.tree_keep * wl.tree_fan)
        t_sel_k = max(sel_kernels) * 1e-3
        sel_roof = {"kernel": "the select call's longest kernel", "bound": "hbm",
                    "achieved": round(rep_bytes / t_sel_k / 1e9, 1), "peak": perf.PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(rep_bytes / t_sel_k / 1e9 / perf.PEAK_HBM_GBPS, 4), "traffic": None,
                    "algorithmic_bytes_per_launch": rep_bytes, "launch_ms": round(t_sel_k * 1e3, 4),
                    "entry_point": {"name": "sa_bucket_tree_select", "ms": round(t_sel * 1e3, 4),
                                    "hbm_frac": round(rep_bytes / t_sel / 1e9 / perf.PEAK_HBM_GBPS, 4),
                                    "kernel_ms": [round(x, 4) for x in sel_kernels]}}
        keys_per_s = n_keys / t_sel
    elif is_bucket:
        n_keys = wl.B * wl.n_buckets
        rep_bytes = wl.n_buckets * wl.d_I * 4
        t_sel_k = sel_kernels[0] * 1e-3
        sel_roof = {"kernel": "k_bucket_scores", "bound": "hbm", "achieved": round(rep_bytes / t_sel_k / 1e9, 1),
                    "peak": perf.PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(rep_bytes / t_sel_k / 1e9 / perf.PEAK_HBM_GBPS, 4), "traffic": None,
                    "algorithmic_bytes_per_launch": rep_bytes, "launch_ms": round(t_sel_k * 1e3, 4),
                    "entry_point": {"name": "sa_bucket_select", "ms": round(t_sel * 1e3, 4),
                                    "hbm_frac": round(rep_bytes / t_sel / 1e9 / perf.PEAK_HBM_GBPS, 4),
                                    "kernel_ms": [round(x, 4) for x in sel_kernels]}}
        keys_per_s = n_keys / t_sel
    elif is_hi:
        sel_roof, keys_per_s, hi_info = hi_roofline(sa, wl, copies[0], hi_means[0], t, sel_kernels, t_sel)
        t_sel_k = sel_roof["launch_ms"] * 1e-3
    elif is_blocks:
        # scored (query, key) pairs: QSA scores each query's complete micro-blocks' pooled keys, MSA every
        # position before each query's local block (all indexer heads over the groups)
        ts_ = wl.t_positions()
        if wl.kind == "qsa":
            pairs = sum((tb + 1) // wl.block for tb in ts_)
        else:
            pairs = sum((tb // wl.block) * wl.block for tb in ts_)
        i_flops = perf.indexer_flops(pairs, wl.H_I, wl.d_I)
        peak = perf.PEAK_TFLOPS["bf16"]
        t_sel_k = max(sel_kernels) * 1e-3
        tf = i_flops / t_sel_k / 1e12
        sel_roof = {"kernel": "scorer (the select call's longest kernel)", "bound": "mfma", "achieved": round(tf, 1),
                    "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4), "traffic": None,
                    "algorithmic_flops_per_launch": i_flops, "launch_ms": round(t_sel_k * 1e3, 4),
                    "entry_point": {"name": f"sa_{wl.kind}_select", "ms": round(t_sel * 1e3, 4),
                                    "mfma_frac": round(i_flops / t_sel / 1e12 / peak, 4),
                                    "kernel_ms": [round(x, 4) for x in sel_kernels]}}
        flat_pairs = sum(max(0, tb - wl.n_window - wl.n_sink + 1) for tb in ts_)
        keys_per_s = flat_pairs / t_sel
    else:
        pairs = sum(max(0, tb - wl.n_window - wl.n_sink + 1) for tb in wl.t_positions())
        i_flops = perf.indexer_flops(pairs, wl.H_I, wl.d_I)
        i_bytes = perf.indexer_bytes(wl.L, wl.B, wl.H_I, wl.d_I, wl.idx_dtype)
        peak = perf.PEAK_TFLOPS["bf16" if idx_mfma else "f32_vector"]
        # the scoring kernel is the select call's longest; it runs every indexer flop where the call is one scoring
        # launch (the per-query kernel, or the stream's fill, scoring launch and merge). Where the positions are
        # scored in several launches (few queries over many positions) the whole entry point is reported.
        per_query = idx_mfma and wl.B >= 64
        one_scorer = per_query or not idx_mfma or len(sel_kernels) == 3
        if one_scorer:
            t_sel_k = max(sel_kernels) * 1e-3
            sname = ("k_stream_select" if per_query else "k_score_stream") if idx_mfma else "k_score_valu"
        else:
            t_sel_k = t_sel
            sname = "sa_select_topk (the whole call: several scoring launches and merges)"
        tf = i_flops / t_sel_k / 1e12
        gbps = i_bytes / t_sel_k / 1e9
        # the bound is whichever peak the algorithmic work needs longer at: the matrix unit for many queries, the
        # key stream for few (one query scores 64 flop per key byte, below the bf16 ridge of about 312)
        hbm_bound = idx_mfma and i_bytes / (perf.PEAK_HBM_GBPS * 1e9) > i_flops / (peak * 1e12)
        if hbm_bound:
            sel_roof = {"kernel": sname, "bound": "hbm", "achieved": round(gbps, 1), "peak": perf.PEAK_HBM_GBPS,
                        "unit": "GB/s", "frac": round(gbps / perf.PEAK_HBM_GBPS, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": i_bytes, "mfma_tflops": round(tf, 1)}
        else:
            sel_roof = {"kernel": sname, "bound": "mfma" if idx_mfma else "alu", "achieved": round(tf, 1),
                        "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4), "traffic": None,
                        "algorithmic_flops_per_launch": i_flops, "hbm_gbps": round(gbps, 1)}
        sel_roof.update({"launch_ms": round(t_sel_k * 1e3, 4),
                         "entry_point": {"name": "sa_select_topk", "ms": round(t_sel * 1e3, 4),
                                         "mfma_frac": round(i_flops / t_sel / 1e12 / peak, 4),
                                         "hbm_frac": round(i_bytes / t_sel / 1e9 / perf.PEAK_HBM_GBPS, 4),
                                         "kernel_ms": [round(x, 4) for x in sel_kernels]}})
        keys_per_s = pairs / t_sel
    # counters are taken on the workload's own shape: with L or B overridden they do not apply
    traffic = None if over else measured_traffic(wl.name)
    if traffic:  # per dispatch of the roofline's kernel (its name up to the first space)
        sel_roof["traffic"] = traffic.get(sel_roof["kernel"].split(" ")[0])
        attn_roof["traffic"] = traffic.get(attn_roof["kernel"].split(" ")[0])
    dominant, other = (sel_roof, attn_roof) if t_sel_k >= t_att_k else (attn_roof, sel_roof)

    res = {
        "metric": METRIC, "value": round(wl.B / (ms_per_step * 1e-3), 1), "unit": "queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"e4m3": "e4m3 index / bf16 attn", "bf16": "bf16", "f32": "f32"}[wl.idx_dtype],
        "data": "synthetic (seeded N(0,1) queries, index keys and latent rows)",
        "config": {"workload": wl.name, "L": wl.L, "B": wl.B, "H_I": wl.H_I, "d_I": wl.d_I, "k_sparse": wl.k_sparse,
                   "n_buckets": wl.n_buckets, "top_b": wl.top_b, "n_sink": wl.n_sink, "n_window": wl.n_window,
                   "H": wl.H, "d_latent": width, "d_v": wl.d_v, "causal_chunk": wl.causal_chunk,
                   "cache_copies_rotated": n_copies},
        "step_ms_p10_p50_p90": [round(pct(step_ms, 0.1), 4), round(pct(step_ms, 0.5), 4), round(pct(step_ms, 0.9), 4)],
        "indexer_keys_scored_per_s": round(keys_per_s, 1),
        "selected_attn_queries_per_s": round(wl.B / t_att, 1),
        "stage_ms": {"select": round(t_sel * 1e3, 4), "attn": round(t_att * 1e3, 4)},
        "roofline": dominant, "roofline_other": other,
        "measured_copy_gbps": copy_gbps,
        "measured_bf16_gemm_tflops": gemm_tflops,
    }
    if hot:
        res["hot_cache"] = hot
    if is_bucket:
        res["bucket_build_ms_per_cache"] = round(build_ms, 3)
        if is_tree:
            res["config"].update(tree_fan=wl.tree_fan, tree_keep=wl.tree_keep)
    if is_blocks:
        res["config"].update(block=wl.block, k_blocks=wl.k_blocks, groups=wl.groups)
    if is_hi:
        res["config"].update(sub_block=wl.sub_block, page_len=wl.page_len, n_pages_keep=wl.n_pages_keep)
        res["hi"] = {**hi_info, "means_build_ms_per_cache": round(build_ms, 3)}

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, base, args.cpu_seconds)
    res["host"] = {**host_info(), "gpu": torch.cuda.get_device_name(0)}
    print(json.dumps(res))


HI_KERNELS = ["k_score_mfma (page scores)", "k_keys_from_scores (pages)", "k_radix_hist<0>", "k_radix_hist<1>",
              "k_radix_hist<2>", "k_radix_count", "k_radix_write", "k_hi_fine", "k_merge"]


def hi_roofline(sa, wl, c, means, t, sel_kernels, t_sel):
    """Roofline of the coarse-to-fine select's longest kernel. Algorithmic work: the page scorer scores every
    visible sub-block mean key of every query; the token stage scores, per query, the candidates inside its
    recalled pages (counted from the pages one extra call returns)."""
    import numpy as np
    assert len(sel_kernels) == len(HI_KERNELS), sel_kernels
    from sa_workloads import perf
    _, _, pages = sa.sa_hi_select(c["q_idx"], c["w"], c["k_idx"], means, wl.sub_block, wl.page_len,
                                  wl.n_pages_keep, wl.k_sparse, wl.n_sink, wl.n_window, t=t, return_pages=True)
    pages = pages.cpu().numpy().astype(np.int64)
    P, g = wl.page_len, wl.page_len // wl.sub_block
    n_sub = (wl.L + wl.sub_block - 1) // wl.sub_block
    ts = np.asarray(wl.t_positions(), dtype=np.int64)
    page_pairs = int(np.minimum(n_sub, (ts // P + 1) * g).sum())
    # candidates of query b inside page p: [max(pP, n_sink), min(pP + P - 1, L - 1, t_b - n_window)]
    lo = np.maximum(pages * P, wl.n_sink)
    hi = np.minimum(np.minimum(pages * P + P - 1, wl.L - 1), (ts - wl.n_window)[:, None])
    token_pairs = int(np.where(pages >= 0, np.maximum(0, hi - lo + 1), 0).sum())
    flat_pairs = int(np.maximum(0, ts - wl.n_window - wl.n_sink + 1).sum())
    peak = perf.PEAK_TFLOPS["bf16"]
    work = {"k_score_mfma (page scores)": perf.indexer_flops(page_pairs, wl.H_I, wl.d_I),
            "k_hi_fine": perf.indexer_flops(token_pairs, wl.H_I, wl.d_I)}
    kernels = {}
    for name, ms in zip(HI_KERNELS, sel_kernels):
        kernels[name] = {"ms": round(ms, 4)}
        if name in work:
            kernels[name]["tflops"] = round(work[name] / (ms * 1e-3) / 1e12, 1)
            kernels[name]["mfma_frac"] = round(work[name] / (ms * 1e-3) / 1e12 / peak, 4)
    j = int(np.argmax(sel_kernels))
    name, ms = HI_KERNELS[j], sel_kernels[j]
    if name in work:
        tf = work[name] / (ms * 1e-3) / 1e12
        roof = {"kernel": name, "bound": "mfma", "achieved": round(tf, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tf / peak, 4), "algorithmic_flops_per_launch": work[name]}
    else:
        roof = {"kernel": name, "bound": "hbm", "achieved": None, "peak": perf.PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": None}
    all_flops = work["k_score_mfma (page scores)"] + work["k_hi_fine"]
    roof.update({"traffic": None, "launch_ms": round(ms, 4),
                 "entry_point": {"name": "sa_hi_select", "ms": round(t_sel * 1e3, 4),
                                 "mfma_frac": round(all_flops / t_sel / 1e12 / peak, 4),
                                 "kernel_ms": [round(x, 4) for x in sel_kernels]}})
    info = {"kernels": kernels, "sub_block_keys_scored": page_pairs, "token_pairs_scored": token_pairs,
            "flat_equivalent_pairs": flat_pairs,
            "token_gather_gbps": round(token_pairs * wl.d_I * 2 / (sel_kernels[HI_KERNELS.index("k_hi_fine")]
                                                                    * 1e-3) / 1e9, 1)}
    return roof, flat_pairs / t_sel, info


def measured_traffic(workload: str):
    """HBM bytes per launch of each kernel from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this
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
    return {k: v["read_bytes"] + v["write_bytes"] for k, v in rec.get("kernels", {}).items()}


STEP_DESC = {"hi": "page scores, top pages, token top-k inside them",
             "qsa": "pooled-key scores of the complete micro-blocks, top micro-blocks expanded plus the tail",
             "msa": "per-group token scores, block maxima, top blocks plus the local block",
             "bucket": "bucket scores, top buckets expanded"}
STEP_DESC_TREE = "parent-node scores, kept parents' bucket scores, top buckets expanded"


def cpu_baseline(wl, base, min_seconds):
    """The oracle as it stands, timed on the host cores over a bounded sample of the same workload: a seeded
    sample of queries (with the first and the last), cycled until min_seconds have passed. For causal workloads the
    queries differ in the number of positions they score, so the rate is taken per scored (query, position) pair
    and divided by the workload's mean pairs per query (extrapolated by pair count)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import sa_oracle as O
    from tests.gpu_helpers import to_f64

    t0 = time.perf_counter()
    kv = to_f64(base["kv"])
    q = base["q"]
    if wl.kind == "bucket":
        kf = to_f64(base["k_idx"])
        assign = base["assign"].cpu().numpy()
        reps, off, mem = O.bucket_build(kf, assign, wl.n_buckets)
        qi = base["q_idx"]
        if wl.tree_fan:  # the parent level, built once per cache as on the GPU: not timed
            import numpy as np
            n_top = (wl.n_buckets + wl.tree_fan - 1) // wl.tree_fan
            top_reps, _, _ = O.bucket_build(kf, assign // wl.tree_fan, n_top)
            levels = [(top_reps, np.minimum(np.arange(n_top + 1) * wl.tree_fan, wl.n_buckets))]
    elif wl.kind == "hi":
        kf = to_f64(base["k_idx"])
        means = O.hi_means(kf, wl.sub_block)       # once per cache, as on the GPU: not timed
        qi, w = base["q_idx"], base["w"].double().cpu().numpy()
    elif wl.kind == "qsa":
        kf = to_f64(base["k_idx"])
        pooled = O.qsa_pool(kf, wl.block)          # once per cache, as on the GPU: not timed
        qi, w = base["q_idx"], base["w"].double().cpu().numpy()
    else:
        kf = to_f64(base["k_idx"])
        qi, w = base["q_idx"], base["w"].double().cpu().numpy()
    prep = time.perf_counter() - t0
    ts = wl.t_positions()
    pairs_of = lambda tb: max(1, tb - wl.n_window - wl.n_sink + 1)
    rng = np.random.default_rng(0)
    n_s = min(wl.B, 64 if wl.L <= 200_000 else 1)
    if n_s == 1:
        sample = [0]
    else:
        others = rng.choice(np.arange(1, wl.B - 1), size=n_s - 2, replace=False).tolist() if n_s > 2 else []
        sample = sorted({0, wl.B - 1, *others})
    qi64, q64 = {}, {}  # per-query inputs decoded to fp64 on first use, outside the timed part
    done, pairs_done, dt = 0, 0, 0.0
    while True:
        b = sample[done % len(sample)]
        if b not in q64:
            t1 = time.perf_counter()
            qi64[b], q64[b] = to_f64(qi[b]), to_f64(q[b])
            prep += time.perf_counter() - t1
        t0 = time.perf_counter()
        if wl.kind == "qsa":
            R, _, _ = O.qsa_select(qi64[b], w[b], pooled, ts[b], wl.block, wl.k_blocks)
            O.sparse_attn(q64[b], kv, R, wl.softmax_scale, wl.d_qk, wl.d_v)
        elif wl.kind == "msa":
            Hg = wl.H // wl.groups
            for g, (R, _, _) in enumerate(O.msa_select(qi64[b], w[b], kf, ts[b], wl.groups, wl.block, wl.k_blocks)):
                O.sparse_attn(q64[b][g * Hg:(g + 1) * Hg], kv, R, wl.softmax_scale, wl.d_qk, wl.d_v)
        elif wl.kind == "hi":
            O.hi_step(qi64[b], w[b], kf, means, q64[b], kv, ts[b], wl.page_len, wl.sub_block, wl.n_pages_keep,
                      wl.k_sparse, wl.n_sink, wl.n_window, wl.softmax_scale, wl.d_qk, wl.d_v)
        elif wl.kind == "bucket" and wl.tree_fan:
            R0, _, _ = O.tree_select(qi64[b], levels, reps, off, mem, ts[b], [wl.tree_keep], wl.top_b, wl.n_sink,
                                     wl.n_window)
            O.sparse_attn(q64[b], kv, O.read_set(ts[b], wl.n_sink, wl.n_window, R0), wl.softmax_scale, wl.d_qk,
                          wl.d_v)
        elif wl.kind == "bucket":
            O.bucket_step(qi64[b], reps, off, mem, q64[b], kv, ts[b], wl.top_b, wl.n_sink, wl.n_window,
                          wl.softmax_scale, wl.d_qk, wl.d_v)
        else:
            O.dsa_step(qi64[b], w[b], kf, q64[b], kv, ts[b], wl.k_sparse, wl.n_sink, wl.n_window,
                       wl.softmax_scale, wl.d_qk, wl.d_v)
        done += 1
        pairs_done += pairs_of(ts[b])
        dt += time.perf_counter() - t0
        if dt >= min_seconds:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    mean_pairs = sum(pairs_of(tb) for tb in ts) / len(ts)
    causal = wl.kind == "dsa" and len(set(ts)) > 1
    value = pairs_done / dt / mean_pairs if causal else done / dt
    which = f"{len(sample)} seeded queries of {wl.name} ({wl.B} in all, first and last included), cycled: " \
            f"{done} query evaluations"
    how = (f"; rate per scored pair ({pairs_done} pairs) divided by the mean {mean_pairs:.0f} pairs per query "
           "(extrapolated by pair count)") if causal else ""
    return {"value": round(value, 3), "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{which}; full per-query path ({STEP_DESC_TREE if wl.tree_fan else STEP_DESC.get(wl.kind, 'score all candidates, exact top-k')}, attention), fp64 numpy"
                      f"{how}; {prep:.1f} s input decode not counted",
            "extrapolated": causal, "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
