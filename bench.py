#!/usr/bin/env python3
"""Benchmark of one decode step of GQA over a paged KV cache on one MI355X.

A step is the whole path over one batch of synthetic input: the split count
(host), kv_store of the batch's new rows, split-KV paged attention and the
log-sum-exp merge.  The headline workload is the largest of the five decode
workloads on one GPU, the ragged batch (B=64, lengths ~ U{1..8192} drawn from
its seed, 32 q / 8 kv heads, D=128, bf16, page_size 16, 32768-page pool,
shuffled page table: 1.15 GB of K+V per step).

Headline timing (first in the run, right after the headline's inputs are
resident): W untimed steps, then exactly K steps launched one call at a
time between two device synchronisations (`eager_ms_per_step`), then the same
K steps captured into one HIP graph (each step on its own copy of the pool,
rotating over `--layers` copies so that no step finds its K/V in the 256 MB
Infinity Cache), replayed once untimed and once timed between two
synchronisations: that replay gives `ms_per_step` and `value` (K+V bytes per
step / time per step).  Each step is one `pkv_decode_step` call (the store
fused into the attention kernel, then the merge when there are several splits).

Per-workload figures (all five workloads, in `workloads`): every measured call
is captured n times back to back in a HIP graph (rotating pools), and the
graph is replayed R times with HIP events around each replay on the stream the
kernels run on; the R per-call means give the median, the interquartile mean
and the mean.  Measured: attention + merge (`pkv_paged_decode_attn_merged`),
the attention kernel alone (`pkv_paged_decode_attn`), the merge alone, the
whole fused step, the store of one step's rows, and the store's bulk fill of
every position beside two copy ceilings of the same bytes (libpkv_bench.so): a
linear copy, and the same rows moved to the same destinations one page run
per workgroup.

`roofline` is the attention kernel at the headline workload: algorithmic bytes
per launch over its graph-timed mean duration.  `cpu_baseline` is the C oracle
(store + fp64 attention) on the host's cores for about `--cpu-seconds` of
whole headline steps.  Prints ONE JSON line on stdout; details go to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--workloads A,B,..]
                    [--reps R] [--no-cpu-baseline] [--no-extras]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak, published
HEADLINE = "ragged_batch"
ALL_WORKLOADS = ["tiny_gqa", "llama3_8b_decode", "ragged_batch", "long_context", "mha_page1"]

# HBM bytes per launch of the attention kernel at the headline workload,
# counted by rocprofv3 in two runs (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), each scaled by what the same counter reads for a 1 GiB copy.
# Keyed by the sha256 of the kernel's sources when the counters were taken:
# any edit to them voids the figure (then `traffic` is null).
COUNTED_TRAFFIC = {
    "workload": HEADLINE,
    "sources_sha256": "714e7776efbba3b64a3767dbcb358b891e1386061080161832643780d5a5409a",
    "read_bytes": 1153932570,    # FETCH_SIZE 563469.0 KiB x (1 GiB / 524311.6 KiB)
    "write_bytes": 4238950,      # WRITE_SIZE 4139.6 KiB x (1 GiB / 1048576.0 KiB)
}
KERNEL_SOURCES = ["pkv_decode_mfma.hip", "pkv_device.h", "pkv_launch.h"]


def kernel_sources_sha256() -> str:
    import hashlib
    from pathlib import Path
    h = hashlib.sha256()
    csrc = Path(__file__).resolve().parent / "paged_kv_gqa_store_amd" / "csrc"
    for name in KERNEL_SOURCES:
        h.update((csrc / name).read_bytes())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--workload", default=HEADLINE, help="headline workload (default: the largest, ragged_batch)")
    ap.add_argument("--workloads", default=",".join(ALL_WORKLOADS),
                    help="workloads measured one by one (comma-separated)")
    ap.add_argument("--layers", type=int, default=3, help="pool copies rotated over consecutive steps")
    ap.add_argument("--reps", type=int, default=20, help="graph replays per measured call")
    ap.add_argument("--calls", type=int, default=10, help="calls captured back to back per graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the secondary rows (prefill, rotary store and attention, embedding gather)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (a known-size reference "
                         "for the HBM byte counters of a profiler run)")
    return ap.parse_args()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def graph_replays(fn, calls: int, reps: int) -> np.ndarray:
    """µs per call of ``fn``: ``calls`` calls (fn(0) .. fn(calls-1)) captured back
    to back in one HIP graph, replayed ``reps`` times with HIP events around each
    replay on the current stream (the stream the library launches on).  The
    replays are enqueued without host synchronisation between them, so the GPU
    never waits for the host inside a timed interval.  Returns one per-call mean
    per replay."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for i in range(calls):           # eager pass first: code objects load outside capture
            fn(i)
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            for i in range(calls):
                fn(i)
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    out = np.array([e0.elapsed_time(e1) * 1e3 / calls for e0, e1 in ev])
    del g
    return out


def stats(us: np.ndarray) -> dict:
    """median, interquartile mean (mean of the middle half) and mean of µs samples."""
    a = np.sort(np.asarray(us, np.float64))
    q = len(a) // 4
    mid = a[q:len(a) - q] if len(a) >= 4 else a
    return {"median": round(float(np.median(a)), 3), "iqm": round(float(mid.mean()), 3),
            "mean": round(float(a.mean()), 3), "min": round(float(a[0]), 3), "n": int(len(a))}


def gbps(nbytes: int, us: float) -> float:
    return nbytes / (us * 1e-6) / 1e9


def pct(nbytes: int, us: float) -> float:
    return round(100 * gbps(nbytes, us) / PEAK_HBM_GBPS, 2)


class DeviceInputs:
    """One workload's inputs resident on the GPU, with rotated pool copies."""

    def __init__(self, inp, dev, layers):
        import torch
        self.inp, self.cfg, self.dev = inp, inp.cfg, dev
        self.q = self.bf16(inp.q)
        self.k_new, self.v_new = self.bf16(inp.k_new), self.bf16(inp.v_new)
        self.page_table, self.seq_lens = self.i32(inp.page_table), self.i32(inp.seq_lens)
        self.slots = self.i32(inp.slot_mapping)
        k0, v0 = self.bf16(inp.k_pool), self.bf16(inp.v_pool)
        self.pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(layers - 1)]
        torch.cuda.synchronize()

    def bf16(self, a):
        import torch
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.dev).view(torch.bfloat16)

    def i32(self, a):
        import torch
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.dev)

    def pool(self, i):
        return self.pools[i % len(self.pools)]


def load_workload(name, args, dev, W):
    cfg = W.WORKLOADS[name]
    t = time.perf_counter()
    inp = W.make_inputs(cfg)
    d = DeviceInputs(inp, dev, args.layers)
    log(f"[bench] {name}: {cfg.describe()} (inputs {time.perf_counter() - t:.1f} s)")
    return inp, d


def measure_workload(name, args, dev, pkv, W, blib, loaded=None):
    """Every per-workload figure of one decode workload (see the module docstring)."""
    import torch
    cfg = W.WORKLOADS[name]
    inp, d = load_workload(name, args, dev, W) if loaded is None else loaded
    B, Hq, Hkv, D, P = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.P
    L, total = inp.max_seq_len, int(inp.seq_lens.sum())
    S = pkv.num_splits(B, Hq, Hkv, L, P, total)
    o_p, l_p = pkv.workspace(B, Hq, D, S, dev)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    n, R = args.calls, args.reps
    kv_b = W.kv_bytes(inp.seq_lens, Hkv, D)
    terms = W.attention_bytes(inp.seq_lens, Hq, Hkv, D, P, S)
    # bytes pkv_paged_decode_attn's kernel must move: K+V, q, page ids and
    # lengths, and the fp32 partials it writes (once; the merge reads them)
    attn_kernel_b = terms["kv"] + terms["q"] + terms["page_ids"] + terms["partials"] // 2

    am = graph_replays(lambda i: pkv.paged_decode_attn_merged(
        d.q, *d.pool(i), d.page_table, d.seq_lens, L, S, out=out, o_partial=o_p, lse_partial=l_p), n, R)
    ak = graph_replays(lambda i: pkv.paged_decode_attn(
        d.q, *d.pool(i), d.page_table, d.seq_lens, L, S, o_partial=o_p, lse_partial=l_p), n, R)
    mg = graph_replays(lambda i: pkv.decode_merge(o_p, l_p, out=out), n, R) if S > 1 else None
    fs = graph_replays(lambda i: pkv.decode_step_fused(
        d.q, d.k_new, d.v_new, *d.pool(i), d.page_table, d.seq_lens, d.slots, L, S, out=out,
        o_partial=o_p, lse_partial=l_p), n, R)
    ss = graph_replays(lambda i: pkv.kv_store(*d.pool(i), d.k_new, d.v_new, d.slots), n, R)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all(), f"{name}: non-finite decode output"

    # kv_store bandwidth on the bulk fill of every position, beside the two
    # copy ceilings of the same bytes
    k_rows, v_rows, bslots = W.bulk_fill_rows(inp)
    src_row, dst_slot, run_rows = W.bulk_fill_runs(inp)
    kr, vr, bs = d.bf16(k_rows), d.bf16(v_rows), d.i32(bslots)
    rs, rd, rr = d.i32(src_row), d.i32(dst_slot), d.i32(run_rows)
    del k_rows, v_rows
    nrow, row_b = bslots.shape[0], cfg.row_elems * 2
    store_b = W.store_bytes(nrow, row_b)
    n_slots = cfg.num_pages * P
    stream = lambda: torch.cuda.current_stream().cuda_stream
    bulk = graph_replays(lambda i: pkv.kv_store(*d.pool(i), kr, vr, bs), 3, R)

    def runs(i):
        kp, vp = d.pool(i)
        st = blib.pkvb_copy_page_runs(kp.data_ptr(), vp.data_ptr(), n_slots, kr.data_ptr(), vr.data_ptr(),
                                      nrow, rs.data_ptr(), rd.data_ptr(), rr.data_ptr(), rr.shape[0], row_b,
                                      stream())
        assert st == 0, st

    same = graph_replays(runs, 3, R)
    src = torch.cat([kr.reshape(-1), vr.reshape(-1)])
    dst = torch.empty_like(src)
    lin_b = src.numel() * 2

    def linear(i):
        assert blib.pkvb_copy_linear(dst.data_ptr(), src.data_ptr(), lin_b, stream()) == 0

    lin = graph_replays(linear, 3, R)
    del src, dst, kr, vr, bs

    am_s, ak_s, fs_s, ss_s = stats(am), stats(ak), stats(fs), stats(ss)
    bulk_s, same_s, lin_s = stats(bulk), stats(same), stats(lin)
    res = {
        "shape": cfg.describe(), "num_splits": S, "chunk": pkv.split_chunk(L, S, P),
        "total_tokens": total, "kv_bytes": kv_b,
        "attn_merge_us": am_s,
        "attn_merge_GBps": round(gbps(kv_b, am_s["median"]), 1),
        "attn_merge_pct_of_peak": pct(kv_b, am_s["median"]),
        "attn_kernel_us": ak_s, "attn_kernel_algorithmic_bytes": attn_kernel_b,
        "attn_kernel_pct_of_peak": pct(attn_kernel_b, ak_s["mean"]),
        "merge_us": None if mg is None else stats(mg),
        "fused_step_us": fs_s,
        "fused_step_pct_of_peak": pct(kv_b, fs_s["median"]),
        "store_step_us": ss_s, "store_step_rows": B,
        "store_bulk_us": bulk_s, "store_bulk_rows": nrow, "store_bulk_bytes": store_b,
        "store_bulk_GBps": round(gbps(store_b, bulk_s["median"]), 1),
        "store_bulk_pct_of_peak": pct(store_b, bulk_s["median"]),
        "copy_same_pattern_GBps": round(gbps(store_b - 4 * nrow, same_s["median"]), 1),
        "copy_same_pattern_pct_of_peak": pct(store_b - 4 * nrow, same_s["median"]),
        "copy_linear_GBps": round(gbps(2 * lin_b, lin_s["median"]), 1),
        "copy_linear_pct_of_peak": pct(2 * lin_b, lin_s["median"]),
        "store_vs_same_pattern_copy": round(gbps(store_b, bulk_s["median"]) /
                                            gbps(store_b - 4 * nrow, same_s["median"]), 4),
    }
    log(f"[bench] {name}: S={S} | attn+merge {am_s['median']:.1f} us (iqm {am_s['iqm']:.1f}) "
        f"= {res['attn_merge_pct_of_peak']:.1f}% | attn kernel {ak_s['mean']:.1f} us | fused step "
        f"{fs_s['median']:.1f} us | step store {ss_s['median']:.1f} us")
    log(f"[bench] {name}: bulk store {bulk_s['median']:.1f} us = {res['store_bulk_pct_of_peak']:.1f}% | "
        f"same-pattern copy {res['copy_same_pattern_pct_of_peak']:.1f}% | linear copy "
        f"{res['copy_linear_pct_of_peak']:.1f}% | store / same-pattern copy {res['store_vs_same_pattern_copy']:.3f}")
    return res, inp, d, S


def measure_extras(args, pkv, W, dev) -> dict:
    """Secondary rows of the path, each on its own synthetic workload, graph-timed."""
    import torch
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    extras = {}
    for name in ("llama3_8b_chunked", "llama3_8b_fresh", "mha_fresh"):
        pcfg = W.PREFILL[name]
        q, kp, vp, pt, kl, qo = W.make_prefill_inputs(pcfg)
        plan = pkv.prefill_plan(np.diff(qo), dev)
        qd, kd, vd, ptd, kld = bf(q), bf(kp), bf(vp), i32(pt), i32(kl)
        out = torch.empty_like(qd)
        s = stats(graph_replays(lambda i: pkv.paged_prefill_attn(qd, kd, vd, ptd, kld, plan, out=out),
                                args.calls, args.reps))
        flops = W.prefill_flops(pcfg.q_lens, pcfg.kv_lens, pcfg.Hq, pcfg.D, causal=True)
        tflops = flops / (s["median"] * 1e-6) / 1e12
        extras["prefill_" + name] = {
            "op": "paged_prefill_attn (causal)", "us": s, "TFLOPs": round(tflops, 1),
            "pct_of_bf16_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), "flops": flops,
            "shape": pcfg.describe()}
        log(f"[bench] prefill {name}: {s['median']:.1f} us, {tflops:.0f} TFLOP/s "
            f"({tflops / PEAK_BF16_TFLOPS:.1%} of {PEAK_BF16_TFLOPS:.0f} bf16 dense)")
        del qd, kd, vd, out
    for name in ("llama3_8b_embed_prefill", "llama3_8b_embed_decode"):
        icfg = W.INDEXING[name]
        table, ids, start = W.make_indexing_inputs(icfg, rank=0)
        t_d, ids_d = bf(table), i32(ids)
        out = torch.empty((icfg.n, icfg.hidden), dtype=torch.bfloat16, device=dev)
        s = stats(graph_replays(lambda i: pkv.indexing(t_d, ids_d, start, out=out), args.calls, args.reps))
        nbytes = W.indexing_bytes(ids, start, table.shape[0], icfg.hidden * 2)
        extras[name] = {"op": "indexing", "us": s, "GBps": round(gbps(nbytes, s["median"]), 1),
                        "pct_of_peak": pct(nbytes, s["median"]), "bytes": nbytes,
                        "shape": f"slice {table.shape[0]}x{icfg.hidden} bf16 (1/{icfg.shards} of "
                                 f"{icfg.vocab}), {icfg.n} ids"}
        log(f"[bench] indexing {name}: {s['median']:.1f} us, {extras[name]['pct_of_peak']:.1f}% of peak")
        del t_d, ids_d, out
    return extras


def measure_rope(args, pkv, W, inp, d, S) -> dict:
    """The store with K rotated on the way (bulk fill) and the attention with q
    rotated in its prologue, at the headline workload."""
    import torch
    cfg = inp.cfg
    L = inp.max_seq_len
    positions = np.concatenate([np.arange(int(x), dtype=np.int32) for x in inp.seq_lens] + [np.zeros(0, np.int32)])
    c_t, s_t = W.rope_tables(L, cfg.D)
    cd, sd = torch.from_numpy(c_t).to(d.dev), torch.from_numpy(s_t).to(d.dev)
    pos_d = d.i32(positions)
    k_rows, v_rows, bslots = W.bulk_fill_rows(inp)
    k3, v3 = d.bf16(k_rows).view(-1, cfg.Hkv, cfg.D), d.bf16(v_rows).view(-1, cfg.Hkv, cfg.D)
    bs = d.i32(bslots)
    store_b = W.store_bytes(bslots.shape[0], cfg.row_elems * 2)
    rope_b = store_b + 4 * bslots.shape[0] + L * cfg.D * 4   # + positions, cos/sin tables once
    su = stats(graph_replays(lambda i: pkv.kv_store_rope(*d.pool(i), k3, v3, bs, pos_d, cd, sd), 3, args.reps))
    o_p, l_p = pkv.workspace(cfg.B, cfg.Hq, cfg.D, S, d.dev)
    qpos = d.i32(np.maximum(inp.seq_lens - 1, 0))
    au = stats(graph_replays(lambda i: pkv.paged_decode_attn(
        d.q, *d.pool(i), d.page_table, d.seq_lens, L, S, o_partial=o_p, lse_partial=l_p,
        q_positions=qpos, rope_cos=cd, rope_sin=sd), args.calls, args.reps))
    log(f"[bench] rope: bulk store {su['median']:.1f} us = {pct(rope_b, su['median']):.1f}%; "
        f"attention with rotated q {au['median']:.1f} us")
    return {"kv_store_rope_bulk_us": su, "kv_store_rope_bulk_pct_of_peak": pct(rope_b, su["median"]),
            "attn_rope_us": au}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this decode step has no multi-GPU path. It would shard "
              "by sequence or by kv head with no exchange, or by context with one all-gather of the "
              "(o, lse) partials before the merge. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_gqa_store_amd as pkv
    from paged_kv_gqa_store_amd import _lib
    from paged_kv_gqa_store_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    blib = _lib.bench_lib()
    names = [w for w in args.workloads.split(",") if w]
    if args.workload not in names:
        names.append(args.workload)
    for w in names:
        if w not in W.WORKLOADS:
            raise SystemExit(f"unknown workload {w}; known: {', '.join(W.WORKLOADS)}")

    # The headline first: its K timed steps right after its inputs are resident,
    # then its per-workload figures, then the other workloads.
    names = [args.workload] + [w for w in names if w != args.workload]
    per_wl = {}
    inp, d = load_workload(args.workload, args, dev, W)

    # ---- the headline: W untimed steps, then exactly K steps (eager, then one graph replay)
    cfg = inp.cfg
    L = inp.max_seq_len
    S = pkv.num_splits(cfg.B, cfg.Hq, cfg.Hkv, L, cfg.P, int(inp.seq_lens.sum()))
    kv_b = W.kv_bytes(inp.seq_lens, cfg.Hkv, cfg.D)
    o_p, l_p = pkv.workspace(cfg.B, cfg.Hq, cfg.D, S, dev)
    out = torch.empty((cfg.B, cfg.Hq, cfg.D), dtype=torch.bfloat16, device=dev)

    def step(i):
        pkv.decode_step_fused(d.q, d.k_new, d.v_new, *d.pool(i), d.page_table, d.seq_lens, d.slots, L, S,
                              out=out, o_partial=o_p, lse_partial=l_p)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    from paged_kv_gqa_store_amd.graph import StepGraph
    g = StepGraph([d.pool(i) for i in range(args.steps)], d.q, d.k_new, d.v_new, d.page_table, d.seq_lens,
                  d.slots, L, S)
    g.replay()                          # untimed replay
    torch.cuda.synchronize()
    ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ge0.record()
    g.replay()
    ge1.record()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = ge0.elapsed_time(ge1) / args.steps
    assert all(torch.isfinite(o.float()).all() for o in g.outputs[-len(d.pools):]), "non-finite output"
    del g
    log(f"[bench] headline {cfg.name}: {args.steps} steps in one graph replay, {ms_per_step * 1e3:.1f} us per "
        f"step (wall; events {ev_ms * 1e3:.1f} us), {eager_ms * 1e3:.1f} us eager")

    res, _, _, _ = measure_workload(args.workload, args, dev, pkv, W, blib, loaded=(inp, d))
    per_wl[args.workload] = res
    h = per_wl[args.workload]
    attn_us = h["attn_kernel_us"]["mean"]
    traffic = None
    if (COUNTED_TRAFFIC["workload"] == args.workload and COUNTED_TRAFFIC["sources_sha256"] == kernel_sources_sha256()
            and COUNTED_TRAFFIC["read_bytes"] is not None):
        traffic = COUNTED_TRAFFIC["read_bytes"] + COUNTED_TRAFFIC["write_bytes"]
    achieved = gbps(h["attn_kernel_algorithmic_bytes"], attn_us)

    rope_info = None
    if not args.no_extras:
        rope_info = measure_rope(args, pkv, W, inp, d, S)
    del d
    torch.cuda.empty_cache()

    for name in names[1:]:
        res, inp_o, d_o, _ = measure_workload(name, args, dev, pkv, W, blib)
        per_wl[name] = res
        del inp_o, d_o
        torch.cuda.empty_cache()
    per_wl = {w: per_wl[w] for w in ALL_WORKLOADS if w in per_wl} | {w: v for w, v in per_wl.items()
                                                                    if w not in ALL_WORKLOADS}

    result = {
        "metric": "paged decode attn µs/step + achieved HBM GB/s (% of peak); kv_store GB/s",
        "value": round(kv_b / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name} (decode step: kv_store + split-KV paged attention + merge; "
                        f"the largest of the five decode workloads on one GPU)",
            "batch": cfg.B, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv, "head_dim": cfg.D, "page_size": cfg.P,
            "seq_len": cfg.seq_len if cfg.seq_len else f"ragged U{{1..{cfg.ragged_max}}}, sum {h['total_tokens']}",
            "pool_pages": cfg.num_pages, "num_splits": S, "layers_rotated": args.layers,
            "launch": f"hip_graph ({args.steps} pkv_decode_step calls per replay)",
        },
        "value_definition": "K+V bytes read per step / time per step of the whole step (kv_store fused into "
                            "the attention kernel, then the merge); K steps in one HIP graph replay",
        "kv_bytes_per_step": kv_b,
        "eager_ms_per_step": round(eager_ms, 5),
        "graph_event_ms_per_step": round(ev_ms, 5),
        "attn_us_per_step": h["attn_merge_us"]["median"],
        "attn_kv_GBps": h["attn_merge_GBps"],
        "attn_pct_of_peak": h["attn_merge_pct_of_peak"],
        "attn_pct_definition": "K+V bytes / graph-timed median of attention + merge (pkv_paged_decode_attn_merged)",
        "kv_store_bulk_GBps": h["store_bulk_GBps"],
        "kv_store_bulk_pct_of_peak": h["store_bulk_pct_of_peak"],
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_decode_mfma_kernel (pkv_paged_decode_attn, split-KV attention)",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": h["attn_kernel_algorithmic_bytes"],
            "duration_us": round(attn_us, 3),
            "duration_from": f"HIP events around {args.reps} replays of a graph of {args.calls} back-to-back "
                             f"launches (mean per launch)",
        },
        "workloads": per_wl,
    }
    if rope_info is not None:
        result["rope"] = rope_info
    if not args.no_extras:
        result["extras"] = measure_extras(args, pkv, W, dev)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 1 GiB read + 1 GiB written by one copy kernel")
        del src, dst

    if not args.no_cpu_baseline:
        from oracle import oracle
        kf, vf = inp.pools_after_store()
        flat = lambda a: a.reshape(cfg.num_pages * cfg.P, cfg.row_elems)
        reps, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and reps < 1000:
            t = time.perf_counter()
            oracle.kv_store(flat(inp.k_pool), flat(inp.v_pool), inp.k_new, inp.v_new, inp.slot_mapping)
            oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)
            t_cpu += time.perf_counter() - t
            reps += 1
        result["cpu_baseline"] = {
            "value": round(kv_b * reps / t_cpu / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{reps} whole {cfg.name} steps (oracle store + fp64 attention), {t_cpu:.1f} s on "
                      f"{cpu_model()}",
            "ms_per_step": round(t_cpu / reps * 1e3, 2),
        }
        log(f"[bench] oracle: {t_cpu / reps * 1e3:.1f} ms/step on {oracle.num_threads()} threads")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
