#!/usr/bin/env python3
"""Benchmark of one decode step of GQA over a paged KV cache on one MI355X.

A step is the whole path over one batch: kv_store of the batch's new rows,
split-KV paged attention, log-sum-exp merge.  The default workload is the
Llama-3-8B-shaped decode batch (B=32, 32 q / 8 kv heads, D=128, bf16,
page_size 16, seq_len 4096, 9000-page pool, shuffled page table).

Timing: W untimed steps, then exactly K steps launched one kernel at a time
between two device synchronisations, with HIP events around every kernel (on
the stream the kernels run on) for the per-kernel figures and the roofline.
Then the same K steps are captured into one HIP graph, replayed once untimed
and once timed between synchronisations: that replay gives `ms_per_step` and
`value` (``--eager`` reports the kernel-at-a-time loop instead).  Consecutive
steps read different copies of the pool ("layers"), so no step finds the
previous step's K/V in the 256 MB Infinity Cache.  Prints ONE JSON line on
stdout; details go to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--eager] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak, published

# HBM bytes per launch of the decode kernel on the default workload, counted by
# rocprofv3 in two runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each
# scaled by what the same counter reads for a 1 GiB device-to-device copy
# (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).  Keyed by the sha256 of the kernel's
# sources when the counters were taken: any edit to them voids the figure.
COUNTED_TRAFFIC = {
    "workload": "llama3_8b_decode",
    "sources_sha256": "3dbaaa07e16ffd896ca51ed4f180da3e95cbcfd920c90a51b25c8283d4c5d00f",
    "read_bytes": 537616869,    # FETCH_SIZE 262517.8 KiB x (1 GiB / 524307.1 KiB)
    "write_bytes": 532480,      # WRITE_SIZE 520.0 KiB x (1 GiB / 1048576.0 KiB)
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
    ap.add_argument("--workload", default="llama3_8b_decode",
                    help="tiny_gqa, llama3_8b_decode (default), ragged_batch, long_context or mha_page1")
    ap.add_argument("--layers", type=int, default=3, help="pool copies rotated over consecutive steps")
    ap.add_argument("--splits", type=int, default=None, help="override the split heuristic")
    ap.add_argument("--kernel", choices=["mfma", "valu"], default="mfma",
                    help="decode kernel: matrix-core QK^T (default) or all-VALU")
    ap.add_argument("--store-reps", type=int, default=20, help="timed bulk-fill kv_store launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--eager", action="store_true",
                    help="report the eagerly launched steps instead of one graph replay of K steps")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the secondary measurements (rotary store and attention, prefill, "
                         "embedding row gather)")
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


def time_launches(fn, reps: int, warmup: int = 3) -> float:
    """Mean µs per call of ``fn`` over ``reps`` back-to-back calls, from HIP
    events on the current stream (the stream the library launches on)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def time_graph_launches(fn, n: int) -> float:
    """Mean µs per call of ``fn`` over ``n`` calls captured back to back in one
    HIP graph, from HIP events around its replay on the current stream: the
    kernel's duration without the per-launch dispatch gap of eager launches."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for i in range(n):               # eager pass first: code objects load outside capture
            fn(i)
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                fn(i)
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / n


def measure_copy_ceiling(dev, reps: int = 10) -> float:
    """GB/s of a plain 16-byte-vector device copy of 1 GiB (bytes read + written),
    the practical ceiling of a read+write move such as kv_store on this machine."""
    import torch
    src = torch.ones(1 << 27, dtype=torch.int64, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        dst.copy_(src)
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
    del src, dst
    return 2 * (1 << 30) / (ms * 1e-3) / 1e9


def measure_extras(args, pkv, W, dev, to_bf16, to_i32) -> dict:
    """Secondary rows of the path, each on its own synthetic workload."""
    import torch
    extras = {}
    for name in ("llama3_8b_chunked", "llama3_8b_fresh", "mha_fresh"):
        pcfg = W.PREFILL[name]
        q, kp, vp, pt, kl, qo = W.make_prefill_inputs(pcfg)
        plan = pkv.prefill_plan(np.diff(qo), dev)
        qd, kd, vd, ptd, kld = to_bf16(q), to_bf16(kp), to_bf16(vp), to_i32(pt), to_i32(kl)
        out = torch.empty_like(qd)
        us = time_launches(lambda i: pkv.paged_prefill_attn(qd, kd, vd, ptd, kld, plan, out=out), reps=20)
        flops = W.prefill_flops(pcfg.q_lens, pcfg.kv_lens, pcfg.Hq, pcfg.D, causal=True)
        tflops = flops / (us * 1e-6) / 1e12
        extras["prefill_" + name] = {
            "op": "paged_prefill_attn (causal)", "us": round(us, 2), "TFLOPs": round(tflops, 1),
            "pct_of_bf16_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), "flops": flops,
            "shape": pcfg.describe()}
        log(f"[bench] prefill {name}: {us:.1f} us, {tflops:.0f} TFLOP/s "
            f"({tflops / PEAK_BF16_TFLOPS:.1%} of {PEAK_BF16_TFLOPS:.0f} bf16 dense)")
        del qd, kd, vd, out
    for name in ("llama3_8b_embed_prefill", "llama3_8b_embed_decode"):
        icfg = W.INDEXING[name]
        table, ids, start = W.make_indexing_inputs(icfg, rank=0)
        t_d, ids_d = to_bf16(table), to_i32(ids)
        out = torch.empty((icfg.n, icfg.hidden), dtype=torch.bfloat16, device=dev)
        us = time_launches(lambda i: pkv.indexing(t_d, ids_d, start, out=out), reps=20)
        nbytes = W.indexing_bytes(ids, start, table.shape[0], icfg.hidden * 2)
        gbps = nbytes / (us * 1e-6) / 1e9
        extras[name] = {"op": "indexing", "us": round(us, 2), "GBps": round(gbps, 1),
                        "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2), "bytes": nbytes,
                        "shape": f"slice {table.shape[0]}x{icfg.hidden} bf16 (1/{icfg.shards} of "
                                 f"{icfg.vocab}), {icfg.n} ids"}
        log(f"[bench] indexing {name}: {us:.1f} us, {gbps:.0f} GB/s ({gbps / PEAK_HBM_GBPS:.1%})")
        del t_d, ids_d, out
    return extras


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this decode step has no multi-GPU path. It would shard "
              "by sequence or by kv head with no exchange, or by context with one all-gather of the "
              "(o, lse) partials before the merge. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_gqa_store_amd as pkv
    from paged_kv_gqa_store_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cfg = W.WORKLOADS[args.workload]
    log(f"[bench] workload {cfg.name}: {cfg.describe()}")
    t = time.perf_counter()
    inp = W.make_inputs(cfg)
    log(f"[bench] inputs drawn in {time.perf_counter() - t:.1f} s")

    to_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    to_i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    q = to_bf16(inp.q)
    k_new, v_new = to_bf16(inp.k_new), to_bf16(inp.v_new)
    page_table, seq_lens, slots = to_i32(inp.page_table), to_i32(inp.seq_lens), to_i32(inp.slot_mapping)
    k0, v0 = to_bf16(inp.k_pool), to_bf16(inp.v_pool)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(args.layers - 1)]
    B, Hq, Hkv, D, P = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.P
    max_len = inp.max_seq_len
    S = args.splits or pkv.num_splits(B, Hq, Hkv, max_len, P, int(inp.seq_lens.sum()))
    o_p, l_p = pkv.workspace(B, Hq, D, S, dev)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    log(f"[bench] num_splits {S}, chunk {pkv.split_chunk(max_len, S, P)}, layers {args.layers}")

    def step(i, ev=None):
        kp, vp = pools[i % len(pools)]
        if ev is not None:
            ev[0].record()
        pkv.kv_store(kp, vp, k_new, v_new, slots)
        if ev is not None:
            ev[1].record()
        pkv.paged_decode_attn(q, kp, vp, page_table, seq_lens, max_len, S, o_partial=o_p, lse_partial=l_p,
                              kernel=args.kernel)
        if ev is not None:
            ev[2].record()
        pkv.decode_merge(o_p, l_p, out=out)
        if ev is not None:
            ev[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    store_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    attn_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    merge_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    ms_per_step = wall * 1e3 / args.steps
    assert torch.isfinite(out.float()).all(), "non-finite decode output"

    kv_b = W.kv_bytes(inp.seq_lens, Hkv, D)
    terms = W.attention_bytes(inp.seq_lens, Hq, Hkv, D, P, S)
    # bytes the attention kernel itself must move: K+V, q, page ids, partials written once
    attn_kernel_b = terms["kv"] + terms["q"] + terms["page_ids"] + terms["partials"] // 2
    attn_us = float(attn_ms.mean() * 1e3)
    traffic = None
    if (cfg.name == COUNTED_TRAFFIC["workload"] and args.splits is None and args.kernel == "mfma"
            and COUNTED_TRAFFIC["sources_sha256"] == kernel_sources_sha256()):
        traffic = COUNTED_TRAFFIC["read_bytes"] + COUNTED_TRAFFIC["write_bytes"]
    achieved = attn_kernel_b / (attn_us * 1e-6) / 1e9
    log(f"[bench] step {ms_per_step * 1e3:.1f} us (wall) | store {store_ms.mean() * 1e3:.1f} us | "
        f"attn {attn_us:.1f} us (median {np.median(attn_ms) * 1e3:.1f}) | merge {merge_ms.mean() * 1e3:.1f} us")
    log(f"[bench] attention kernel {achieved:.0f} GB/s = {achieved / PEAK_HBM_GBPS:.1%} of {PEAK_HBM_GBPS:.0f} GB/s")

    # The same K steps captured into one HIP graph (each step on its own pool
    # copy, rotating as above) and replayed once: the launch mode of a decode
    # server, and the figure `value` and `ms_per_step` report unless --eager.
    eager_ms_per_step = ms_per_step
    launch = "eager"
    attn_graph_us = None
    if not args.eager:
        from paged_kv_gqa_store_amd.graph import StepGraph
        g = StepGraph([pools[i % len(pools)] for i in range(args.steps)], q, k_new, v_new,
                      page_table, seq_lens, slots, max_len, S)
        g.replay()                       # warm-up replay (K more untimed steps)
        torch.cuda.synchronize()
        ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ge0.record()
        g.replay()
        ge1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / args.steps
        assert all(torch.isfinite(o.float()).all() for o in g.outputs[-len(pools):]), "non-finite output"
        log(f"[bench] graph-captured: {args.steps} steps in one replay, {ms_per_step * 1e3:.1f} us per step "
            f"(wall; events {ge0.elapsed_time(ge1) * 1e3 / args.steps:.1f} us) vs {eager_ms_per_step * 1e3:.1f} us eager")
        launch = f"hip_graph ({args.steps} steps per replay)"
        del g
        # the attention kernel alone, K launches back to back in one graph
        # (rotating pools as above): its average duration for the roofline
        attn_graph_us = time_graph_launches(lambda i: pkv.paged_decode_attn(
            q, pools[i % len(pools)][0], pools[i % len(pools)][1], page_table, seq_lens, max_len, S,
            o_partial=o_p, lse_partial=l_p, kernel=args.kernel), args.steps)
        achieved = attn_kernel_b / (attn_graph_us * 1e-6) / 1e9
        log(f"[bench] attention kernel alone, {args.steps} launches in one graph: {attn_graph_us:.1f} us per launch, "
            f"{achieved:.0f} GB/s = {achieved / PEAK_HBM_GBPS:.1%} of {PEAK_HBM_GBPS:.0f} GB/s")

    # kv_store bandwidth: bulk fill of every position (prefill-style), same kernel and ABI
    k_rows, v_rows, bslots = W.bulk_fill_rows(inp)
    k_rows_d, v_rows_d, bslots_d = to_bf16(k_rows), to_bf16(v_rows), to_i32(bslots)
    row_b = cfg.row_elems * 2
    store_b = W.store_bytes(bslots.shape[0], row_b)
    for i in range(3):
        kp, vp = pools[i % len(pools)]
        pkv.kv_store(kp, vp, k_rows_d, v_rows_d, bslots_d)
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.store_reps)]
    torch.cuda.synchronize()
    for i in range(args.store_reps):
        kp, vp = pools[i % len(pools)]
        sev[i][0].record()
        pkv.kv_store(kp, vp, k_rows_d, v_rows_d, bslots_d)
        sev[i][1].record()
    torch.cuda.synchronize()
    bulk_us = float(np.mean([a.elapsed_time(b) for a, b in sev]) * 1e3)
    store_gbps = store_b / (bulk_us * 1e-6) / 1e9
    log(f"[bench] kv_store bulk fill: {bslots.shape[0]} rows, {store_b / 1e6:.1f} MB in {bulk_us:.1f} us = "
        f"{store_gbps:.0f} GB/s ({store_gbps / PEAK_HBM_GBPS:.1%})")
    copy_gbps = measure_copy_ceiling(dev)
    log(f"[bench] device copy on this box (practical ceiling of a read+write move): {copy_gbps:.0f} GB/s "
        f"({copy_gbps / PEAK_HBM_GBPS:.1%}); kv_store bulk fill at {store_gbps / copy_gbps:.0%} of it")
    rope_info = None
    if not args.no_extras:
        # the same bulk fill through the store with rotary embedding of K, and the
        # attention with q rotated in its prologue
        positions = np.concatenate([np.arange(int(L), dtype=np.int32) for L in inp.seq_lens] +
                                   [np.zeros(0, np.int32)])
        c_t, s_t = W.rope_tables(max_len, D)
        cd, sd = torch.from_numpy(c_t).to(dev), torch.from_numpy(s_t).to(dev)
        pos_d = to_i32(positions)
        k3, v3 = k_rows_d.view(-1, Hkv, D), v_rows_d.view(-1, Hkv, D)
        us = time_launches(lambda i: pkv.kv_store_rope(pools[i % len(pools)][0], pools[i % len(pools)][1],
                                                       k3, v3, bslots_d, pos_d, cd, sd), reps=args.store_reps)
        rope_b = store_b + 4 * bslots.shape[0] + max_len * D * 4   # + positions, cos/sin tables once
        qpos = to_i32(np.maximum(inp.seq_lens - 1, 0))
        ua = time_launches(lambda i: pkv.paged_decode_attn(
            q, pools[i % len(pools)][0], pools[i % len(pools)][1], page_table, seq_lens, max_len, S,
            o_partial=o_p, lse_partial=l_p, q_positions=qpos, rope_cos=cd, rope_sin=sd), reps=30)
        ub = time_launches(lambda i: pkv.paged_decode_attn(
            q, pools[i % len(pools)][0], pools[i % len(pools)][1], page_table, seq_lens, max_len, S,
            o_partial=o_p, lse_partial=l_p), reps=30)
        rope_info = {
            "kv_store_rope_bulk_us": round(us, 2),
            "kv_store_rope_bulk_GBps": round(rope_b / (us * 1e-6) / 1e9, 1),
            "kv_store_rope_bulk_pct_of_peak": round(100 * rope_b / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2),
            "attn_rope_us": round(ua, 2), "attn_plain_us_same_loop": round(ub, 2),
        }
        log(f"[bench] kv_store_rope bulk fill: {us:.1f} us = {rope_b / (us * 1e-6) / 1e9:.0f} GB/s; "
            f"attention with q rotated in the prologue {ua:.1f} us vs {ub:.1f} us plain (back to back)")
        del cd, sd, pos_d
    del k_rows_d, v_rows_d, bslots_d

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
            "workload": f"{cfg.name} (decode step: kv_store + split-KV paged attention + merge)",
            "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "page_size": P,
            "seq_len": cfg.seq_len if cfg.seq_len else "ragged", "pool_pages": cfg.num_pages,
            "num_splits": S, "layers_rotated": len(pools), "decode_kernel": args.kernel,
            "launch": launch,
        },
        "eager_ms_per_step": round(eager_ms_per_step, 5),
        "value_definition": "K+V bytes read per step / wall time of the whole step (store + attention + merge); "
                            "the K timed steps run as one HIP graph replay unless launch says eager",
        "attn_us_per_step": round(attn_us + float(merge_ms.mean() * 1e3), 2),
        "attn_kernel_us": round(attn_us, 2),
        "attn_kernel_graph_us": None if attn_graph_us is None else round(attn_graph_us, 2),
        "merge_kernel_us": round(float(merge_ms.mean() * 1e3), 2),
        "store_step_us": round(float(store_ms.mean() * 1e3), 2),
        "attn_kv_GBps": round(kv_b / ((attn_us + merge_ms.mean() * 1e3) * 1e-6) / 1e9, 1),
        "attn_pct_of_peak": round(100 * kv_b / ((attn_us + merge_ms.mean() * 1e3) * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2),
        "kv_store_bulk_GBps": round(store_gbps, 1),
        "kv_store_bulk_pct_of_peak": round(100 * store_gbps / PEAK_HBM_GBPS, 2),
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "copy_ceiling_kernel": "torch copy_ of 1 GiB int64 to 1 GiB (read + write bytes counted), median of 10",
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_decode (split-KV attention)",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": attn_kernel_b,
            "duration_us": round(attn_us if attn_graph_us is None else attn_graph_us, 2),
            "duration_from": ("HIP events around each eager launch" if attn_graph_us is None else
                              f"HIP events around one graph of {args.steps} back-to-back launches"),
        },
    }

    if not args.no_extras:
        result["rope"] = rope_info
        result["extras"] = measure_extras(args, pkv, W, dev, to_bf16, to_i32)

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
        flat = lambda a: a.reshape(cfg.num_pages * P, cfg.row_elems)
        reps, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and reps < 1000:
            t = time.perf_counter()
            oracle.kv_store(flat(inp.k_pool), flat(inp.v_pool), inp.k_new, inp.v_new, inp.slot_mapping)
            oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)
            t_cpu += time.perf_counter() - t
            reps += 1
        cpu_gbps = kv_b * reps / t_cpu / 1e9
        result["cpu_baseline"] = {
            "value": round(cpu_gbps, 3), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the full {cfg.name} step (oracle store + fp64 attention), {reps} run(s), "
                      f"{t_cpu:.1f} s on {cpu_model()}",
            "ms_per_step": round(t_cpu / reps * 1e3, 2),
        }
        log(f"[bench] oracle: {t_cpu / reps * 1e3:.1f} ms/step on {oracle.num_threads()} threads")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
