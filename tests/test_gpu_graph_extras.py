"""The secondary rows inside a HIP graph, as bench.py times them: the paged
prefill, the row gather and the store with rotary embedding, each captured
once and replayed three times with eager work and synchronisations between
the replays; every replay must equal the eager call bit for bit."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import bf16_dev, i32_dev

pytestmark = pytest.mark.gpu


def capture(fn):
    """fn() once eagerly on a side stream (code objects load outside capture),
    then captured into a graph on that stream."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def replay_and_check(g, outputs, eager, what):
    for rep in range(3):
        for t in outputs:
            t.view(torch.uint8).fill_(0xAB)          # poison: a replay must rewrite every byte
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = (torch.arange(4096, device=outputs[0].device) * 3).sum().item()   # eager work between replays
        for t, e in zip(outputs, eager):
            assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), f"{what}: replay {rep} differs"


@pytest.mark.parametrize("name", ["ragged_chunks", "llama3_8b_fresh"])
def test_prefill_replays_equal_eager(gpu_device, name):
    cfg = W.PREFILL[name]
    print(f"prefill in a graph: {cfg.describe()}", flush=True)
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    plan = pkv.prefill_plan(np.diff(qo), gpu_device)
    qd, kd, vd, ptd, kld = (bf16_dev(q, gpu_device), bf16_dev(kp, gpu_device), bf16_dev(vp, gpu_device),
                            i32_dev(pt, gpu_device), i32_dev(kl, gpu_device))
    eager_out, eager_lse = pkv.paged_prefill_attn(qd, kd, vd, ptd, kld, plan, want_lse=True)
    out = torch.empty_like(eager_out)
    held = {}

    def call():   # the lse of the captured call lives in the graph's memory pool
        held["r"] = pkv.paged_prefill_attn(qd, kd, vd, ptd, kld, plan, out=out, want_lse=True)

    g = capture(call)
    replay_and_check(g, [out, held["r"][1]], [eager_out.clone(), eager_lse.clone()], f"prefill {name}")


def test_indexing_replays_equal_eager(gpu_device):
    icfg = W.IndexingConfig("graph_gather", 16000, 1024, 4, 5000)
    table, ids, start = W.make_indexing_inputs(icfg, rank=1)
    t_d, ids_d = bf16_dev(table, gpu_device), torch.from_numpy(ids).to(gpu_device)
    eager = pkv.indexing(t_d, ids_d, start)
    out = torch.empty_like(eager)
    g = capture(lambda: pkv.indexing(t_d, ids_d, start, out=out))
    replay_and_check(g, [out], [eager.clone()], "indexing")


def test_store_rope_replays_equal_eager(gpu_device):
    inp = W.make_inputs(W.WORKLOADS["llama3_8b_decode"])
    cfg = inp.cfg
    k_rows, v_rows, slots = W.bulk_fill_rows(inp)
    n = 20000
    k_rows, v_rows, slots = k_rows[:n], v_rows[:n], slots[:n]
    positions = np.arange(n, dtype=np.int32) % 4096
    c, s = W.rope_tables(4096, cfg.D)
    cd, sd = torch.from_numpy(c).to(gpu_device), torch.from_numpy(s).to(gpu_device)
    kr = bf16_dev(k_rows, gpu_device).view(-1, cfg.Hkv, cfg.D)
    vr = bf16_dev(v_rows, gpu_device).view(-1, cfg.Hkv, cfg.D)
    sl, pos = i32_dev(slots, gpu_device), i32_dev(positions, gpu_device)
    kp0, vp0 = bf16_dev(inp.k_pool, gpu_device), bf16_dev(inp.v_pool, gpu_device)
    ek, ev = kp0.clone(), vp0.clone()
    pkv.kv_store_rope(ek, ev, kr, vr, sl, pos, cd, sd)
    kp, vp = kp0.clone(), vp0.clone()
    g = capture(lambda: pkv.kv_store_rope(kp, vp, kr, vr, sl, pos, cd, sd))
    for rep in range(3):
        kp.copy_(kp0)
        vp.copy_(vp0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(kp.view(torch.int16), ek.view(torch.int16)), f"store rope K: replay {rep}"
        assert torch.equal(vp.view(torch.int16), ev.view(torch.int16)), f"store rope V: replay {rep}"
