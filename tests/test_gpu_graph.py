"""The graph-captured multi-layer step: every replay, with eager work and
synchronisations between replays, must equal the eager step bit for bit
(the kernels are deterministic), pools included."""
import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W
from paged_kv_gqa_store_amd.graph import StepGraph

from .gpu_util import DeviceStep, bf16_dev, check_attention

pytestmark = pytest.mark.gpu


def _layer_inputs(inp, n_layers, dev):
    """Per-layer inputs over the same sequences (one page table, one slot
    mapping): layer l draws its own q and rolls K/V along the head dimension by
    l, which keeps every NaN canary where it was."""
    layers = []
    for layer in range(n_layers):
        rng = np.random.Generator(np.random.PCG64(inp.seed + 1000 * (layer + 1)))
        q = W.to_bf16_bits(rng.standard_normal(inp.q.shape).astype(np.float32))
        roll = lambda a: np.ascontiguousarray(np.roll(a, layer, axis=-1))
        kf, vf = inp.pools_after_store()
        D = inp.cfg.D
        rows = lambda a: roll(a.reshape(a.shape[0], -1, D)).reshape(a.shape)
        layers.append(dataclasses.replace(
            inp, q=q, k_pool=roll(inp.k_pool), v_pool=roll(inp.v_pool),
            k_new=rows(inp.k_new), v_new=rows(inp.v_new),
            extra={**inp.extra, "k_full": roll(kf), "v_full": roll(vf)}))
    return layers


@pytest.mark.parametrize("wl,n_layers,splits,fused", [("tiny_gqa", 3, 2, True), ("ragged_batch", 2, None, True), ("llama3_8b_decode", 2, 1, True),
                                                      ("tiny_gqa", 2, 2, False), ("llama3_8b_decode", 2, 1, False)])
def test_replays_equal_the_eager_step(gpu_device, wl, n_layers, splits, fused):
    base = W.make_inputs(W.WORKLOADS[wl])
    layers = _layer_inputs(base, n_layers, gpu_device)
    total = int(base.seq_lens.sum())
    print(f"graph step {wl}, {n_layers} layers, splits {splits}, fused {fused}", flush=True)
    # graph side: one set of device tensors per layer (page table, lengths, slots shared)
    dsteps = [DeviceStep(li, gpu_device) for li in layers]
    shared = dsteps[0]
    g = StepGraph([(d.k_pool, d.v_pool) for d in dsteps], [d.q for d in dsteps],
                  [d.k_new for d in dsteps], [d.v_new for d in dsteps], shared.page_table,
                  shared.seq_lens, shared.slot_mapping, base.max_seq_len, splits, total, fused=fused)
    # eager side: fresh copies of the same inputs
    esteps = [DeviceStep(li, gpu_device) for li in layers]
    eager = [e.step(g.splits)[0] for e in esteps]
    torch.cuda.synchronize()
    for rep in range(3):
        outs = g.replay()
        torch.cuda.synchronize()
        for layer in range(n_layers):
            assert torch.equal(outs[layer].view(torch.int16), eager[layer].view(torch.int16)), (rep, layer)
            assert torch.equal(dsteps[layer].k_pool.view(torch.int16), esteps[layer].k_pool.view(torch.int16))
            assert torch.equal(dsteps[layer].v_pool.view(torch.int16), esteps[layer].v_pool.view(torch.int16))
        # eager work between replays: an unrelated step on the eager copies, then a sync
        esteps[0].attend(g.splits)
        torch.cuda.synchronize()
    # and the replayed result is the oracle's
    kf, vf = layers[-1].pools_after_store()
    ref, _ = oracle.paged_decode(layers[-1].q, kf, vf, layers[-1].page_table, layers[-1].seq_lens)
    check_attention(g.outputs[-1], ref, f"graph {wl}")


def test_replay_follows_inputs_refilled_in_place(gpu_device):
    """Static buffers: new q written in place between replays is what the next replay reads."""
    inp = W.make_inputs(W.WORKLOADS["tiny_gqa"])
    d = DeviceStep(inp, gpu_device)
    g = StepGraph([(d.k_pool, d.v_pool)], d.q, d.k_new, d.v_new, d.page_table, d.seq_lens,
                  d.slot_mapping, inp.max_seq_len, 2)
    first = g.replay()[0].clone()
    rng = np.random.Generator(np.random.PCG64(3))
    q2 = W.to_bf16_bits(rng.standard_normal(inp.q.shape).astype(np.float32))
    d.q.copy_(bf16_dev(q2, gpu_device))
    second = g.replay()[0]
    torch.cuda.synchronize()
    assert not torch.equal(first, second)
    kf, vf = inp.pools_after_store()
    ref, _ = oracle.paged_decode(q2, kf, vf, inp.page_table, inp.seq_lens)
    check_attention(second, ref, "graph after q refill")
