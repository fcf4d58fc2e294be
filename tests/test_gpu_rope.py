"""Rotary embedding fused into the store (K rotated on the way into the pool)
and into the attention prologue (q rotated), through the C ABI, against the
oracle's rotary embedding: the stored pools bit for bit, the attention bit for
bit against the plain attention on an oracle-rotated q."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import DeviceStep, bf16_dev, check_attention, host_u16, i32_dev

pytestmark = pytest.mark.gpu


def tables(dev, rows, D):
    c, s = W.rope_tables(rows, D)
    return c, s, torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev)


def rotated_step(inp):
    """Oracle side of a rotary decode step: the new K rows rotated at their
    positions (L_b - 1), the pools after the store, q rotated at L_b - 1."""
    cfg = inp.cfg
    pos = (inp.seq_lens[inp.seq_lens > 0] - 1).astype(np.int32)
    c, s = W.rope_tables(max(int(inp.seq_lens.max()), 1), cfg.D)
    k_rot = oracle.rope(inp.k_new, pos, c, s, cfg.Hkv)
    flat = lambda a: a.reshape(cfg.num_pages * cfg.P, cfg.row_elems)
    kf, vf = oracle.kv_store(flat(inp.k_pool), flat(inp.v_pool), k_rot, inp.v_new, inp.slot_mapping)
    qpos = np.maximum(inp.seq_lens - 1, 0).astype(np.int32)
    q_rot = oracle.rope(inp.q.reshape(cfg.B, -1), qpos, c, s, cfg.Hq).reshape(inp.q.shape)
    return pos, qpos, kf.reshape(inp.k_pool.shape), vf.reshape(inp.v_pool.shape), q_rot


@pytest.mark.parametrize("wl", ["tiny_gqa", "llama3_8b_decode", "ragged_batch", "long_context", "mha_page1"])
def test_store_rope_pools_bit_exact(gpu_device, wl):
    inp = W.make_inputs(W.WORKLOADS[wl])
    cfg = inp.cfg
    print(f"store+rope {wl}: {cfg.describe()}", flush=True)
    pos, _, kf, vf, _ = rotated_step(inp)
    _, _, cd, sd = tables(gpu_device, max(int(inp.seq_lens.max()), 1), cfg.D)
    st = DeviceStep(inp, gpu_device)
    pkv.kv_store_rope(st.k_pool, st.v_pool, st.k_new.view(-1, cfg.Hkv, cfg.D),
                      st.v_new.view(-1, cfg.Hkv, cfg.D), st.slot_mapping, i32_dev(pos, gpu_device), cd, sd)
    torch.cuda.synchronize()
    assert host_u16(st.k_pool).tobytes() == kf.tobytes()
    assert host_u16(st.v_pool).tobytes() == vf.tobytes()


@pytest.mark.parametrize("D,Hkv", [(64, 1), (64, 8), (128, 2), (128, 8)])
def test_store_rope_bulk_fill_bit_exact(gpu_device, D, Hkv):
    rng = np.random.Generator(np.random.PCG64(D + Hkv))
    n, slots_total, rows = 700, 1000, 65536
    k = W.to_bf16_bits(rng.standard_normal((n, Hkv * D)).astype(np.float32))
    v = W.to_bf16_bits(rng.standard_normal((n, Hkv * D)).astype(np.float32))
    slots = rng.permutation(slots_total)[:n].astype(np.int32)
    pos = rng.integers(0, rows, n).astype(np.int32)
    c, s, cd, sd = tables(gpu_device, rows, D)
    pool0 = np.full((slots_total, Hkv * D), W.BF16_NAN, np.uint16)
    kp, vp = bf16_dev(pool0, gpu_device), bf16_dev(pool0, gpu_device)
    pkv.kv_store_rope(kp.view(slots_total, 1, Hkv, D), vp.view(slots_total, 1, Hkv, D),
                      bf16_dev(k, gpu_device).view(n, Hkv, D), bf16_dev(v, gpu_device).view(n, Hkv, D),
                      i32_dev(slots, gpu_device), i32_dev(pos, gpu_device), cd, sd)
    torch.cuda.synchronize()
    kf, vf = oracle.kv_store(pool0, pool0, oracle.rope(k, pos, c, s, Hkv), v, slots)
    assert host_u16(kp).tobytes() == kf.tobytes() and host_u16(vp).tobytes() == vf.tobytes()


# long_context at one split: 4096 page ids per split, refetched from LDS in two segments
@pytest.mark.parametrize("wl,splits", [("tiny_gqa", 3), ("llama3_8b_decode", None), ("long_context", None),
                                       ("long_context", 1), ("mha_page1", None)])
def test_attention_rope_equals_attention_on_rotated_q(gpu_device, wl, splits):
    inp = W.make_inputs(W.WORKLOADS[wl])
    cfg = inp.cfg
    pos, qpos, kf, vf, q_rot = rotated_step(inp)
    _, _, cd, sd = tables(gpu_device, max(int(inp.seq_lens.max()), 1), cfg.D)
    st = DeviceStep(inp, gpu_device, pools=(kf, vf))
    S = splits or pkv.num_splits(cfg.B, cfg.Hq, cfg.Hkv, inp.max_seq_len, cfg.P, int(inp.seq_lens.sum()))
    o1, l1 = pkv.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens,
                                   inp.max_seq_len, S, q_positions=i32_dev(qpos, gpu_device),
                                   rope_cos=cd, rope_sin=sd)
    out1 = pkv.decode_merge(o1, l1)
    o2, l2 = pkv.paged_decode_attn(bf16_dev(q_rot, gpu_device), st.k_pool, st.v_pool, st.page_table,
                                   st.seq_lens, inp.max_seq_len, S)
    out2 = pkv.decode_merge(o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    ref, _ = oracle.paged_decode(q_rot, kf, vf, inp.page_table, inp.seq_lens)
    check_attention(out1, ref, f"rope attention {wl}")


def test_positions_outside_the_table_give_nan_rows(gpu_device):
    inp = W.make_inputs(W.WORKLOADS["tiny_gqa"])
    cfg = inp.cfg
    _, _, cd, sd = tables(gpu_device, 64, cfg.D)          # table shorter than position 99
    st = DeviceStep(inp, gpu_device)
    pos = np.array([36, 99], np.int32)                      # the second is outside
    pkv.kv_store_rope(st.k_pool, st.v_pool, st.k_new.view(-1, 1, cfg.D), st.v_new.view(-1, 1, cfg.D),
                      st.slot_mapping, i32_dev(pos, gpu_device), cd, sd)
    torch.cuda.synchronize()
    flat = st.k_pool.view(-1, cfg.row_elems)
    assert torch.isfinite(flat[int(inp.slot_mapping[0])].float()).all()
    assert torch.isnan(flat[int(inp.slot_mapping[1])].float()).all()
    o, l = pkv.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, inp.max_seq_len, 1,
                                 q_positions=i32_dev(np.array([5, 64], np.int32), gpu_device),
                                 rope_cos=cd, rope_sin=sd)
    out = pkv.decode_merge(o, l).float()
    torch.cuda.synchronize()
    assert torch.isnan(out[1]).all()


def test_rope_argument_errors(gpu_device):
    inp = W.make_inputs(W.WORKLOADS["tiny_gqa"])
    cfg = inp.cfg
    st = DeviceStep(inp, gpu_device)
    _, _, cd, sd = tables(gpu_device, 128, cfg.D)
    pos = i32_dev(np.array([1, 2], np.int32), gpu_device)
    with pytest.raises(RuntimeError):      # tables of the wrong width
        pkv.kv_store_rope(st.k_pool, st.v_pool, st.k_new.view(-1, 1, cfg.D), st.v_new.view(-1, 1, cfg.D),
                          st.slot_mapping, pos, cd[:, :8].contiguous(), sd[:, :8].contiguous())
    with pytest.raises(RuntimeError):      # misaligned table base (through the C ABI check)
        bad = torch.empty(cd.numel() + 1, dtype=torch.float32, device=gpu_device)[1:].view(cd.shape)
        pkv.kv_store_rope(st.k_pool, st.v_pool, st.k_new.view(-1, 1, cfg.D), st.v_new.view(-1, 1, cfg.D),
                          st.slot_mapping, pos, bad, sd)
    with pytest.raises(RuntimeError):      # q positions without tables
        pkv.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, 100, 1, q_positions=pos)
