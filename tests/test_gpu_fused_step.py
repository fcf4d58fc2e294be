"""pkv_decode_step on the GPU through the C ABI: the store fused into the
attention kernel gives the same pools, output and lse, bit for bit, as
pkv_kv_store followed by pkv_paged_decode_attn_merged, on the decode
workloads (one split and several, page tiles and page_size 1), and on the
edges of the fused store (the new token first in a split, an empty sequence,
a slot outside the pool)."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import DeviceStep, check_attention

pytestmark = pytest.mark.gpu


def bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


def run_both(inp, dev, splits, max_len=None, slots=None, new_rows=None, outputs=True):
    max_len = inp.max_seq_len if max_len is None else max_len
    a, b = DeviceStep(inp, dev), DeviceStep(inp, dev)
    if slots is not None:
        a.slot_mapping = b.slot_mapping = torch.from_numpy(np.asarray(slots, np.int32)).to(dev)
    if new_rows is not None:
        for st in (a, b):
            st.k_new = torch.from_numpy(new_rows[0].view(np.int16)).to(dev).view(torch.bfloat16)
            st.v_new = torch.from_numpy(new_rows[1].view(np.int16)).to(dev).view(torch.bfloat16)
    pkv.kv_store(a.k_pool, a.v_pool, a.k_new, a.v_new, a.slot_mapping)
    ref = pkv.paged_decode_attn_merged(a.q, a.k_pool, a.v_pool, a.page_table, a.seq_lens, max_len, splits,
                                       want_lse=True)
    got = pkv.decode_step_fused(b.q, b.k_new, b.v_new, b.k_pool, b.v_pool, b.page_table, b.seq_lens,
                                b.slot_mapping, max_len, splits, want_lse=True)
    torch.cuda.synchronize()
    if outputs:
        assert torch.equal(bits(got[0]), bits(ref[0])), "output differs from the unfused step"
        assert torch.equal(bits(got[1]), bits(ref[1])), "lse differs from the unfused step"
    assert torch.equal(bits(b.k_pool), bits(a.k_pool)) and torch.equal(bits(b.v_pool), bits(a.v_pool)), \
        "pools differ from the unfused step"
    return got


@pytest.mark.parametrize("wl,splits", [("tiny_gqa", 1), ("llama3_8b_decode", 1), ("llama3_8b_decode", 3), ("ragged_batch", None), ("long_context", None), ("mha_page1", 1)])
def test_fused_step_equals_store_then_attention(gpu_device, wl, splits):
    inp = W.make_inputs(W.WORKLOADS[wl])
    S = splits or pkv.num_splits(inp.cfg.B, inp.cfg.Hq, inp.cfg.Hkv, inp.max_seq_len, inp.cfg.P,
                                 int(inp.seq_lens.sum()))
    print(f"fused step {wl} ({inp.cfg.describe()}), num_splits {S}", flush=True)
    out, _ = run_both(inp, gpu_device, S)
    kf, vf = inp.pools_after_store()
    ref, _ = oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)
    check_attention(out, ref, f"fused step {wl} S={S}")


def test_fused_step_edges(gpu_device):
    # lengths with the new token first in a split (chunk 48 at S=4, max 129), last in a
    # page, and alone; an empty sequence (its row is still stored, by split 0)
    cfg = W.custom_config(B=5, Hq=8, Hkv=2, D=128, P=16, num_pages=40, seq_lens=(49, 129, 16, 1, 0))
    inp = W.make_inputs(cfg)
    # one new row per sequence: the empty one's row goes to the last slot of the pool
    # (no sequence owns it), like any other row of the store
    slots = np.concatenate([inp.slot_mapping, [cfg.num_pages * cfg.P - 1]]).astype(np.int32)
    kn = np.concatenate([inp.k_new, inp.k_new[:1]])
    vn = np.concatenate([inp.v_new, inp.v_new[:1]])
    for S in (1, 4):
        run_both(inp, gpu_device, S, max_len=129, slots=slots, new_rows=(kn, vn))
    # a slot outside the pool is not written, as by the store: the pools match.  (The
    # outputs differ there by design: that slot is no longer position L - 1's, which
    # the fused step reads from the new row.)
    bad = slots.copy()
    bad[1] = cfg.num_pages * cfg.P + 3
    run_both(inp, gpu_device, 1, max_len=129, slots=bad, new_rows=(kn, vn), outputs=False)


@pytest.mark.parametrize("D,G,P,lens,S", [(64, 4, 1, (5000, 2100, 1), 1), (128, 4, 16, (40000, 33000), 1)])
def test_fused_step_with_splits_longer_than_one_page_id_segment(gpu_device, D, G, P, lens, S):
    """The new token's position lies past the first LDS segment of page ids."""
    cfg = W.custom_config(name=f"fused_long_split_d{D}p{P}", B=len(lens), Hq=G, Hkv=1, D=D, P=P,
                          num_pages=-(-sum(lens) // P) + len(lens) + 3, seq_lens=lens)
    inp = W.make_inputs(cfg)
    print(f"fused step, long splits D{D} P{P} lens {lens} S{S}", flush=True)
    out, _ = run_both(inp, gpu_device, S)
    kf, vf = inp.pools_after_store()
    ref, _ = oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)
    check_attention(out, ref, f"fused step long splits D{D} P{P}")
