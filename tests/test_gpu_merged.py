"""pkv_paged_decode_attn_merged on the GPU through the C ABI: the same bits
as pkv_paged_decode_attn followed by pkv_decode_merge (one kernel with one
split, two launches with more), on the decode workloads and the degenerate
rows (empty sequence, NaN query row), and within the tolerance of the fp64
oracle."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import DeviceStep, bf16_dev, check_attention

pytestmark = pytest.mark.gpu


def both(st, splits, max_len=None):
    max_len = st.inp.max_seq_len if max_len is None else max_len
    o_p, l_p = pkv.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, max_len, splits)
    ref_out, ref_lse = pkv.decode_merge(o_p, l_p, want_lse=True)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    pkv.paged_decode_attn_merged(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, max_len, splits,
                                 out=out, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.contiguous().view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


@pytest.mark.parametrize("wl,splits", [("tiny_gqa", 1), ("llama3_8b_decode", 1), ("llama3_8b_decode", 2), ("ragged_batch", None), ("mha_page1", 1)])
def test_merged_equals_attention_then_merge(gpu_device, wl, splits):
    inp = W.make_inputs(W.WORKLOADS[wl])
    S = splits or pkv.num_splits(inp.cfg.B, inp.cfg.Hq, inp.cfg.Hkv, inp.max_seq_len, inp.cfg.P,
                                 int(inp.seq_lens.sum()))
    print(f"merged decode {wl} ({inp.cfg.describe()}), num_splits {S}", flush=True)
    st = DeviceStep(inp, gpu_device)
    st.store()
    out, lse, ref_out, ref_lse = both(st, S)
    assert same_bits(out, ref_out) and same_bits(lse, ref_lse)
    kf, vf = inp.pools_after_store()
    ref, _ = oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)
    check_attention(out, ref, f"merged {wl} S={S}")


def test_merged_degenerate_rows(gpu_device):
    # an empty sequence (out 0, lse -inf) and a NaN query row (out NaN, lse NaN), one split
    cfg = W.custom_config(B=3, Hq=4, Hkv=1, D=64, P=16, num_pages=20, seq_lens=(0, 3, 200))
    inp = W.make_inputs(cfg)
    q = inp.q.copy()
    q[2, 1] = W.BF16_NAN
    st = DeviceStep(inp, gpu_device)
    st.q = bf16_dev(q, gpu_device)
    st.store()
    for S in (1, 3):
        out, lse, ref_out, ref_lse = both(st, S, 200)
        assert same_bits(out, ref_out) and same_bits(lse, ref_lse), f"S={S}"
        assert (out[0].float() == 0).all() and torch.isneginf(lse[0]).all()
        assert torch.isnan(out[2, 1].float()).all() and torch.isnan(lse[2, 1])


def test_merged_one_split_needs_no_partials(gpu_device):
    inp = W.make_inputs(W.WORKLOADS["tiny_gqa"])
    st = DeviceStep(inp, gpu_device)
    st.store()
    out = pkv.paged_decode_attn_merged(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens,
                                       inp.max_seq_len, 1)
    torch.cuda.synchronize()
    kf, vf = inp.pools_after_store()
    check_attention(out, oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)[0], "no partials")
