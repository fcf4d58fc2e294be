"""The library keeps no state between calls (apart from the no-allocation
call's documented scratch): two independent decode steps enqueued on two
streams at once, interleaved call by call, give each the bits it gives alone
on the default stream."""
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import DeviceStep

pytestmark = pytest.mark.gpu


def one_step(st, S):
    return pkv.decode_step_fused(st.q, st.k_new, st.v_new, st.k_pool, st.v_pool, st.page_table, st.seq_lens,
                                 st.slot_mapping, st.inp.max_seq_len, S, want_lse=True)


def test_two_streams_equal_one(gpu_device):
    a_inp = W.make_inputs(W.WORKLOADS["llama3_8b_decode"])
    b_inp = W.make_inputs(W.custom_config(seed_id=7700, name="streams_b", B=24, Hq=16, Hkv=16, D=64, P=1,
                                          num_pages=60000, seq_lens=tuple(range(100, 2500, 100))))
    Sa, Sb = 3, 2
    ref_a = one_step(DeviceStep(a_inp, gpu_device), Sa)
    ref_b = one_step(DeviceStep(b_inp, gpu_device), Sb)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        a, b = DeviceStep(a_inp, gpu_device), DeviceStep(b_inp, gpu_device)
        torch.cuda.synchronize()
        outs = {}
        for k in range(4):                      # four steps on each stream, interleaved
            with torch.cuda.stream(sa):
                outs["a"] = one_step(a, Sa)
            with torch.cuda.stream(sb):
                outs["b"] = one_step(b, Sb)
        torch.cuda.synchronize()
        for key, ref in (("a", ref_a), ("b", ref_b)):
            got = outs[key]
            assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)), (rep, key)
            assert torch.equal(got[1], ref[1]), (rep, key)
