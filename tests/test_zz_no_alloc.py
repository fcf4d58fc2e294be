"""The no-allocation merged attention (pkv_paged_decode_attn_merged_static)
through the C ABI: its partials live in the library's static device scratch,
and its output must equal pkv_paged_decode_attn_merged's (caller workspace)
bit for bit, on consecutive calls of different sizes."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import DeviceStep, check_attention

pytestmark = pytest.mark.gpu


def _ragged_cfg(name, seed_id, B, Hq, Hkv, D, P, max_len):
    rng = np.random.Generator(np.random.PCG64(W.SEED_BASE + 500 + seed_id))
    lens = tuple(int(x) for x in rng.integers(1, max_len + 1, B))
    pages = -(-sum(lens) // P) + B + 3
    return W.custom_config(seed_id=500 + seed_id, name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, P=P,
                           num_pages=pages, seq_lens=lens)


def _both(st, S):
    """(out, lse) of the workspace call and of the static-scratch call."""
    a = st.inp
    ref = pkv.paged_decode_attn_merged(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens,
                                       a.max_seq_len, S, want_lse=True)
    got = pkv.paged_decode_attn_merged_static(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens,
                                              a.max_seq_len, S, want_lse=True)
    torch.cuda.synchronize()
    return ref, got


def test_static_scratch_equals_workspace_on_consecutive_calls(gpu_device):
    # 1: near the scratch limit: 63 * 64 * 8 rows x (128 + 1) floats = 15.9 MiB
    big = _ragged_cfg("static_big", 1, B=63, Hq=64, Hkv=8, D=128, P=16, max_len=400)
    inp = W.make_inputs(big)
    print(f"static scratch, call 1: {big.describe()} S=8", flush=True)
    st = DeviceStep(inp, gpu_device)
    st.store()
    (o1, l1), (o2, l2) = _both(st, 8)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    kf, vf = inp.pools_after_store()
    ref, _ = oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)
    check_attention(o2, ref, "static scratch, call 1")

    # 2: a smaller batch right after (the scratch still holds call 1's partials)
    small = _ragged_cfg("static_small", 2, B=5, Hq=8, Hkv=4, D=64, P=4, max_len=90)
    inp2 = W.make_inputs(small)
    print(f"static scratch, call 2: {small.describe()} S=3", flush=True)
    st2 = DeviceStep(inp2, gpu_device)
    st2.store()
    (o3, l3), (o4, l4) = _both(st2, 3)
    assert torch.equal(o3.view(torch.int16), o4.view(torch.int16))
    assert torch.equal(l3, l4)
    kf, vf = inp2.pools_after_store()
    ref2, _ = oracle.paged_decode(inp2.q, kf, vf, inp2.page_table, inp2.seq_lens)
    check_attention(o4, ref2, "static scratch, call 2")

    # 3: one split uses no scratch; same bits as the workspace call
    (o5, l5), (o6, l6) = _both(st2, 1)
    assert torch.equal(o5.view(torch.int16), o6.view(torch.int16))
    assert torch.equal(l5, l6)

    # 4: partials beyond the 16 MiB scratch are refused before any launch
    with pytest.raises(RuntimeError, match="static scratch"):
        pkv.paged_decode_attn_merged_static(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens,
                                            inp.max_seq_len, 9, want_lse=True)
