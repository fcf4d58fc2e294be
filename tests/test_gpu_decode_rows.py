"""The decode attention for one q head per kv head (the kernel that reads whole
token rows, 512 / D heads per workgroup) through the C ABI: against the fp64
oracle over head sizes, page sizes, split counts and ragged tails, the bitwise
invariants (placement, determinism, length one, 2^k scaling), the degenerate
cases (empty sequences and splits, NaN queries, bad page ids), the fused step
and the rotated-q prologue on the same kernel."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import DeviceStep, bf16_dev, check_attention, host_f64_from_bf16, host_u16, i32_dev
from .test_gpu_fused_step import run_both
from .test_gpu_rope import rotated_step, tables

pytestmark = pytest.mark.gpu


def mha(D, Hkv, P, lens, name="rows", seed_id=300):
    return W.custom_config(seed_id=seed_id, name=f"{name}_d{D}h{Hkv}p{P}", B=len(lens), Hq=Hkv, Hkv=Hkv, D=D,
                           P=P, num_pages=-(-sum(lens) // P) + len(lens) + 3, seq_lens=tuple(lens))


def oracle_full(inp):
    kf, vf = inp.pools_after_store()
    return oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)


@pytest.mark.parametrize("D,Hkv", [(64, 8), (64, 16), (128, 4), (128, 8)])
@pytest.mark.parametrize("P", [1, 2, 16, 64])
def test_rows_kernel_matches_oracle(gpu_device, D, Hkv, P):
    lens = (1, max(P - 1, 1), P, 3 * P + 1, 777, 1500, 33)
    inp = W.make_inputs(mha(D, Hkv, P, lens))
    ref, ref_lse = oracle_full(inp)
    for S in (1, 3, 7):
        st = DeviceStep(inp, gpu_device)
        (out, lse), o_p, l_p = st.step(splits=S, want_lse=True)
        torch.cuda.synchronize()
        check_attention(out, ref, f"rows D{D} Hkv{Hkv} P{P} S{S}")
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
        lp, op = l_p.cpu().numpy(), o_p.cpu().numpy()
        assert not np.isnan(lp).any() and not np.isnan(op).any()
        assert (op[np.isneginf(lp)] == 0).all()


def test_rows_kernel_partials_match_oracle_split_mode(gpu_device):
    inp = W.make_inputs(mha(64, 8, 1, (300, 2049, 17, 1024)))
    S = 5
    st = DeviceStep(inp, gpu_device)
    st.store()
    _, o_p, l_p = st.attend(splits=S)
    torch.cuda.synchronize()
    kf, vf = inp.pools_after_store()
    chunk = oracle.split_chunk(inp.max_seq_len, S, inp.cfg.P)
    o_ref, l_ref = oracle.paged_decode_split(inp.q, kf, vf, inp.page_table, inp.seq_lens, chunk, S)
    go, gl = o_p.cpu().numpy().astype(np.float64), l_p.cpu().numpy().astype(np.float64)
    assert (np.isneginf(gl) == np.isneginf(l_ref)).all()
    fin = np.isfinite(l_ref)
    assert np.abs(gl[fin] - l_ref[fin]).max() <= 1e-4
    assert np.abs(go - o_ref).max() <= 1e-4


@pytest.mark.parametrize("lens,S", [((5000, 2100, 1), 1), ((4097,), 2), ((6000, 10), 3)])
def test_rows_kernel_splits_longer_than_one_page_id_segment(gpu_device, lens, S):
    """Splits of more than the 2048 page ids staged in LDS at a time."""
    inp = W.make_inputs(mha(64, 8, 1, lens, name="rows_long"))
    st = DeviceStep(inp, gpu_device)
    out, _, _ = st.step(splits=S)
    torch.cuda.synchronize()
    check_attention(out, oracle_full(inp)[0], f"rows long splits {lens} S{S}")


def test_rows_kernel_bitwise_invariants(gpu_device):
    inp = W.make_inputs(mha(64, 16, 1, (700, 1, 129, 1500), name="rows_inv"))
    # paged == contiguous
    st = DeviceStep(inp, gpu_device)
    out1, _, _ = st.step(splits=3)
    kc, vc, ptc = W.contiguous_layout(inp)
    st2 = DeviceStep(inp, gpu_device, pools=(kc, vc), page_table=ptc)
    out2, _, _ = st2.attend(splits=3)
    # run to run
    out3, _, _ = st.attend(splits=3)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))
    # V x 2^5 scales the output exactly
    st.v_pool.mul_(2.0 ** 5)
    out4, _, _ = st.attend(splits=3)
    torch.cuda.synchronize()
    assert torch.equal((out1.float() * 2.0 ** 5).to(torch.bfloat16).view(torch.int16), out4.view(torch.int16))
    # a sequence of length 1 returns its V row exactly
    got = host_u16(out1)
    kf, vf = inp.pools_after_store()
    assert (got[1] == vf[inp.page_table[1, 0], 0]).all()


def test_rows_kernel_empty_sequences_nan_queries_and_bad_pages(gpu_device):
    inp = W.make_inputs(mha(128, 4, 2, (0, 40, 300, 5), name="rows_edge"))
    q = inp.q.copy()
    q[2, 1] = W.BF16_NAN                    # one NaN query row
    pt = inp.page_table.copy()
    pt[3, 1] = inp.cfg.num_pages + 9        # a page id outside the pool in sequence 3
    st = DeviceStep(inp, gpu_device, page_table=pt)
    st.q = bf16_dev(q, gpu_device)
    st.store()
    o_p, l_p = pkv.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, 300, 7)
    out, lse = pkv.decode_merge(o_p, l_p, want_lse=True)
    torch.cuda.synchronize()
    g = host_f64_from_bf16(out)
    assert (g[0] == 0).all() and torch.isneginf(lse[0]).all()                  # empty sequence
    assert torch.isneginf(l_p[1, :, 1:]).all() and (o_p[1, :, 1:] == 0).all()  # empty splits
    assert np.isnan(g[2, 1]).all() and np.isfinite(g[2, [0, 2, 3]]).all()      # NaN query: its row only
    assert np.isnan(g[3]).all()                                              # bad page: its sequence
    kf, vf = inp.pools_after_store()
    ref, _ = oracle.paged_decode(q, kf, vf, inp.page_table, inp.seq_lens)
    check_attention(out[1:2], ref[1:2], "rows edge: sequence 1")
    check_attention(out[2, [0, 2, 3]], ref[2, [0, 2, 3]], "rows edge: sequence 2, finite rows")


@pytest.mark.parametrize("S", [2, 4])
def test_rows_kernel_longest_first_order(gpu_device, S):
    """Several splits and few (sequence, split) pairs: the pairs run longest
    first (ranked in the kernel); results do not depend on that order."""
    rng = np.random.Generator(np.random.PCG64(77))
    lens = tuple(int(x) for x in rng.integers(1, 3000, 24))
    inp = W.make_inputs(mha(64, 8, 16, lens, name="rows_lpt"))
    st = DeviceStep(inp, gpu_device)
    out, _, _ = st.step(splits=S)
    torch.cuda.synchronize()
    check_attention(out, oracle_full(inp)[0], f"rows longest first S{S}")


@pytest.mark.parametrize("lens,S", [((49, 129, 16, 1, 300), 4), ((2048, 7), 1), ((4097, 3000), 2)])
def test_rows_kernel_fused_step_equals_store_then_attention(gpu_device, lens, S):
    inp = W.make_inputs(mha(64, 8, 1, lens, name="rows_fused"))
    out, _ = run_both(inp, gpu_device, S)
    check_attention(out, oracle_full(inp)[0], f"rows fused step {lens} S{S}")


def test_rows_kernel_fused_step_empty_sequence(gpu_device):
    cfg = mha(128, 4, 16, (49, 0, 16), name="rows_fused_empty")
    inp = W.make_inputs(cfg)
    slots = np.concatenate([inp.slot_mapping[:1], [cfg.num_pages * cfg.P - 1], inp.slot_mapping[1:]])
    kn = np.concatenate([inp.k_new[:1], inp.k_new[:1], inp.k_new[1:]])
    vn = np.concatenate([inp.v_new[:1], inp.v_new[:1], inp.v_new[1:]])
    for S in (1, 3):
        run_both(inp, gpu_device, S, slots=slots.astype(np.int32), new_rows=(kn, vn))


@pytest.mark.parametrize("D,Hkv,P", [(64, 8, 1), (128, 4, 16)])
def test_rows_kernel_rotated_q_equals_attention_on_rotated_q(gpu_device, D, Hkv, P):
    inp = W.make_inputs(mha(D, Hkv, P, (5, 400, 1000, 77), name="rows_rope"))
    cfg = inp.cfg
    _, qpos, kf, vf, q_rot = rotated_step(inp)
    _, _, cd, sd = tables(gpu_device, max(int(inp.seq_lens.max()), 1), D)
    st = DeviceStep(inp, gpu_device, pools=(kf, vf))
    o1, l1 = pkv.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, inp.max_seq_len, 3,
                                   q_positions=i32_dev(qpos, gpu_device), rope_cos=cd, rope_sin=sd)
    o2, l2 = pkv.paged_decode_attn(bf16_dev(q_rot, gpu_device), st.k_pool, st.v_pool, st.page_table,
                                   st.seq_lens, inp.max_seq_len, 3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref, _ = oracle.paged_decode(q_rot, kf, vf, inp.page_table, inp.seq_lens)
    check_attention(pkv.decode_merge(o1, l1), ref, f"rows rope D{D}")

