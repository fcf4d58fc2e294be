"""The decode step on the GPU (store -> split-KV attention -> merge), through
the C ABI, against the fp64 oracle, plus the invariants that hold bit for bit
on the GPU (placement, determinism, 2^k scaling, length one)."""
import math

import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import DeviceStep, bf16_dev, check_attention, host_f64_from_bf16, host_u16, i32_dev

pytestmark = pytest.mark.gpu

_cache = {}


@pytest.fixture(params=["mfma", "valu"])
def decode_kernel(request):
    """Every test runs on both decode kernels: the matrix-core one behind every
    decode entry point, and the all-VALU one (pkv_paged_decode_attn_valu)."""
    return request.param


def inputs(wl):
    if wl not in _cache:
        _cache.clear()
        _cache[wl] = W.make_inputs(W.WORKLOADS[wl])
    return _cache[wl]


def _oracle_full(inp):
    kf, vf = inp.pools_after_store()
    return oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)


@pytest.mark.parametrize("wl", ["tiny_gqa", "llama3_8b_decode", "ragged_batch", "long_context", "mha_page1"])
def test_decode_step_matches_oracle(gpu_device, decode_kernel, wl):
    inp = inputs(wl)
    S = pkv.num_splits(inp.cfg.B, inp.cfg.Hq, inp.cfg.Hkv, inp.max_seq_len, inp.cfg.P,
                       int(inp.seq_lens.sum()))
    print(f"decode step {wl} ({inp.cfg.describe()}), num_splits {S}", flush=True)
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    (out, lse), o_p, l_p = st.step(want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle_full(inp)
    check_attention(out, ref, f"cfg {wl}")
    g_lse = lse.cpu().numpy().astype(np.float64)
    assert np.abs(g_lse - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
    # every partial written and finite or an exact empty split
    lp = l_p.cpu().numpy()
    op = o_p.cpu().numpy()
    assert not np.isnan(lp).any() and not np.isnan(op).any()
    assert (op[np.isneginf(lp)] == 0).all()


@pytest.mark.parametrize("wl", ["tiny_gqa", "llama3_8b_decode", "long_context"])
def test_partials_match_oracle_split_mode(gpu_device, decode_kernel, wl):
    inp = inputs(wl)
    cfg = inp.cfg
    S = pkv.num_splits(cfg.B, cfg.Hq, cfg.Hkv, inp.max_seq_len, cfg.P, int(inp.seq_lens.sum()))
    if wl in ("tiny_gqa", "llama3_8b_decode"):
        S = 3 if wl == "tiny_gqa" else 2  # force several splits where the heuristic picks one
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    st.store()
    _, o_p, l_p = st.attend(splits=S)
    torch.cuda.synchronize()
    kf, vf = inp.pools_after_store()
    chunk = oracle.split_chunk(inp.max_seq_len, S, cfg.P)
    assert pkv.split_chunk(inp.max_seq_len, S, cfg.P) == chunk
    rows = W.sample_rows(cfg, 16)
    o_ref, l_ref = oracle.paged_decode_split(inp.q, kf, vf, inp.page_table, inp.seq_lens, chunk, S)
    for b, h in rows:
        go = o_p[b, h].cpu().numpy().astype(np.float64)
        gl = l_p[b, h].cpu().numpy().astype(np.float64)
        assert (np.isneginf(gl) == np.isneginf(l_ref[b, h])).all()
        fin = np.isfinite(l_ref[b, h])
        assert np.abs(gl[fin] - l_ref[b, h][fin]).max(initial=0) <= 1e-4
        assert np.abs(go - o_ref[b, h]).max() <= 1e-4, (b, h)


def test_merge_alone_on_oracle_partials(gpu_device):
    """decode_merge fed the oracle's partials (rounded to fp32) vs the fp64 merge."""
    inp = inputs("tiny_gqa")
    kf, vf = inp.pools_after_store()
    S = 5
    chunk = oracle.split_chunk(inp.max_seq_len, S, inp.cfg.P)
    o_ref, l_ref = oracle.paged_decode_split(inp.q, kf, vf, inp.page_table, inp.seq_lens, chunk, S)
    out_ref, lse_ref = oracle.merge(o_ref, l_ref)
    o_dev = torch.from_numpy(o_ref.astype(np.float32)).to(gpu_device)
    l_dev = torch.from_numpy(l_ref.astype(np.float32)).to(gpu_device)
    out, lse = pkv.decode_merge(o_dev, l_dev, want_lse=True)
    torch.cuda.synchronize()
    g = host_f64_from_bf16(out)
    # one bf16 rounding of a value known to ~1e-6
    assert (np.abs(g - out_ref) <= np.abs(out_ref) * 2.0 ** -8 + 1e-6).all()
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


def test_length_one_returns_the_value_row_bit_exact(gpu_device, decode_kernel):
    cfg = W.custom_config(B=5, Hq=16, Hkv=2, D=128, P=16, num_pages=12, seq_lens=(1,) * 5)
    inp = W.make_inputs(cfg)
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    out, _, _ = st.step(splits=3)
    torch.cuda.synchronize()
    got = host_u16(out)
    kf, vf = inp.pools_after_store()
    for b in range(5):
        page = inp.page_table[b, 0]
        for h in range(16):
            assert (got[b, h] == vf[page, 0, h // 8]).all()


def test_identical_keys_give_mean_of_values(gpu_device, decode_kernel):
    cfg = W.custom_config(B=3, Hq=8, Hkv=2, D=64, P=16, num_pages=40, seq_lens=(5, 300, 129))
    inp = W.make_inputs(cfg)
    kf, vf = inp.pools_after_store()
    key = kf[inp.page_table[0, 0], 0].copy()
    kp = inp.k_pool.copy()
    kp[:] = key
    knew = np.tile(key.reshape(1, -1), (3, 1))
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel, pools=(kp, inp.v_pool))
    st.k_new = bf16_dev(knew, gpu_device)
    out, _, _ = st.step(splits=2)
    torch.cuda.synchronize()
    g = host_f64_from_bf16(out)
    for b in range(3):
        L = int(inp.seq_lens[b])
        t = np.arange(L)
        rows = vf[inp.page_table[b, t // 16], t % 16]          # [L, Hkv, D]
        mean = W.bf16_bits_to_f32(rows).astype(np.float64).mean(axis=0)
        for h in range(8):
            assert np.abs(g[b, h] - mean[h // 4]).max() <= 2.0 ** -8 * np.abs(mean[h // 4]).max() + 1e-3


@pytest.mark.parametrize("wl", ["tiny_gqa", "ragged_batch"])
def test_paged_equals_contiguous_bitwise(gpu_device, decode_kernel, wl):
    inp = inputs(wl)
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    out1, _, _ = st.step()
    kc, vc, ptc = W.contiguous_layout(inp)
    st2 = DeviceStep(inp, gpu_device, kernel=decode_kernel, pools=(kc, vc), page_table=ptc)
    out2, _, _ = st2.attend()
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_run_to_run_determinism(gpu_device, decode_kernel):
    inp = inputs("llama3_8b_decode")
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    st.store()
    a, _, _ = st.attend()
    b, _, _ = st.attend()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_split_count_invariance(gpu_device, decode_kernel):
    """S = 1 and S = k agree to within one bf16 rounding step."""
    inp = inputs("llama3_8b_decode")
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    st.store()
    outs = [host_f64_from_bf16(st.attend(splits=s)[0]) for s in (1, 2, 5, 16)]
    for o in outs[1:]:
        assert (np.abs(o - outs[0]) <= np.abs(outs[0]) * 2.0 ** -7 + 1e-6).all()


def test_value_scaling_by_power_of_two_is_exact(gpu_device, decode_kernel):
    inp = inputs("tiny_gqa")
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    out1, _, _ = st.step(splits=2)
    st.v_pool.mul_(2.0 ** 5)
    out2, _, _ = st.attend(splits=2)
    torch.cuda.synchronize()
    assert torch.equal((out1.float() * 2.0 ** 5).to(torch.bfloat16).view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("D,G,P", [(64, 1, 1), (64, 2, 2), (64, 8, 64), (128, 1, 16), (128, 2, 4),
                                   (128, 4, 1), (128, 8, 16), (128, 8, 256), (64, 4, 1024)])
def test_shapes_and_ragged_tails(gpu_device, decode_kernel, D, G, P):
    Hkv = 2
    lens = (1, P - 1 if P > 1 else 1, P, 3 * P + 1, 777, 1500)
    cfg = W.custom_config(name=f"d{D}g{G}p{P}", B=len(lens), Hq=G * Hkv, Hkv=Hkv, D=D, P=P,
                          num_pages=-(-sum(lens) // P) + len(lens) + 3, seq_lens=lens)
    inp = W.make_inputs(cfg)
    for S in (1, 3):
        st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
        out, _, _ = st.step(splits=S)
        torch.cuda.synchronize()
        check_attention(out, _oracle_full(inp)[0], f"D{D} G{G} P{P} S{S}")


@pytest.mark.parametrize("D,G,P,lens,S", [
    (64, 4, 1, (5000, 2100, 1), 1),       # 5000 page ids in one split: three LDS segments
    (64, 1, 1, (4097,), 2),               # two splits of 2049 pages: each past one segment
    (128, 4, 16, (40000, 33000), 1),      # 2500 and 2063 pages: two segments each
])
def test_splits_longer_than_one_page_id_segment(gpu_device, decode_kernel, D, G, P, lens, S):
    """A split whose pages exceed the 2048 page ids staged in LDS at a time
    refetches them segment by segment."""
    cfg = W.custom_config(name=f"long_split_d{D}g{G}p{P}", B=len(lens), Hq=G, Hkv=1, D=D, P=P,
                          num_pages=-(-sum(lens) // P) + len(lens) + 3, seq_lens=lens)
    inp = W.make_inputs(cfg)
    print(f"long splits D{D} G{G} P{P} lens {lens} S{S}", flush=True)
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    out, _, _ = st.step(splits=S)
    torch.cuda.synchronize()
    check_attention(out, _oracle_full(inp)[0], f"long splits D{D} G{G} P{P} S{S}")


def test_empty_sequence_and_empty_splits(gpu_device, decode_kernel):
    cfg = W.custom_config(B=3, Hq=4, Hkv=1, D=64, P=16, num_pages=20, seq_lens=(0, 3, 200))
    inp = W.make_inputs(cfg)
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    st.store()
    o_p, l_p = pkv.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, 200, 7,
                                     kernel=decode_kernel)
    out, lse = pkv.decode_merge(o_p, l_p, want_lse=True)
    torch.cuda.synchronize()
    g = host_f64_from_bf16(out)
    assert (g[0] == 0).all() and torch.isneginf(lse[0]).all()
    assert torch.isneginf(l_p[1, :, 1:]).all() and (o_p[1, :, 1:] == 0).all()
    ref, _ = _oracle_full(inp)
    check_attention(out[1:], ref[1:], "nonempty rows")


def test_canary_reaches_output_when_store_is_skipped(gpu_device, decode_kernel):
    inp = inputs("tiny_gqa")
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    out, _, _ = st.attend()
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()


def test_bad_page_id_poisons_only_its_row(gpu_device, decode_kernel):
    inp = inputs("tiny_gqa")
    pt = inp.page_table.copy()
    pt[1, 2] = inp.cfg.num_pages + 5
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel, page_table=pt)
    out, _, _ = st.step()
    torch.cuda.synchronize()
    o = out.float().cpu()
    assert torch.isnan(o[1]).all() and torch.isfinite(o[0]).all()


def test_max_splits(gpu_device, decode_kernel):
    cfg = W.custom_config(B=1, Hq=8, Hkv=1, D=128, P=1, num_pages=3000, seq_lens=(2049,))
    inp = W.make_inputs(cfg)
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    out, o_p, _ = st.step(splits=1024)
    torch.cuda.synchronize()
    assert o_p.shape[2] == 1024
    check_attention(out, _oracle_full(inp)[0], "S=1024")


def test_errors_raise(gpu_device, decode_kernel):
    inp = inputs("tiny_gqa")
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    with pytest.raises(RuntimeError):
        pkv.paged_decode_attn(st.q.float(), st.k_pool, st.v_pool, st.page_table, st.seq_lens, 100,
                              kernel=decode_kernel)
    with pytest.raises(RuntimeError):   # max_seq_len beyond max_pages * page_size
        pkv.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, 10_000,
                              kernel=decode_kernel)
    with pytest.raises(RuntimeError):
        q_bad = torch.empty(st.q.numel() + 8, dtype=torch.bfloat16, device=gpu_device)[1:1 + st.q.numel()]
        pkv.paged_decode_attn(q_bad.view(st.q.shape), st.k_pool, st.v_pool, st.page_table, st.seq_lens, 100,
                              kernel=decode_kernel)


@pytest.mark.parametrize("head", [2, 0])
def test_nan_query_gives_nan_rows(gpu_device, decode_kernel, head):
    """Every score of a row NaN: the row is NaN (as in the oracle), not an empty
    split's zeros, and no other row of its kv-head group (head 0 is the row the
    matrix-core kernel's prefetches past a wave's range read) is touched."""
    inp = inputs("tiny_gqa")
    q = inp.q.copy()
    q[1, head] = W.BF16_NAN
    st = DeviceStep(inp, gpu_device, kernel=decode_kernel)
    st.q = bf16_dev(q, gpu_device)
    (out, lse), _, _ = st.step(splits=3, want_lse=True)
    torch.cuda.synchronize()
    kf, vf = inp.pools_after_store()
    ref, ref_lse = oracle.paged_decode(q, kf, vf, inp.page_table, inp.seq_lens)
    g = host_f64_from_bf16(out)
    assert np.isnan(ref[1, head]).all() and np.isnan(ref_lse[1, head])
    assert np.isnan(g[1, head]).all() and torch.isnan(lse[1, head])
    mask = np.ones(g.shape[:2], bool)
    mask[1, head] = False
    assert np.isfinite(g[mask]).all()
