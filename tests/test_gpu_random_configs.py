"""A seeded sweep over the shape envelope of the decode step, through every
decode entry point of the C ABI.  Each case draws the head size, the group
size, the kv-head count (odd ones included), the page size (1 to 256), the
split count (1 to 16, more than a short sequence has tokens included) and
ragged lengths (empty sequences included).  It checks the store + attention +
merge against the fp64 oracle, and checks bit for bit that:

- the merged call equals the attention followed by the merge;
- the call with its partials in the static scratch equals the merged call;
- the fused step equals the store followed by the merged call;
- q rotated in the attention prologue equals the attention on a q that the
  oracle rotated.
"""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import DeviceStep, bf16_dev, check_attention, i32_dev
from .test_gpu_fused_step import bits, run_both
from .test_gpu_rope import rotated_step, tables

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw(k: int) -> dict:
    rng = np.random.Generator(np.random.PCG64(W.SEED_BASE + 7100 + k))
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8, 16]))
    G = int(rng.choice([1, 2, 4, 8]))
    while G * Hkv > 64:
        G //= 2
    P = int(2 ** rng.integers(0, 9))
    B = int(rng.integers(1, 10))
    # lengths log-uniform on [1, 4000], about one in eight empty
    lens = np.exp(rng.uniform(0.0, np.log(4000.0), B)).astype(np.int64)
    lens[rng.random(B) < 0.125] = 0
    if lens.max() == 0:
        lens[0] = int(rng.integers(1, 300))
    S = int(rng.choice([1, 2, 3, 5, 8, 16]))
    return dict(D=D, G=G, Hkv=Hkv, P=P, lens=tuple(int(x) for x in lens), S=S)


def config(k: int, c: dict) -> W.Config:
    lens, P = c["lens"], c["P"]
    return W.custom_config(seed_id=7100 + k, name=f"random{k}", B=len(lens), Hq=c["G"] * c["Hkv"],
                           Hkv=c["Hkv"], D=c["D"], P=P, num_pages=-(-sum(lens) // P) + len(lens) + 3,
                           seq_lens=lens)


def fused_rows(inp):
    """slot_mapping and new K/V rows with one entry per sequence, as the fused
    step takes them.  The inputs carry rows for the non-empty sequences only;
    an empty sequence's row goes to a spare page (owned by no sequence, not
    the page-table padding), one page per empty sequence so the slots stay
    distinct."""
    cfg, lens = inp.cfg, inp.seq_lens
    taken = set(int(x) for x in inp.page_table.ravel())
    spare = iter(p for p in range(cfg.num_pages) if p not in taken)
    slots = np.empty(cfg.B, np.int32)
    kn = np.empty((cfg.B, inp.k_new.shape[1]), inp.k_new.dtype)
    vn = np.empty_like(kn)
    j = 0
    for b in range(cfg.B):
        if lens[b] > 0:
            slots[b], kn[b], vn[b] = inp.slot_mapping[j], inp.k_new[j], inp.v_new[j]
            j += 1
        else:
            slots[b], kn[b], vn[b] = next(spare) * cfg.P, inp.k_new[0], inp.v_new[0]
    return slots, (kn, vn)


def test_draws_cover_the_envelope():
    """The sweep reaches every head size, group size and split count, page
    sizes 1 and >= 64, an odd kv-head count and an empty sequence."""
    cs = [draw(k) for k in range(N_CASES)]
    assert {c["D"] for c in cs} == {64, 128}
    assert {c["G"] for c in cs} == {1, 2, 4, 8}
    assert {c["S"] for c in cs} == {1, 2, 3, 5, 8, 16}
    assert any(c["P"] == 1 for c in cs) and any(c["P"] >= 64 for c in cs)
    assert any(c["Hkv"] == 3 for c in cs)
    assert any(0 in c["lens"] for c in cs)


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_decode_case(gpu_device, k):
    c = draw(k)
    cfg = config(k, c)
    S, L = c["S"], max(c["lens"])
    print(f"random case {k}: {cfg.describe()} num_splits {S}", flush=True)
    inp = W.make_inputs(cfg)
    kf, vf = inp.pools_after_store()
    ref, ref_lse = oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)

    # store, attention, merge: against the oracle
    st = DeviceStep(inp, gpu_device)
    (out, lse), o_p, l_p = st.step(splits=S, want_lse=True)
    torch.cuda.synchronize()
    check_attention(out, ref, f"random case {k}")
    gl = lse.cpu().numpy().astype(np.float64)
    empty = np.asarray(c["lens"]) == 0
    assert np.isneginf(gl[empty]).all() and np.isfinite(gl[~empty]).all()
    assert np.abs(gl[~empty] - ref_lse[~empty]).max(initial=0.0) <= 1e-4 * max(1.0, np.abs(ref_lse[~empty]).max(initial=0.0))

    # merged, and merged with its partials in the static scratch: the same bits
    m_out, m_lse = pkv.paged_decode_attn_merged(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, L, S,
                                                want_lse=True)
    s_out, s_lse = pkv.paged_decode_attn_merged_static(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens,
                                                       L, S, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(bits(m_out), bits(out)) and torch.equal(bits(m_lse), bits(lse)), "merged != attn + merge"
    assert torch.equal(bits(s_out), bits(out)) and torch.equal(bits(s_lse), bits(lse)), "static != merged"

    # the fused step: pools, output and lse as the store followed by the merged call
    slots, rows = fused_rows(inp)
    run_both(inp, gpu_device, S, slots=slots, new_rows=rows)

    # q rotated in the prologue: the attention on the oracle-rotated q, bit for bit
    _, qpos, kr, vr, q_rot = rotated_step(inp)
    _, _, cd, sd = tables(gpu_device, max(L, 1), cfg.D)
    rt = DeviceStep(inp, gpu_device, pools=(kr, vr))
    o1, l1 = pkv.paged_decode_attn(rt.q, rt.k_pool, rt.v_pool, rt.page_table, rt.seq_lens, L, S,
                                   q_positions=i32_dev(qpos, gpu_device), rope_cos=cd, rope_sin=sd)
    o2, l2 = pkv.paged_decode_attn(bf16_dev(q_rot, gpu_device), rt.k_pool, rt.v_pool, rt.page_table,
                                   rt.seq_lens, L, S)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "rotated prologue != attention on rotated q"
