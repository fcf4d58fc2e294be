"""Paged prefill on the GPU through the C ABI against the fp64 oracle: ragged
packed queries, causal and not, every supported head size, group size and
page size, the full Llama-3-8B-shaped chunk on sampled rows, and the bitwise
invariants (placement, determinism)."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import MAX_ABS, MEAN_ABS, REL_L2, bf16_dev, check_attention, host_f64_from_bf16, i32_dev

pytestmark = pytest.mark.gpu


def run(q, kp, vp, pt, kl, qo, dev, causal=True, want_lse=True):
    q_lens = np.diff(qo)
    plan = pkv.prefill_plan(q_lens, dev)
    res = pkv.paged_prefill_attn(bf16_dev(q, dev), bf16_dev(kp, dev), bf16_dev(vp, dev), i32_dev(pt, dev),
                                 i32_dev(kl, dev), plan, causal=causal, want_lse=want_lse)
    torch.cuda.synchronize()
    return res


def check_lse(lse, ref):
    g = lse.cpu().numpy().astype(np.float64)
    assert np.abs(g - ref).max() <= 1e-3 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("causal", [True, False])
def test_page_example_batch(gpu_device, causal):
    cfg = W.PREFILL["ragged_chunks"]
    print(f"prefill {cfg.name} causal={causal}: {cfg.describe()}", flush=True)
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    out, lse = run(q, kp, vp, pt, kl, qo, gpu_device, causal)
    ref, ref_lse = oracle.paged_prefill(q, kp, vp, pt, kl, qo, causal)
    check_attention(out, ref, f"prefill {cfg.name} causal={causal}")
    check_lse(lse, ref_lse)


@pytest.mark.parametrize("D,G,P", [(64, 1, 1), (64, 2, 16), (64, 8, 4), (128, 1, 16), (128, 4, 16),
                                   (128, 8, 1), (128, 2, 256), (64, 4, 1024), (128, 8, 512)])
def test_shapes_and_ragged_tails(gpu_device, D, G, P):
    Hkv = 2
    q_lens = (1, 63, 64, 65, 130, 7)
    kv_lens = (1, 63, 200, 65, 131, 500)
    cfg = W.PrefillConfig(0, f"d{D}g{G}p{P}", G * Hkv, Hkv, D, P,
                          -(-sum(kv_lens) // P) + len(kv_lens) + 4, q_lens, kv_lens)
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    for causal in (True, False):
        out, lse = run(q, kp, vp, pt, kl, qo, gpu_device, causal)
        ref, ref_lse = oracle.paged_prefill(q, kp, vp, pt, kl, qo, causal)
        check_attention(out, ref, f"prefill D{D} G{G} P{P} causal={causal}")
        check_lse(lse, ref_lse)


@pytest.mark.parametrize("D,P", [(128, 16), (128, 1), (64, 16), (64, 4)])
def test_one_head_per_kv_head_on_tile_pairs(gpu_device, D, P):
    """G = 1 with long requests (at least 8 host tiles of 64 rows per request
    on average) runs 128-row workgroups over pairs of host tiles.  The tile
    counts 21, 11, 2, 15 and 1 put request boundaries inside pairs (each side
    then runs as a job of its own) and leave a last tile alone."""
    Hkv = 3
    q_lens = (1300, 700, 65, 960, 1)
    kv_lens = (1300, 1500, 65, 2000, 9)
    assert sum(-(-q // 64) for q in q_lens) >= 8 * len(q_lens)
    cfg = W.PrefillConfig(0, f"pairs_d{D}_p{P}", Hkv, Hkv, D, P,
                          -(-sum(kv_lens) // P) + len(kv_lens) + 4, q_lens, kv_lens)
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    for causal in (True, False):
        print(f"prefill G=1 tile pairs D={D} P={P} causal={causal}: {cfg.describe()}", flush=True)
        out, lse = run(q, kp, vp, pt, kl, qo, gpu_device, causal)
        ref, ref_lse = oracle.paged_prefill(q, kp, vp, pt, kl, qo, causal)
        check_attention(out, ref, f"prefill G1 pairs D{D} P{P} causal={causal}")
        check_lse(lse, ref_lse)


@pytest.mark.parametrize("D,G,Hkv", [(128, 1, 16), (64, 2, 16), (128, 4, 16)])
def test_xcd_interleaved_work_order(gpu_device, D, G, Hkv):
    """With at least 8 host tiles per request on average and a multiple of 8
    kv-head groups, the groups of one XCD interleave their q chunks in the
    work order; every row must still be computed once and right."""
    q_lens, kv_lens = (700, 600), (900, 600)
    assert sum(-(-q // 64) for q in q_lens) >= 8 * len(q_lens)
    cfg = W.PrefillConfig(0, f"interleave_d{D}_g{G}_h{Hkv}", G * Hkv, Hkv, D, 16,
                          -(-sum(kv_lens) // 16) + len(kv_lens) + 4, q_lens, kv_lens)
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    print(f"prefill interleaved order D={D} G={G} Hkv={Hkv}: {cfg.describe()}", flush=True)
    out, lse = run(q, kp, vp, pt, kl, qo, gpu_device, True)
    ref, ref_lse = oracle.paged_prefill(q, kp, vp, pt, kl, qo, True)
    check_attention(out, ref, f"prefill interleaved D{D} G{G} Hkv{Hkv}")
    check_lse(lse, ref_lse)


@pytest.mark.parametrize("G", [1, 2, 4])
def test_empty_requests_in_the_batch(gpu_device, G):
    """Requests with no query rows (q_len = 0) among others get no Q tile, and
    the rows after them still find their own request."""
    Hkv, D, P = 2, 128, 16
    q_lens = (0, 37, 0, 64, 0, 1)
    kv_lens = (10, 100, 5, 64, 33, 20)
    cfg = W.PrefillConfig(0, f"empty_requests_g{G}", G * Hkv, Hkv, D, P,
                          -(-sum(kv_lens) // P) + len(kv_lens) + 4, q_lens, kv_lens)
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    for causal in (True, False):
        print(f"prefill with empty requests G={G} causal={causal}: {cfg.describe()}", flush=True)
        out, lse = run(q, kp, vp, pt, kl, qo, gpu_device, causal)
        ref, ref_lse = oracle.paged_prefill(q, kp, vp, pt, kl, qo, causal)
        check_attention(out, ref, f"prefill empty requests G{G} causal={causal}")
        check_lse(lse, ref_lse)


def test_batch_with_no_query_rows(gpu_device):
    """Every request empty: no tile, nothing launched, empty outputs."""
    cfg = W.PrefillConfig(0, "no_rows", 8, 2, 128, 16, 8, (0, 0), (5, 9))
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    out, lse = run(q, kp, vp, pt, kl, qo, gpu_device)
    assert tuple(out.shape) == (0, 8, 128) and tuple(lse.shape) == (0, 8)


@pytest.mark.parametrize("name", ["llama3_8b_chunked", "llama3_8b_fresh", "mha_fresh"])
def test_full_size_on_sampled_rows(gpu_device, name):
    cfg = W.PREFILL[name]
    print(f"prefill {name}: {cfg.describe()}", flush=True)
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    out, lse = run(q, kp, vp, pt, kl, qo, gpu_device, True)
    rng = np.random.Generator(np.random.PCG64(9))
    total_q = int(qo[-1])
    rows = np.stack([rng.integers(0, total_q, 48), rng.integers(0, cfg.Hq, 48)], 1)
    rows = np.concatenate([rows, [[0, 0], [total_q - 1, cfg.Hq - 1], [int(qo[1]) - 1, 3]]])
    ref, ref_lse = oracle.paged_prefill(q, kp, vp, pt, kl, qo, True, rows=rows)
    g = host_f64_from_bf16(out)[rows[:, 0], rows[:, 1]]
    err = np.abs(g - ref)
    rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
    print(f"{name}: sampled max_abs {err.max():.2e} mean_abs {err.mean():.2e} rel_l2 {rel:.2e}", flush=True)
    assert np.isfinite(g).all() and err.max() <= MAX_ABS and err.mean() <= MEAN_ABS and rel <= REL_L2
    gl = lse.cpu().numpy().astype(np.float64)[rows[:, 0], rows[:, 1]]
    assert np.abs(gl - ref_lse).max() <= 1e-3 * max(1.0, np.abs(ref_lse).max())
    # every output row finite
    assert torch.isfinite(out.float()).all()


def test_paged_equals_contiguous_and_deterministic(gpu_device):
    cfg = W.PREFILL["ragged_chunks"]
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    a = run(q, kp, vp, pt, kl, qo, gpu_device, True, want_lse=False)
    b = run(q, kp, vp, pt, kl, qo, gpu_device, True, want_lse=False)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the same sequences laid out contiguously, pages in order
    P = cfg.P
    n_pages = -(-kl.astype(np.int64) // P)
    order = np.concatenate([pt[i, :n_pages[i]] for i in range(cfg.B)])
    kc, vc = kp[order], vp[order]
    ptc = np.zeros_like(pt)
    starts = np.concatenate([[0], np.cumsum(n_pages)])
    for i in range(cfg.B):
        ptc[i, :n_pages[i]] = np.arange(starts[i], starts[i + 1])
    c = run(q, kc, vc, ptc, kl, qo, gpu_device, True, want_lse=False)
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_single_row_requests_match_the_decode_oracle(gpu_device):
    cfg = W.PrefillConfig(0, "rows1", 32, 8, 128, 16, 400, (1,) * 5, (1, 17, 300, 1024, 2000))
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    out, _ = run(q, kp, vp, pt, kl, qo, gpu_device, True)
    ref, _ = oracle.paged_decode(q, kp, vp, pt, kl)
    check_attention(out, ref, "prefill one row per request")


def test_bad_page_poisons_its_request_only(gpu_device):
    cfg = W.PREFILL["ragged_chunks"]
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    pt = pt.copy()
    pt[1, 0] = cfg.num_pages + 3
    out = run(q, kp, vp, pt, kl, qo, gpu_device, True, want_lse=False).float()
    assert torch.isnan(out[qo[1]:qo[2]]).all()
    assert torch.isfinite(out[:qo[1]]).all() and torch.isfinite(out[qo[2]:]).all()


@pytest.mark.parametrize("rate", [0.006, 0.05])
def test_scores_growing_along_positions(gpu_device, rate):
    """Keys aligned with their group's queries and growing along the positions
    make every row's running max climb from tile to tile: slowly (a few
    binades per 64 positions, so probabilities above 1 against an older max)
    or fast (the max moves on every tile)."""
    Hkv, G, D, P = 2, 4, 128, 16
    q_lens, kv_lens = (40, 200, 1), (300, 700, 129)
    cfg = W.PrefillConfig(0, f"growing{rate}", G * Hkv, Hkv, D, P,
                          -(-sum(kv_lens) // P) + len(kv_lens) + 4, q_lens, kv_lens)
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    as_f32 = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32)
    rng = np.random.Generator(np.random.PCG64(31))
    u = rng.standard_normal((Hkv, D)).astype(np.float32)
    qf = 0.3 * as_f32(q) + np.repeat(u, G, axis=0)[None]
    kf = as_f32(kp)
    for b in range(len(kv_lens)):
        t = np.arange(kv_lens[b])
        pages, slots = pt[b, t // P], t % P
        kf[pages, slots] = 0.3 * kf[pages, slots] + rate * t[:, None, None] * u[None]
    q, kp = W.to_bf16_bits(qf), W.to_bf16_bits(kf)
    for causal in (True, False):
        out, lse = run(q, kp, vp, pt, kl, qo, gpu_device, causal)
        ref, ref_lse = oracle.paged_prefill(q, kp, vp, pt, kl, qo, causal)
        check_attention(out, ref, f"prefill growing scores rate={rate} causal={causal}")
        check_lse(lse, ref_lse)


def test_page_table_entries_past_the_sequence_are_not_read(gpu_device):
    cfg = W.PREFILL["ragged_chunks"]
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    a = run(q, kp, vp, pt, kl, qo, gpu_device, True, want_lse=False)
    pt = pt.copy()
    for b in range(cfg.B):
        pt[b, -(-int(kl[b]) // cfg.P):] = -7          # out of the pool, but unused
    c = run(q, kp, vp, pt, kl, qo, gpu_device, True, want_lse=False)
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_prefill_errors(gpu_device):
    cfg = W.PREFILL["ragged_chunks"]
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    plan = pkv.prefill_plan(np.diff(qo), gpu_device)
    qd = bf16_dev(q, gpu_device)
    with pytest.raises(RuntimeError):     # q rows do not match the plan
        pkv.paged_prefill_attn(qd[:10], bf16_dev(kp, gpu_device), bf16_dev(vp, gpu_device),
                               i32_dev(pt, gpu_device), i32_dev(kl, gpu_device), plan)
    with pytest.raises(RuntimeError):     # head size 96 is not supported
        q96 = torch.zeros((qd.shape[0], qd.shape[1], 96), dtype=torch.bfloat16, device=gpu_device)
        k96 = torch.zeros((4, 16, 2, 96), dtype=torch.bfloat16, device=gpu_device)
        pkv.paged_prefill_attn(q96, k96, k96, i32_dev(pt, gpu_device), i32_dev(kl, gpu_device), plan)
