"""The longest-first order of the (sequence, split) pairs at its edges, through
the C ABI, on both decode kernels, against the oracle: exactly 256 pairs (the
most the kernels rank), every split full (lengths that are multiples of the
chunk), every sequence with a partial split, a batch that is mostly empty
sequences, and 258 pairs (past the limit: launch order instead).  The order
changes which workgroup runs a pair, never its result, so every case also
matches the one-split result within one bf16 step."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import DeviceStep, check_attention, host_f64_from_bf16

pytestmark = pytest.mark.gpu


def lens_for(kind: str, B: int, S: int, chunk: int, rng) -> tuple:
    if kind == "full":            # every split of every sequence full, or empty
        n = rng.integers(0, S + 1, B)
        n[0] = S
        return tuple(int(x) * chunk for x in n)
    if kind == "partial":         # every sequence ends inside a split
        lens = rng.integers(0, S, B) * chunk + rng.integers(1, chunk, B)
        lens[0] = S * chunk - 1
        return tuple(int(x) for x in lens)
    if kind == "mostly_empty":    # one sequence in eight non-empty
        lens = np.where(rng.random(B) < 0.125, rng.integers(1, S * chunk + 1, B), 0)
        lens[1] = S * chunk
        return tuple(int(x) for x in lens)
    lens = rng.integers(0, S * chunk + 1, B)                          # "mixed"
    lens[0] = S * chunk
    return tuple(int(x) for x in lens)


CASES = [
    # (kind, B, S, G, D): B * S pairs
    ("full", 64, 4, 4, 128),
    ("partial", 64, 4, 4, 128),
    ("mostly_empty", 128, 2, 1, 64),
    ("mixed", 32, 8, 2, 64),
    ("mixed", 86, 3, 4, 64),          # 258 pairs: no ranking
]


@pytest.mark.parametrize("kind,B,S,G,D", CASES, ids=[f"{c[0]}-B{c[1]}-S{c[2]}-G{c[3]}" for c in CASES])
def test_ranking_edges(gpu_device, kind, B, S, G, D):
    P, chunk = 16, 48
    rng = np.random.Generator(np.random.PCG64(W.SEED_BASE + 7500 + B * S + G))
    lens = lens_for(kind, B, S, chunk, rng)
    Hkv = 8 if G == 1 else 2            # the row kernel at G = 1 (Hkv a multiple of 512 / D)
    cfg = W.custom_config(seed_id=7500 + B * S + G, name=f"rank_{kind}", B=B, Hq=G * Hkv, Hkv=Hkv, D=D,
                          P=P, num_pages=-(-sum(lens) // P) + B + 3, seq_lens=lens)
    inp = W.make_inputs(cfg)
    L = max(lens)                       # the longest sequence fixes the chunk
    assert pkv.split_chunk(L, S, P) == chunk
    print(f"ranking edge {kind}: {cfg.describe()} num_splits {S} ({B * S} pairs)", flush=True)
    st = DeviceStep(inp, gpu_device)
    st.store()
    out = pkv.paged_decode_attn_merged(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, L, S)
    one = pkv.paged_decode_attn_merged(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, L, 1)
    torch.cuda.synchronize()
    kf, vf = inp.pools_after_store()
    ref, _ = oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)
    check_attention(out, ref, f"ranking edge {kind} B{B} S{S}")
    a, b = host_f64_from_bf16(out), host_f64_from_bf16(one)
    assert (np.abs(a - b) <= np.abs(b) * 2.0 ** -7 + 1e-6).all(), "S splits and one split differ by more than one bf16 step"


@pytest.mark.parametrize("G,D", [(4, 128), (1, 64)])
def test_large_batch(gpu_device, G, D):
    """4096 sequences of 0-48 tokens (some empty): a grid of 4096 x Hkv x S
    workgroups in launch order (far past the ranking limit), on the
    matrix-core kernel (G = 4) and the row kernel (G = 1)."""
    rng = np.random.Generator(np.random.PCG64(W.SEED_BASE + 7600 + G))
    B, P = 4096, 16
    lens = rng.integers(0, 49, B)
    lens[0] = 48
    Hkv = 8
    cfg = W.custom_config(seed_id=7600 + G, name=f"large_batch_g{G}", B=B, Hq=G * Hkv, Hkv=Hkv, D=D, P=P,
                          num_pages=int((-(-lens // P)).sum()) + 8, seq_lens=tuple(int(x) for x in lens))
    inp = W.make_inputs(cfg)
    print(f"large batch: {cfg.describe()}", flush=True)
    kf, vf = inp.pools_after_store()
    ref, _ = oracle.paged_decode(inp.q, kf, vf, inp.page_table, inp.seq_lens)
    for S in (1, 3):
        st = DeviceStep(inp, gpu_device)
        out, _, _ = st.step(splits=S)
        torch.cuda.synchronize()
        check_attention(out, ref, f"large batch G{G} S{S}")
