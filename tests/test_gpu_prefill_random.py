"""A seeded sweep over the shape envelope of the paged prefill, through the C
ABI, against the fp64 oracle.  Each case draws the head size, group size,
kv-head count (odd ones included), page size (1 to 256), causal or not, and
a batch of requests with ragged cached lengths: fresh prompts (q_len =
kv_len), chunks over a cached context, single rows and requests with no
query rows."""
import numpy as np
import pytest

from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import check_attention
from .test_gpu_prefill import check_lse, run

pytestmark = pytest.mark.gpu

N_CASES = 16
WORK_CAP = 10e9     # q.k and p.v FLOP per case (non-causal count), so the oracle takes ~1 s


def draw(k: int) -> dict:
    rng = np.random.Generator(np.random.PCG64(W.SEED_BASE + 7300 + k))
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    while G * Hkv > 32:
        G //= 2
    P = int(2 ** rng.integers(0, 9))
    B = int(rng.integers(1, 6))
    causal = bool(rng.integers(0, 2))
    kv = np.exp(rng.uniform(0.0, np.log(1500.0), B)).astype(np.int64) + 1
    u = rng.random(B)
    ql = np.where(u < 0.3, kv, np.where(u < 0.4, 0, rng.integers(1, kv + 1)))
    if ql.max() == 0:
        ql[0] = kv[0]
    while (ql * kv).sum() * G * Hkv * D * 4 > WORK_CAP:
        kv = np.maximum(kv // 2, 1)
        ql = np.minimum(ql, kv)
    return dict(D=D, G=G, Hkv=Hkv, P=P, causal=causal, q_lens=tuple(int(x) for x in ql),
                kv_lens=tuple(int(x) for x in kv))


def config(k: int, c: dict) -> W.PrefillConfig:
    kv = c["kv_lens"]
    return W.PrefillConfig(7300 + k, f"prefill_random{k}", c["G"] * c["Hkv"], c["Hkv"], c["D"], c["P"],
                           -(-sum(kv) // c["P"]) + len(kv) + 4, c["q_lens"], kv)


def test_draws_cover_the_envelope():
    cs = [draw(k) for k in range(N_CASES)]
    assert {c["D"] for c in cs} == {64, 128}
    assert {c["G"] for c in cs} == {1, 2, 4, 8}
    assert {c["causal"] for c in cs} == {True, False}
    assert any(c["P"] == 1 for c in cs) and any(c["P"] >= 64 for c in cs)
    assert any(c["Hkv"] == 3 for c in cs)
    assert any(0 in c["q_lens"] for c in cs)
    assert any(q == kv for c in cs for q, kv in zip(c["q_lens"], c["kv_lens"]))
    assert all(q <= kv for c in cs for q, kv in zip(c["q_lens"], c["kv_lens"]))


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_prefill_case(gpu_device, k):
    c = draw(k)
    cfg = config(k, c)
    print(f"random prefill case {k}: {cfg.describe()} causal={c['causal']}", flush=True)
    q, kp, vp, pt, kl, qo = W.make_prefill_inputs(cfg)
    out, lse = run(q, kp, vp, pt, kl, qo, gpu_device, c["causal"])
    ref, ref_lse = oracle.paged_prefill(q, kp, vp, pt, kl, qo, c["causal"])
    check_attention(out, ref, f"random prefill case {k}")
    check_lse(lse, ref_lse)
