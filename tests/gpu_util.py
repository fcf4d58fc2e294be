"""Helpers of the GPU tests: move the generated numpy inputs to the device,
run the step through the C ABI, and compare with the oracle's fp64 results."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_gqa_store_amd as pkv
from paged_kv_gqa_store_amd import workloads as W

# Tolerance of the bf16 output against the fp64 oracle: the two absolute gates
# stated for this decode step (N(0,1) inputs), plus a relative-L2 gate, because
# at long context the output itself is only ~0.01 in magnitude and the
# absolute gates alone would not see a dropped split.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_L2 = 1e-2


def bf16_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def i32_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64_from_bf16(t: torch.Tensor) -> np.ndarray:
    return W.bf16_bits_to_f32(host_u16(t)).astype(np.float64)


class DeviceStep:
    """One decode step's inputs resident on the GPU."""

    def __init__(self, inp: W.Inputs, dev, pools=None, page_table=None, kernel: str = "mfma"):
        self.inp = inp
        self.dev = dev
        self.kernel = kernel
        k_pool, v_pool = (inp.k_pool, inp.v_pool) if pools is None else pools
        self.q = bf16_dev(inp.q, dev)
        self.k_pool = bf16_dev(k_pool, dev)
        self.v_pool = bf16_dev(v_pool, dev)
        self.page_table = i32_dev(inp.page_table if page_table is None else page_table, dev)
        self.seq_lens = i32_dev(inp.seq_lens, dev)
        self.slot_mapping = i32_dev(inp.slot_mapping, dev)
        self.k_new = bf16_dev(inp.k_new, dev)
        self.v_new = bf16_dev(inp.v_new, dev)

    def store(self):
        pkv.kv_store(self.k_pool, self.v_pool, self.k_new, self.v_new, self.slot_mapping)

    def attend(self, splits=None, want_lse=False):
        o_p, l_p = pkv.paged_decode_attn(self.q, self.k_pool, self.v_pool, self.page_table,
                                         self.seq_lens, self.inp.max_seq_len, splits,
                                         total_tokens=int(self.inp.seq_lens.sum()), kernel=self.kernel)
        res = pkv.decode_merge(o_p, l_p, want_lse=want_lse)
        return res, o_p, l_p

    def step(self, splits=None, want_lse=False):
        self.store()
        return self.attend(splits, want_lse)


def check_attention(out: torch.Tensor, ref: np.ndarray, what: str):
    g = host_f64_from_bf16(out)
    assert g.shape == ref.shape
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300)
    msg = f"{what}: max_abs {err.max():.3e} mean_abs {err.mean():.3e} rel_l2 {rel:.3e}"
    print(msg, flush=True)
    assert err.max() <= MAX_ABS, msg
    assert err.mean() <= MEAN_ABS, msg
    assert rel <= REL_L2, msg
    return err, rel
