"""The vocabulary-slice row gather on the GPU, through the C ABI, against the
oracle: bit-exact on every byte of the output."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import bf16_dev, host_u16, i32_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_llama3_embedding_slice_bit_exact(gpu_device, rank):
    cfg = W.IndexingConfig("llama3_8b_embed", 128256, 4096, 8, 4096)
    table, ids, start = W.make_indexing_inputs(cfg, rank)
    print(f"indexing rank {rank}: slice [{start}, {start + table.shape[0]}) x {cfg.hidden}, n {cfg.n}", flush=True)
    out = pkv.indexing(bf16_dev(table, gpu_device), i32_dev(ids, gpu_device), start)
    torch.cuda.synchronize()
    assert host_u16(out).tobytes() == oracle.indexing(table, ids, start).tobytes()


def test_slices_add_up_to_the_full_lookup(gpu_device):
    """The all-reduce identity the zero rows exist for, on the GPU: the per-rank
    outputs of a 4-way split sum (exactly: one nonzero term per row) to the
    lookup in the whole table."""
    rng = np.random.Generator(np.random.PCG64(5))
    vocab, hidden = 1000, 256
    full = torch.from_numpy(rng.standard_normal((vocab, hidden)).astype(np.float32)).to(gpu_device)
    ids = torch.from_numpy(rng.integers(0, vocab, 777).astype(np.int32)).to(gpu_device)
    total = torch.zeros((777, hidden), device=gpu_device)
    for start in range(0, vocab, 250):
        total += pkv.indexing(full[start:start + 250].contiguous(), ids, start)
    torch.cuda.synchronize()
    assert torch.equal(total, full[ids.long()])


@pytest.mark.parametrize("row_bytes,offset", [(2, 0), (6, 0), (16, 0), (24, 8), (128, 0), (2048, 4),
                                              (8192, 0), (8194, 2)])
def test_row_sizes_and_alignment(gpu_device, row_bytes, offset):
    rng = np.random.Generator(np.random.PCG64(row_bytes + offset))
    length, n, start = 53, 211, 17
    table = rng.integers(0, 256, (length, row_bytes), dtype=np.uint8)
    ids = rng.integers(start - 10, start + length + 10, n).astype(np.int32)
    # place the table and the output at a chosen byte offset from a 256-aligned base
    tb = torch.zeros(length * row_bytes + 256, dtype=torch.uint8, device=gpu_device)
    t = tb[offset:offset + length * row_bytes].view(length, row_bytes)
    t.copy_(torch.from_numpy(table))
    ob = torch.full((n * row_bytes + 256,), 0xA5, dtype=torch.uint8, device=gpu_device)
    o = ob[offset:offset + n * row_bytes].view(n, row_bytes)
    pkv.indexing(t, i32_dev(ids, gpu_device), start, out=o)
    torch.cuda.synchronize()
    assert o.cpu().numpy().tobytes() == oracle.indexing(table, ids, start).tobytes()
    # bytes around the output untouched
    assert (ob[:offset].cpu().numpy() == 0xA5).all() and (ob[offset + n * row_bytes:].cpu().numpy() == 0xA5).all()


def test_extreme_ids_and_empty(gpu_device):
    table = torch.arange(40, dtype=torch.int32, device=gpu_device).view(10, 4)
    ids = torch.tensor([-(1 << 31), -1, 0, 9, 10, (1 << 31) - 1, 5], dtype=torch.int32, device=gpu_device)
    out = pkv.indexing(table, ids, 0)
    torch.cuda.synchronize()
    assert out.cpu().numpy().tobytes() == oracle.indexing(table.cpu().numpy(), ids.cpu().numpy(), 0).tobytes()
    empty = pkv.indexing(table, torch.zeros(0, dtype=torch.int32, device=gpu_device), 0)
    assert empty.shape == (0, 4)
    none = pkv.indexing(table[:0], ids, 0)            # a rank with an empty slice: all zeros
    torch.cuda.synchronize()
    assert not none.any()
    with pytest.raises(RuntimeError):
        pkv.indexing(table, ids.long(), 0)
