"""The copy kernels that bound the store in bench.py (libpkv_bench.so): the
linear copy moves every byte, and the page-run copy of a bulk fill leaves the
pools exactly as pkv_kv_store does with the same rows and slots."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from paged_kv_gqa_store_amd import _lib
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import bf16_dev, host_u16, i32_dev

pytestmark = pytest.mark.gpu


def _stream():
    return torch.cuda.current_stream().cuda_stream


def test_linear_copy_moves_every_byte(gpu_device):
    rng = np.random.Generator(np.random.PCG64(11))
    for nbytes in (16, 4096 + 48, (1 << 22) + 16 * 257):
        src = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).to(gpu_device)
        dst = torch.zeros(nbytes + 16, dtype=torch.uint8, device=gpu_device)
        assert _lib.bench_lib().pkvb_copy_linear(dst.data_ptr(), src.data_ptr(), nbytes, _stream()) == 0
        torch.cuda.synchronize()
        assert torch.equal(dst[:nbytes], src) and int(dst[nbytes:].sum()) == 0


def test_page_run_copy_equals_the_store_on_a_bulk_fill(gpu_device):
    cfg = W.custom_config(name="runs", B=5, Hq=8, Hkv=2, D=64, P=16, num_pages=60,
                          seq_lens=(1, 16, 17, 200, 333))
    inp = W.make_inputs(cfg)
    k_rows, v_rows, slots = W.bulk_fill_rows(inp)
    src_row, dst_slot, rows = W.bulk_fill_runs(inp)
    assert rows.sum() == slots.shape[0]
    kp1, vp1 = bf16_dev(inp.k_pool, gpu_device), bf16_dev(inp.v_pool, gpu_device)
    kp2, vp2 = kp1.clone(), vp1.clone()
    kr, vr = bf16_dev(k_rows, gpu_device), bf16_dev(v_rows, gpu_device)
    pkv.kv_store(kp1, vp1, kr, vr, i32_dev(slots, gpu_device))
    n_slots = cfg.num_pages * cfg.P
    rb = cfg.row_elems * 2
    # the index tensors stay referenced until the copy has run
    rs, rd, rr = i32_dev(src_row, gpu_device), i32_dev(dst_slot, gpu_device), i32_dev(rows, gpu_device)
    st = _lib.bench_lib().pkvb_copy_page_runs(kp2.data_ptr(), vp2.data_ptr(), n_slots, kr.data_ptr(),
                                              vr.data_ptr(), kr.shape[0], rs.data_ptr(), rd.data_ptr(),
                                              rr.data_ptr(), rows.shape[0], rb, _stream())
    assert st == 0
    torch.cuda.synchronize()
    assert host_u16(kp1).tobytes() == host_u16(kp2).tobytes()
    assert host_u16(vp1).tobytes() == host_u16(vp2).tobytes()
