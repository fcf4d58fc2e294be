"""kv_store on the GPU, through the C ABI, against the oracle's per-row copy:
whole pools compared byte for byte (bit-exact is the only acceptable result)."""
import json
from pathlib import Path

import numpy as np
import pytest
import torch

import paged_kv_gqa_store_amd as pkv
from oracle import oracle
from paged_kv_gqa_store_amd import workloads as W

from .gpu_util import DeviceStep, bf16_dev, host_u16, i32_dev

pytestmark = pytest.mark.gpu
GOLDEN = Path(__file__).parent / "golden"


def _bytes_dev(a: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("wl", ["tiny_gqa", "llama3_8b_decode", "ragged_batch", "long_context", "mha_page1"])
def test_step_store_whole_pool_bit_exact(gpu_device, wl):
    inp = W.make_inputs(W.WORKLOADS[wl])
    print(f"store step {wl}: {inp.cfg.describe()}", flush=True)
    st = DeviceStep(inp, gpu_device)
    st.store()
    torch.cuda.synchronize()
    cfg = inp.cfg
    flat = lambda a: a.reshape(cfg.num_pages * cfg.P, cfg.row_elems)
    ko, vo = oracle.kv_store(flat(inp.k_pool), flat(inp.v_pool), inp.k_new, inp.v_new, inp.slot_mapping)
    assert host_u16(st.k_pool).tobytes() == ko.tobytes()
    assert host_u16(st.v_pool).tobytes() == vo.tobytes()


def _selfcheck(dev, pool_slots, rows, row_bytes, seed, dtype=np.uint8):
    rng = np.random.Generator(np.random.PCG64(seed))
    item = np.dtype(dtype).itemsize
    kc = rng.integers(0, 256, (pool_slots, row_bytes), dtype=np.uint8).view(dtype)
    vc = rng.integers(0, 256, (pool_slots, row_bytes), dtype=np.uint8).view(dtype)
    k = rng.integers(0, 256, (rows, row_bytes), dtype=np.uint8).view(dtype)
    v = rng.integers(0, 256, (rows, row_bytes), dtype=np.uint8).view(dtype)
    idx = rng.permutation(pool_slots)[:rows].astype(np.int32)
    ko, vo = oracle.kv_store(kc, vc, k, v, idx)
    tdt = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[item]
    conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view({1: np.uint8, 2: np.int16, 4: np.int32}[item])).to(dev)
    dk, dv, nk, nv = conv(kc), conv(vc), conv(k), conv(v)
    assert dk.dtype == tdt
    pkv.kv_store(dk, dv, nk, nv, i32_dev(idx, dev))
    torch.cuda.synchronize()
    return dk.cpu().numpy().tobytes() == ko.tobytes() and dv.cpu().numpy().tobytes() == vo.tobytes()


def test_store_selfcheck_shapes(gpu_device):
    """The two self-check shapes of the store page: 16-byte and element paths."""
    cases = json.loads((GOLDEN / "store_selfcheck_shapes.json").read_text())["cases"]
    a, b = cases
    assert _selfcheck(gpu_device, a["pool_slots"], a["rows"], a["row_bytes"], 11, np.uint16)
    assert _selfcheck(gpu_device, b["pool_slots"], b["rows"], b["row_bytes"], 12, np.uint16)
    assert _selfcheck(gpu_device, b["pool_slots"], b["rows"], b["row_bytes"], 13, np.uint8)


@pytest.mark.parametrize("row_bytes", [2, 16, 48, 128, 1000, 2048, 4096, 4112])
def test_store_row_sizes(gpu_device, row_bytes):
    dt = np.uint16 if row_bytes % 2 == 0 else np.uint8
    assert _selfcheck(gpu_device, 700, 333, row_bytes, row_bytes, dt)


def test_store_strided_and_misaligned(gpu_device):
    """Row strides larger than the row, and a base offset that forbids 16-byte units."""
    rng = np.random.Generator(np.random.PCG64(21))
    pool = rng.integers(-2**15, 2**15, (400, 136), dtype=np.int16)
    new = rng.integers(-2**15, 2**15, (50, 144), dtype=np.int16)
    idx = rng.permutation(400)[:50].astype(np.int32)
    for off in [0, 1, 4]:   # element offsets of the views' base pointers
        dk = torch.from_numpy(pool.copy()).to(gpu_device)
        dv = torch.from_numpy(pool[::-1].copy()).to(gpu_device)
        dn = torch.from_numpy(new.copy()).to(gpu_device)
        kview = dk[:, off:off + 128]
        vview = dv[:, off:off + 128]
        nview = dn[:, off:off + 128]
        pkv.kv_store(kview, vview, nview, nview, i32_dev(idx, gpu_device))
        torch.cuda.synchronize()
        ek = pool.copy()
        ek[idx, off:off + 128] = new[:, off:off + 128]
        ev = pool[::-1].copy()
        ev[idx, off:off + 128] = new[:, off:off + 128]
        assert (dk.cpu().numpy() == ek).all() and (dv.cpu().numpy() == ev).all(), off


@pytest.mark.parametrize("wl", ["tiny_gqa", "llama3_8b_decode", "mha_page1"])
def test_bulk_fill_bit_exact(gpu_device, wl):
    """Every position of every sequence stored in one call (the bandwidth workload)."""
    inp = W.make_inputs(W.WORKLOADS[wl])
    cfg = inp.cfg
    k_rows, v_rows, slots = W.bulk_fill_rows(inp)
    print(f"bulk fill {wl}: {slots.shape[0]} rows", flush=True)
    flat = lambda a: a.reshape(cfg.num_pages * cfg.P, cfg.row_elems)
    dk = bf16_dev(flat(inp.k_pool), gpu_device)
    dv = bf16_dev(flat(inp.v_pool), gpu_device)
    pkv.kv_store(dk, dv, bf16_dev(k_rows, gpu_device), bf16_dev(v_rows, gpu_device), i32_dev(slots, gpu_device))
    torch.cuda.synchronize()
    ko, vo = oracle.kv_store(flat(inp.k_pool), flat(inp.v_pool), k_rows, v_rows, slots)
    assert host_u16(dk).tobytes() == ko.tobytes()
    assert host_u16(dv).tobytes() == vo.tobytes()


def test_out_of_range_slot_is_skipped(gpu_device):
    pool = np.arange(64 * 64, dtype=np.int16).reshape(64, 64)
    dk = torch.from_numpy(pool.copy()).to(gpu_device)
    dv = torch.from_numpy(pool.copy()).to(gpu_device)
    rows = torch.full((3, 64), 7, dtype=torch.int16, device=gpu_device)
    pkv.kv_store(dk, dv, rows, rows, i32_dev(np.array([5, 64, -1], np.int32), gpu_device))
    torch.cuda.synchronize()
    exp = pool.copy()
    exp[5] = 7
    assert (dk.cpu().numpy() == exp).all() and (dv.cpu().numpy() == exp).all()


def test_store_empty_and_errors(gpu_device):
    dk = torch.zeros((8, 16), dtype=torch.int16, device=gpu_device)
    rows = torch.zeros((0, 16), dtype=torch.int16, device=gpu_device)
    pkv.kv_store(dk, dk, rows, rows, torch.zeros(0, dtype=torch.int32, device=gpu_device))
    with pytest.raises(RuntimeError):
        pkv.kv_store(dk, dk, dk, dk, torch.zeros(8, dtype=torch.int64, device=gpu_device))
