"""The C-ABI library without a GPU: it loads, exports every symbol that
include/pkv.h declares, and its host-only logic and argument validation behave
(no call here reaches a kernel launch)."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

from oracle import oracle
from paged_kv_gqa_store_amd import _lib

ROOT = Path(__file__).resolve().parents[1]
HEADER = (ROOT / "include" / "pkv.h").read_text()

OK, NULL, SHAPE, UNSUP, ALIGN, SCRATCH = 0, -1, -2, -3, -4, -6


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def declared_symbols():
    return sorted(set(re.findall(r"^\S.*?\b(pkv_[a-z_0-9]+)\s*\(", HEADER, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted(["pkv_kv_store", "pkv_paged_decode_attn", "pkv_decode_merge",
                                         "pkv_num_splits", "pkv_num_splits_batch", "pkv_split_chunk",
                                         "pkv_status_str", "pkv_indexing", "pkv_kv_store_rope",
                                         "pkv_paged_decode_attn_rope", "pkv_paged_decode_attn_valu",
                                         "pkv_prefill_plan", "pkv_paged_prefill_attn",
                                         "pkv_paged_decode_attn_merged", "pkv_decode_step",
                                         "pkv_paged_decode_attn_merged_static"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert {s[0] for s in _lib.SIGNATURES} == set(declared_symbols())


def test_contracted_split_count_signature():
    """pkv_num_splits takes (B, Hkv, max_seq_len, page_size, num_cus), as the
    boundary contract states; the form with the group size and token count is
    pkv_num_splits_batch."""
    decl = re.search(r"int32_t pkv_num_splits\((.*?)\);", HEADER, flags=re.S).group(1)
    names = [a.split()[-1] for a in decl.replace("\n", " ").split(",")]
    assert names == ["B", "Hkv", "max_seq_len", "page_size", "num_cus"]
    decl = re.search(r"int32_t pkv_num_splits_batch\((.*?)\);", HEADER, flags=re.S).group(1)
    names = [a.split()[-1] for a in decl.replace("\n", " ").split(",")]
    assert names == ["B", "Hq", "Hkv", "max_seq_len", "total_tokens", "page_size", "num_cus"]


def test_bench_library_exports_its_header():
    text = (ROOT / "include" / "pkv_bench.h").read_text()
    names = sorted(set(re.findall(r"^\S.*?\b(pkvb_[a-z_0-9]+)\s*\(", text, flags=re.M)))
    assert names == ["pkvb_copy_linear", "pkvb_copy_page_runs"]
    blib = _lib.bench_lib()
    assert {s[0] for s in _lib.BENCH_SIGNATURES} == set(names)
    p = ctypes.c_void_p(256)
    # argument checks return before any launch
    assert blib.pkvb_copy_linear(p, p, 0, None) == OK
    assert blib.pkvb_copy_linear(p, p, 24, None) == SHAPE
    assert blib.pkvb_copy_linear(None, p, 32, None) == NULL
    assert blib.pkvb_copy_linear(ctypes.c_void_p(264), p, 32, None) == ALIGN
    assert blib.pkvb_copy_page_runs(p, p, 10, p, p, 10, p, p, p, 0, 2048, None) == OK
    assert blib.pkvb_copy_page_runs(p, p, 10, p, p, 10, p, p, p, 3, 2047, None) == SHAPE
    assert blib.pkvb_copy_page_runs(p, p, 10, p, p, 10, None, p, p, 3, 2048, None) == NULL


def test_status_strings(lib):
    for code in [OK, NULL, SHAPE, UNSUP, ALIGN, -5, SCRATCH, 7]:
        assert lib.pkv_status_str(code)


def test_split_heuristic_on_the_five_workloads(lib):
    # B, Hq, Hkv, max_seq_len, total_tokens, page_size -> S at 256 CUs
    cases = {(2, 4, 1, 100, 137, 16): 1,            # tiny, ragged: capped by ceil(100 / 256)
             (32, 32, 8, 4096, 32 * 4096, 16): 1,   # uniform: 256 streams fill 256 CUs
             (64, 32, 8, 8192, 281358, 16): 4,      # ragged: splits of at most 2048 positions
             (4, 64, 8, 65536, 4 * 65536, 16): 16,  # uniform, G = 8: two workgroups per CU
             (128, 16, 16, 2048, 128 * 2048, 1): 1}
    for args, s in cases.items():
        assert lib.pkv_num_splits_batch(*args, 256) == s, args
    # the same shapes without a token count are treated as ragged
    assert lib.pkv_num_splits_batch(32, 32, 8, 4096, -1, 16, 256) == 2
    assert lib.pkv_num_splits_batch(4, 64, 8, 65536, -1, 16, 256) == 32


def test_contracted_split_count_formula(lib):
    """Without Hq and the token count: one workgroup per (sequence, kv head,
    split), ragged lengths."""
    for B in [1, 2, 4, 32, 64, 128, 500]:
        for Hkv in [1, 8, 16]:
            for L in [0, 1, 100, 255, 256, 2049, 4096, 8192, 65536, 100000]:
                for P in [1, 16]:
                    s = lib.pkv_num_splits(B, Hkv, L, P, 256)
                    cap = min(1024, max(1, -(-L // 256)))
                    assert s == max(1, min(cap, max(-(-256 // (B * Hkv)), -(-L // 2048))))
                    if Hkv == 1:   # G = 1 with one kv head: no head blocks, the batch form agrees
                        assert s == lib.pkv_num_splits_batch(B, Hkv, Hkv, L, -1, P, 256)


def test_batch_split_count_counts_head_blocks_for_one_q_head_per_kv_head(lib):
    # 16 sequences x 16 kv heads, one q head each: 32 row-kernel workgroups per split
    assert lib.pkv_num_splits_batch(16, 16, 16, 4096, 16 * 4096, 1, 256) == 8
    # the same heads in groups of 4 q heads: 256 workgroups per split
    assert lib.pkv_num_splits_batch(16, 64, 16, 4096, 16 * 4096, 1, 256) == 1
    assert lib.pkv_num_splits_batch(16, 12, 12, 4096, 16 * 4096, 1, 256) == 6   # 12 % 8: blocks of 4
    assert lib.pkv_num_splits(32, 8, 4096, 16, 256) == 2
    assert lib.pkv_num_splits(0, 8, 10, 16, 256) == SHAPE
    assert lib.pkv_num_splits(1, 0, 10, 16, 256) == SHAPE
    assert lib.pkv_num_splits(1, 8, -1, 16, 256) == SHAPE
    assert lib.pkv_num_splits(1, 8, 10, 12, 256) == SHAPE
    assert lib.pkv_num_splits(1, 8, 10, 16, 0) == SHAPE


def test_split_heuristic_properties(lib):
    for B in [1, 3, 32, 500]:
        for Hq, Hkv in [(1, 1), (8, 1), (32, 8), (64, 8)]:
            for L in [0, 1, 255, 256, 2049, 100000]:
                cap = max(1, -(-L // 256))
                for total in [-1, B * L, B * L // 2]:
                    s = lib.pkv_num_splits_batch(B, Hq, Hkv, L, total, 16, 256)
                    assert 1 <= s <= min(cap, 1024)
                    if L > 0 and (total < 0 or 10 * total < 9 * B * L):
                        assert s >= min(-(-L // 2048), cap)
    assert lib.pkv_num_splits_batch(0, 8, 8, 10, -1, 16, 256) == SHAPE
    assert lib.pkv_num_splits_batch(1, 8, 8, 10, -1, 12, 256) == SHAPE
    assert lib.pkv_num_splits_batch(1, 12, 8, 10, -1, 16, 256) == SHAPE


def test_split_chunk_agrees_with_the_oracle_reading(lib):
    for L in [1, 15, 16, 17, 100, 4096, 65536, 8191, 123457]:
        for S in [1, 2, 3, 4, 7, 32, 1024]:
            for P in [1, 2, 16, 64]:
                assert lib.pkv_split_chunk(L, S, P) == oracle.split_chunk(L, S, P)
    assert lib.pkv_split_chunk(0, 4, 16) == 0
    assert lib.pkv_split_chunk(10, 0, 16) == SHAPE


def test_store_validation(lib):
    p = ctypes.c_void_p(16)
    assert lib.pkv_kv_store(p, p, 10, 8, p, p, 8, p, 0, 8, 2, None) == OK           # n == 0: no launch
    assert lib.pkv_kv_store(None, p, 10, 8, p, p, 8, p, 3, 8, 2, None) == NULL
    assert lib.pkv_kv_store(p, p, 10, 8, p, p, 8, None, 3, 8, 2, None) == NULL
    assert lib.pkv_kv_store(p, p, 10, 8, p, p, 8, p, -1, 8, 2, None) == SHAPE
    assert lib.pkv_kv_store(p, p, 10, 8, p, p, 8, p, 3, 9, 2, None) == SHAPE        # row > stride
    assert lib.pkv_kv_store(p, p, 10, 8, p, p, 8, p, 3, 8, 3, None) == UNSUP


def test_indexing_validation(lib):
    p = ctypes.c_void_p(16)
    assert lib.pkv_indexing(p, p, 10, 8, 2, p, 0, 0, None) == OK                # n == 0: no launch
    assert lib.pkv_indexing(None, p, 10, 8, 2, p, 3, 0, None) == NULL
    assert lib.pkv_indexing(p, None, 10, 8, 2, p, 3, 0, None) == NULL
    assert lib.pkv_indexing(p, p, 10, 8, 2, None, 3, 0, None) == NULL
    assert lib.pkv_indexing(p, p, -1, 8, 2, p, 3, 0, None) == SHAPE
    assert lib.pkv_indexing(p, p, 10, 8, 2, p, -3, 0, None) == SHAPE
    assert lib.pkv_indexing(p, p, 10, 8, 3, p, 3, 0, None) == UNSUP


def test_rope_validation(lib):
    p, f = ctypes.c_void_p(256), ctypes.c_void_p(512)
    # pools/rows of 1 head x 64, 16-byte aligned; tables of 10 rows
    ok = lambda **kw: lib.pkv_kv_store_rope(*[kw.get(k, d) for k, d in [
        ("kp", p), ("vp", p), ("slots_n", 100), ("ps", 64), ("kn", p), ("vn", p), ("is_", 64),
        ("sm", p), ("n", 3), ("Hkv", 1), ("D", 64), ("pos", p), ("c", f), ("s", f), ("rows", 10)]], None)
    assert ok(n=0) == OK
    assert ok(pos=None) == NULL
    assert ok(c=None) == NULL
    assert ok(rows=0) == SHAPE
    assert ok(D=60) == SHAPE
    assert ok(c=ctypes.c_void_p(516)) == ALIGN
    assert ok(kp=ctypes.c_void_p(258)) == ALIGN
    assert ok(ps=63) == SHAPE


def test_prefill_plan_reproduces_the_worked_example(lib):
    import json
    g = json.loads((ROOT / "tests" / "golden" / "prefill_schedule_example.json").read_text())
    assert g["tile_rows"] == 64
    q_lens = np.array(g["q_lens"], np.int32)
    B = len(q_lens)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    qo = np.zeros(B + 1, np.int32)
    assert lib.pkv_prefill_plan(ptr(q_lens), B, ptr(qo), None, None, 0) == 6   # size query
    tb, ti = np.full(6, -1, np.int32), np.full(6, -1, np.int32)
    assert lib.pkv_prefill_plan(ptr(q_lens), B, ptr(qo), ptr(tb), ptr(ti), 6) == 6
    assert qo.tolist() == g["qo_indptr"]
    assert tb.tolist() == g["q_tile_to_batch"] and ti.tolist() == g["q_tile_to_index"]
    assert lib.pkv_prefill_plan(ptr(q_lens), B, ptr(qo), ptr(tb), ptr(ti), 5) == SHAPE
    zero = np.array([0, 64, 65], np.int32)
    assert lib.pkv_prefill_plan(ptr(zero), 3, ptr(qo), ptr(tb), ptr(ti), 6) == 3   # empty request: no tile
    assert tb[:3].tolist() == [1, 2, 2] and ti[:3].tolist() == [0, 0, 1]


def _attn(lib, fn="pkv_paged_decode_attn", **kw):
    p = ctypes.c_void_p(256)
    a = dict(q=p, k=p, v=p, pt=p, sl=p, B=2, Hq=8, Hkv=2, D=128, P=16, pages=10, mp=4, L=64, S=2,
             scale=0.088, o=p, lse=p)
    a.update(kw)
    return getattr(lib, fn)(a["q"], a["k"], a["v"], a["pt"], a["sl"], a["B"], a["Hq"], a["Hkv"],
                            a["D"], a["P"], a["pages"], a["mp"], a["L"], a["S"], a["scale"],
                            a["o"], a["lse"], None)


@pytest.mark.parametrize("fn", ["pkv_paged_decode_attn", "pkv_paged_decode_attn_valu"])
def test_attention_validation(lib, fn):
    def attn(lib, **kw):
        return _attn(lib, fn, **kw)

    assert attn(lib, B=0) == OK
    assert attn(lib, q=None) == NULL
    assert attn(lib, lse=None) == NULL
    assert attn(lib, Hq=7) == SHAPE
    assert attn(lib, D=96) == UNSUP
    assert attn(lib, Hq=32) == UNSUP            # G = 16
    assert attn(lib, P=12) == UNSUP
    assert attn(lib, L=65) == SHAPE             # beyond max_pages * P
    assert attn(lib, S=0) == SHAPE
    assert attn(lib, S=1025) == SHAPE
    assert attn(lib, scale=0.0) == SHAPE
    assert attn(lib, q=ctypes.c_void_p(258)) == ALIGN
    assert attn(lib, k=ctypes.c_void_p(264)) == ALIGN


def _merged(lib, out=ctypes.c_void_p(256), lse_out=None, **kw):
    p = ctypes.c_void_p(256)
    a = dict(q=p, k=p, v=p, pt=p, sl=p, B=2, Hq=8, Hkv=2, D=128, P=16, pages=10, mp=4, L=64, S=2,
             scale=0.088, o=p, lse=p)
    a.update(kw)
    return lib.pkv_paged_decode_attn_merged(a["q"], a["k"], a["v"], a["pt"], a["sl"], a["B"], a["Hq"],
                                            a["Hkv"], a["D"], a["P"], a["pages"], a["mp"], a["L"], a["S"],
                                            a["scale"], a["o"], a["lse"], out, lse_out, None)


def test_merged_attention_validation(lib):
    # the attention's checks, then the output's; nothing launches on an error
    assert _merged(lib, B=0) == OK
    assert _merged(lib, q=None) == NULL
    assert _merged(lib, D=96) == UNSUP
    assert _merged(lib, S=0) == SHAPE
    assert _merged(lib, out=None) == NULL
    assert _merged(lib, out=ctypes.c_void_p(258)) == ALIGN
    assert _merged(lib, o=None) == NULL            # several splits need the partials
    assert _merged(lib, lse=None) == NULL
    assert _merged(lib, o=ctypes.c_void_p(260)) == ALIGN
    assert _merged(lib, S=1, o=None, lse=None, out=None) == NULL    # one split: only out is needed
    assert _merged(lib, S=1, o=None, lse=None, out=ctypes.c_void_p(264)) == ALIGN


def _static(lib, out=ctypes.c_void_p(256), **kw):
    p = ctypes.c_void_p(256)
    a = dict(q=p, k=p, v=p, pt=p, sl=p, B=2, Hq=8, Hkv=2, D=128, P=16, pages=10, mp=4, L=64, S=2,
             scale=0.088)
    a.update(kw)
    return lib.pkv_paged_decode_attn_merged_static(a["q"], a["k"], a["v"], a["pt"], a["sl"], a["B"], a["Hq"],
                                                   a["Hkv"], a["D"], a["P"], a["pages"], a["mp"], a["L"],
                                                   a["S"], a["scale"], out, None, None)


def test_static_scratch_validation(lib):
    """The no-allocation call checks its arguments like the merged call, and
    rejects partials beyond its 16 MiB scratch before touching the GPU."""
    assert _static(lib, B=0) == OK
    assert _static(lib, q=None) == NULL
    assert _static(lib, out=None) == NULL
    assert _static(lib, out=ctypes.c_void_p(258)) == ALIGN
    assert _static(lib, D=96) == UNSUP
    assert _static(lib, S=0) == SHAPE
    # B * Hq * S * (D + 1) floats against 4 Mi: 128 * 32 * 8 * 129 = 4.2 Mi does not fit
    big = dict(B=128, Hq=32, Hkv=8, pages=100000, mp=512, L=8192)
    assert _static(lib, S=8, **big) == SCRATCH
    assert _static(lib, S=1024, B=64, Hq=64, Hkv=8, pages=100000, mp=512, L=8192) == SCRATCH
    assert _static(lib, S=1025) == SHAPE


def _step(lib, kn=ctypes.c_void_p(256), stride=256, slots=ctypes.c_void_p(256), out=ctypes.c_void_p(256), **kw):
    p = ctypes.c_void_p(256)
    a = dict(q=p, k=p, v=p, pt=p, sl=p, B=2, Hq=8, Hkv=2, D=128, P=16, pages=10, mp=4, L=64, S=1,
             scale=0.088, o=None, lse=None)
    a.update(kw)
    return lib.pkv_decode_step(a["q"], kn, p, stride, slots, a["k"], a["v"], a["pt"], a["sl"], a["B"], a["Hq"],
                               a["Hkv"], a["D"], a["P"], a["pages"], a["mp"], a["L"], a["S"], a["scale"],
                               a["o"], a["lse"], out, None, None)


def test_decode_step_validation(lib):
    assert _step(lib, B=0) == OK
    assert _step(lib, kn=None) == NULL
    assert _step(lib, slots=None) == NULL
    assert _step(lib, out=None) == NULL
    assert _step(lib, stride=255) == SHAPE         # shorter than a row of Hkv*D
    assert _step(lib, stride=260) == ALIGN         # rows not 16-byte aligned
    assert _step(lib, kn=ctypes.c_void_p(264)) == ALIGN
    assert _step(lib, S=2) == NULL                 # several splits need the partials
    assert _step(lib, D=96) == UNSUP


def test_merge_validation(lib):
    p = ctypes.c_void_p(256)
    assert lib.pkv_decode_merge(p, p, 0, 8, 128, 2, p, None, None) == OK
    assert lib.pkv_decode_merge(None, p, 2, 8, 128, 2, p, None, None) == NULL
    assert lib.pkv_decode_merge(p, p, 2, 8, 96, 2, p, None, None) == UNSUP
    assert lib.pkv_decode_merge(p, p, 2, 8, 128, 0, p, None, None) == SHAPE
    assert lib.pkv_decode_merge(p, p, 2, 8, 128, 2, ctypes.c_void_p(258), None, None) == ALIGN


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", tmp_path / "missing.so")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()
