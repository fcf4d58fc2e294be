"""Python face of the CPU oracle (``pkv_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are its only callers; the HIP library and its
Python binding never import it.  It shares no code with them.

Every routine works on numpy arrays: bf16 tensors travel as ``uint16`` bit
patterns and are widened exactly to fp64 inside the C code.  See the header of
``pkv_oracle.c`` for the passages each routine follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "pkv_oracle.c"
_LIB = _HERE / "liboracle.so"

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-shared", "-fPIC", "-Wall", "-Wextra"]


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (strict IEEE fp64: no fast-math, no FMA contraction)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(f".so.tmp{os.getpid()}")
        subprocess.run(["gcc", *CFLAGS, str(_SRC), "-o", str(tmp), "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


class use_library:
    """Temporarily route every call through another build of the oracle
    (the mutation tests compile deliberately broken copies and check that the
    pins catch them)."""

    def __init__(self, path):
        self.path = Path(path)

    def __enter__(self):
        global _lib
        self._saved = _lib
        _lib = None
        _load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False

_p = ctypes.c_void_p
_i64 = ctypes.c_int64


def _load(path: Path | None = None):
    global _lib
    if _lib is None:
        if path is None:
            build(force=False)
            path = _LIB
        lib = ctypes.CDLL(str(path))
        lib.oracle_kv_store.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _i64, _i64]
        lib.oracle_kv_store.restype = ctypes.c_int
        common = [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64]
        lib.oracle_paged_decode.argtypes = common + [_p, _p]
        lib.oracle_paged_decode.restype = ctypes.c_int
        lib.oracle_paged_decode_rows.argtypes = common + [_p, _i64, _p, _p]
        lib.oracle_paged_decode_rows.restype = ctypes.c_int
        lib.oracle_softmax_weights.argtypes = common + [_i64, _i64, _p]
        lib.oracle_softmax_weights.restype = ctypes.c_int
        lib.oracle_split_chunk.argtypes = [_i64, _i64, _i64]
        lib.oracle_split_chunk.restype = _i64
        lib.oracle_paged_decode_split.argtypes = common + [_i64, _i64, _p, _p]
        lib.oracle_paged_decode_split.restype = ctypes.c_int
        lib.oracle_merge.argtypes = [_p, _p, _i64, _i64, _i64, _p, _p]
        lib.oracle_merge.restype = None
        lib.oracle_paged_prefill.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                             ctypes.c_int, _p, _i64, _p, _p]
        lib.oracle_paged_prefill.restype = ctypes.c_int
        lib.oracle_rope.argtypes = [_p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _i64]
        lib.oracle_rope.restype = ctypes.c_int
        lib.oracle_indexing.argtypes = [_p, _p, _i64, _i64, _p, _i64, _i64]
        lib.oracle_indexing.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def num_threads() -> int:
    return _load().oracle_num_threads()


def kv_store(k_pool, v_pool, k_new, v_new, slot_mapping, row_elems=None):
    """Row scatter.  Pools are 2-D ``[num_slots, pool_stride]`` and new rows
    2-D ``[n, in_stride]`` of one dtype; the first ``row_elems`` elements of
    each row are copied.  Returns new pool arrays (the inputs are not touched)."""
    k_out = np.array(k_pool, copy=True, order="C")
    v_out = np.array(v_pool, copy=True, order="C")
    k_new = np.ascontiguousarray(k_new)
    v_new = np.ascontiguousarray(v_new)
    assert k_out.ndim == 2 and k_new.ndim == 2 and k_out.dtype == k_new.dtype
    assert k_out.shape == v_out.shape and k_new.shape == v_new.shape
    slots = _c(slot_mapping, np.int32)
    n = slots.shape[0]
    assert k_new.shape[0] == n
    it = k_out.itemsize
    row_elems = k_new.shape[1] if row_elems is None else row_elems
    rc = _load().oracle_kv_store(_ptr(k_out), _ptr(v_out), k_out.shape[0], k_out.shape[1] * it,
                                 _ptr(k_new), _ptr(v_new), k_new.shape[1] * it, _ptr(slots), n,
                                 row_elems * it)
    _check(rc, "kv_store")
    return k_out, v_out


def paged_prefill(q, k_pool, v_pool, page_table, kv_lens, qo_indptr, causal: bool = True, rows=None):
    """Prefill attention of packed query rows.  q uint16 ``[total_q, Hq, D]``,
    pools ``[num_pages, P, Hkv, D]``, page_table int32 ``[B, max_pages]``,
    kv_lens int32 ``[B]``, qo_indptr int32 ``[B+1]``.  Returns
    (out fp64 ``[total_q, Hq, D]``, lse fp64 ``[total_q, Hq]``), or with
    ``rows`` (pairs (packed row, head)) just those: ``[n, D]``, ``[n]``."""
    q = _c(q, np.uint16)
    k_pool = _c(k_pool, np.uint16)
    v_pool = _c(v_pool, np.uint16)
    pt = _c(page_table, np.int32)
    kl = _c(kv_lens, np.int32)
    qo = _c(qo_indptr, np.int32)
    total_q, Hq, D = q.shape
    num_pages, P, Hkv, D2 = k_pool.shape
    B = kl.shape[0]
    assert D2 == D and qo.shape == (B + 1,) and int(qo[-1]) == total_q and pt.shape[0] == B
    if rows is None:
        out = np.empty((total_q, Hq, D), np.float64)
        lse = np.empty((total_q, Hq), np.float64)
        r_ptr, n = None, 0
    else:
        r = _c(rows, np.int64).reshape(-1, 2)
        n = r.shape[0]
        out = np.empty((n, D), np.float64)
        lse = np.empty((n,), np.float64)
        r_ptr = _ptr(r)
    rc = _load().oracle_paged_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(pt), _ptr(kl), _ptr(qo),
                                      B, Hq, Hkv, D, P, pt.shape[1], int(bool(causal)), r_ptr, n,
                                      _ptr(out), _ptr(lse))
    _check(rc, "paged_prefill")
    return out, lse


def rope(x, positions, cos, sin, heads: int):
    """Rotary embedding of bf16 rows: ``x`` uint16 ``[n, heads*D]`` (or any
    shape with ``n`` leading rows of ``heads*D`` elements), ``positions`` int32
    ``[n]``, ``cos``/``sin`` float32 ``[rows, D/2]``.  Returns uint16 rows of
    the same shape (see ``oracle_rope`` for the rounding)."""
    x = _c(x, np.uint16)
    shape = x.shape
    n = shape[0]
    x2 = x.reshape(n, -1)
    D = x2.shape[1] // heads
    assert heads * D == x2.shape[1] and D % 2 == 0
    cos = _c(cos, np.float32)
    sin = _c(sin, np.float32)
    assert cos.shape == sin.shape and cos.shape[1] == D // 2
    pos = _c(positions, np.int32)
    assert pos.shape == (n,)
    out = np.empty_like(x2)
    rc = _load().oracle_rope(_ptr(out), _ptr(x2), n, heads, D, x2.shape[1], _ptr(pos), _ptr(cos),
                             _ptr(sin), cos.shape[0])
    _check(rc, "rope")
    return out.reshape(shape)


def indexing(weight, ids, start: int):
    """Row gather of a vocabulary slice: ``weight`` is the slice ``[length, row]``
    (any dtype), ``ids`` int32 ``[n]``; returns ``[n, row]`` with zero rows for
    ids outside ``[start, start + length)``."""
    weight = np.ascontiguousarray(weight)
    assert weight.ndim == 2
    ids = _c(ids, np.int32)
    n = ids.shape[0]
    out = np.empty((n, weight.shape[1]), weight.dtype)
    out.view(np.uint8)[...] = 0xA5   # canary: a row the routine fails to write shows
    _load().oracle_indexing(_ptr(out), _ptr(weight), weight.shape[0], weight.shape[1] * weight.itemsize,
                            _ptr(ids), n, start)
    return out


def _problem(q, k_pool, v_pool, page_table, seq_lens):
    q = _c(q, np.uint16)
    k_pool = _c(k_pool, np.uint16)
    v_pool = _c(v_pool, np.uint16)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    B, Hq, D = q.shape
    _, P, Hkv, D2 = k_pool.shape
    assert D2 == D and v_pool.shape == k_pool.shape and pt.shape[0] == B and sl.shape == (B,)
    keep = (q, k_pool, v_pool, pt, sl)
    args = [_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(pt), _ptr(sl), B, Hq, Hkv, D, P, pt.shape[1]]
    return keep, args, (B, Hq, Hkv, D, P)


def paged_decode(q, k_pool, v_pool, page_table, seq_lens):
    """Exact-definition attention.  q ``[B,Hq,D]`` bf16 bits, pools
    ``[num_pages,P,Hkv,D]`` bf16 bits.  Returns (out fp64 [B,Hq,D], lse fp64 [B,Hq])."""
    keep, args, (B, Hq, _, D, _) = _problem(q, k_pool, v_pool, page_table, seq_lens)
    out = np.empty((B, Hq, D), np.float64)
    lse = np.empty((B, Hq), np.float64)
    _check(_load().oracle_paged_decode(*args, _ptr(out), _ptr(lse)), "paged_decode")
    del keep
    return out, lse


def paged_decode_rows(q, k_pool, v_pool, page_table, seq_lens, rows):
    """Like :func:`paged_decode` for the listed (b, h) pairs only."""
    keep, args, (_, _, _, D, _) = _problem(q, k_pool, v_pool, page_table, seq_lens)
    rows = _c(rows, np.int64).reshape(-1, 2)
    out = np.empty((rows.shape[0], D), np.float64)
    lse = np.empty((rows.shape[0],), np.float64)
    _check(_load().oracle_paged_decode_rows(*args, _ptr(rows), rows.shape[0], _ptr(out), _ptr(lse)),
           "paged_decode_rows")
    del keep
    return out, lse


def softmax_weights(q, k_pool, v_pool, page_table, seq_lens, b, h):
    keep, args, _ = _problem(q, k_pool, v_pool, page_table, seq_lens)
    w = np.empty((int(np.asarray(seq_lens)[b]),), np.float64)
    _check(_load().oracle_softmax_weights(*args, b, h, _ptr(w)), "softmax_weights")
    del keep
    return w


def split_chunk(max_seq_len: int, num_splits: int, page_size: int) -> int:
    return int(_load().oracle_split_chunk(max_seq_len, num_splits, page_size))


def paged_decode_split(q, k_pool, v_pool, page_table, seq_lens, chunk, num_splits):
    """Split mode: (o_part fp64 [B,Hq,S,D], lse_part fp64 [B,Hq,S])."""
    keep, args, (B, Hq, _, D, _) = _problem(q, k_pool, v_pool, page_table, seq_lens)
    o = np.empty((B, Hq, num_splits, D), np.float64)
    lse = np.empty((B, Hq, num_splits), np.float64)
    _check(_load().oracle_paged_decode_split(*args, chunk, num_splits, _ptr(o), _ptr(lse)),
           "paged_decode_split")
    del keep
    return o, lse


def merge(o_part, lse_part):
    """fp64 log-sum-exp merge in ascending split order.  o_part ``[...,S,D]``,
    lse_part ``[...,S]`` -> (out ``[...,D]``, lse ``[...]``)."""
    o_part = _c(o_part, np.float64)
    lse_part = _c(lse_part, np.float64)
    S, D = o_part.shape[-2:]
    lead = o_part.shape[:-2]
    assert lse_part.shape == lead + (S,)
    rows = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (D,), np.float64)
    lse = np.empty(lead, np.float64)
    _load().oracle_merge(_ptr(o_part), _ptr(lse_part), rows, S, D, _ptr(out), _ptr(lse))
    return out, lse
