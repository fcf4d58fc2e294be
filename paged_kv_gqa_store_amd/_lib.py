"""Loads ``libpkv.so`` (built in-tree by ``paged_kv_gqa_store_amd.build``) with
ctypes and declares the signatures of ``include/pkv.h``.

There is no fallback: if the library is missing or does not export a symbol,
:func:`lib` raises ``RuntimeError``.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libpkv.so"

# (name, restype, argtypes) for every entry point of include/pkv.h
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
SIGNATURES = [
    ("pkv_kv_store", _i32, [_p, _p, _i64, _i64, _p, _p, _i64, _p, _i64, _i64, _i32, _p]),
    ("pkv_indexing", _i32, [_p, _p, _i64, _i64, _i32, _p, _i64, _i64, _p]),
    ("pkv_kv_store_rope", _i32, [_p, _p, _i64, _i64, _p, _p, _i64, _p, _i64, _i32, _i32, _p, _p, _p,
                                 _i32, _p]),
    ("pkv_paged_decode_attn_rope", _i32, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                          _i32, _i32, _f32, _p, _p, _p, _p, _p, _i32, _p]),
    ("pkv_paged_decode_attn", _i32, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _i32, _i32, _f32, _p, _p, _p]),
    ("pkv_decode_merge", _i32, [_p, _p, _i32, _i32, _i32, _i32, _p, _p, _p]),
    ("pkv_decode_step", _i32, [_p, _p, _p, _i64, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                               _i32, _i32, _i32, _f32, _p, _p, _p, _p, _p]),
    ("pkv_paged_decode_attn_merged", _i32, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _f32, _p, _p, _p, _p, _p]),
    ("pkv_paged_decode_attn_merged_static", _i32, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                                   _i32, _i32, _i32, _f32, _p, _p, _p]),
    ("pkv_prefill_plan", _i32, [_p, _i32, _p, _p, _p, _i32]),
    ("pkv_paged_prefill_attn", _i32, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _i32, _f32, _p, _p, _p]),
    ("pkv_paged_decode_attn_valu", _i32, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                          _i32, _i32, _f32, _p, _p, _p]),
    ("pkv_num_splits", _i32, [_i32, _i32, _i32, _i32, _i32]),
    ("pkv_num_splits_batch", _i32, [_i32, _i32, _i32, _i32, _i64, _i32, _i32]),
    ("pkv_split_chunk", _i32, [_i32, _i32, _i32]),
    ("pkv_status_str", ctypes.c_char_p, [_i32]),
]

_lib = None

BENCH_LIB_PATH = Path(__file__).resolve().parent / "libpkv_bench.so"
# include/pkv_bench.h: the copy kernels that bound the store (measurement only)
BENCH_SIGNATURES = [
    ("pkvb_copy_linear", _i32, [_p, _p, _i64, _p]),
    ("pkvb_copy_page_runs", _i32, [_p, _p, _i64, _p, _p, _i64, _p, _p, _p, _i64, _i64, _p]),
]
_bench_lib = None


def bench_lib() -> ctypes.CDLL:
    """libpkv_bench.so (bench.py's copy ceilings); raises if it is not built."""
    global _bench_lib
    if _bench_lib is None:
        if not BENCH_LIB_PATH.exists():
            raise RuntimeError(f"{BENCH_LIB_PATH} is not built; run `python -m paged_kv_gqa_store_amd.build`")
        handle = ctypes.CDLL(str(BENCH_LIB_PATH))
        for name, res, args in BENCH_SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _bench_lib = handle
    return _bench_lib


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m paged_kv_gqa_store_amd.build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(str(LIB_PATH))
        for name, res, args in SIGNATURES:
            try:
                fn = getattr(handle, name)
            except AttributeError as e:
                raise RuntimeError(f"{LIB_PATH} does not export {name}") from e
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().pkv_status_str(status).decode()
        raise RuntimeError(f"{what}: {msg} (status {status})")
