"""Python binding of libpkv: argument marshalling only.

Every function checks dtypes, devices and contiguity, passes raw device
pointers and the current HIP stream to the C ABI (``include/pkv.h``) and raises
``RuntimeError`` on a nonzero status.  All arithmetic of the decode step runs
in the library's HIP kernels; PyTorch only provides device memory and streams.
"""
from __future__ import annotations

import ctypes
import math
from typing import NamedTuple

import numpy as np
import torch

from ._lib import check, lib

_num_cus_cache: dict = {}


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise RuntimeError(msg)


def _on_gpu(*ts):
    dev = ts[0].device
    for t in ts:
        _require(t.is_cuda and t.device == dev, "all tensors must be on the same GPU")


def num_cus(device=None) -> int:
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    key = device.index
    if key not in _num_cus_cache:
        _num_cus_cache[key] = torch.cuda.get_device_properties(device).multi_processor_count
    return _num_cus_cache[key]


def num_splits(B: int, Hq: int, Hkv: int, max_seq_len: int, page_size: int,
               total_tokens: int = -1, n_cus: int | None = None) -> int:
    """The split-count heuristic of the library (host only,
    ``pkv_num_splits_batch``).  ``total_tokens`` is the sum of the sequence
    lengths if known (-1: unknown, treated as ragged)."""
    n_cus = num_cus() if n_cus is None else n_cus
    s = lib().pkv_num_splits_batch(B, Hq, Hkv, max_seq_len, total_tokens, page_size, n_cus)
    check(min(s, 0), "pkv_num_splits_batch")
    return s


def split_chunk(max_seq_len: int, num_splits: int, page_size: int) -> int:
    c = lib().pkv_split_chunk(max_seq_len, num_splits, page_size)
    check(min(c, 0), "pkv_split_chunk")
    return c


def _rows(t: torch.Tensor, name: str, pool: bool) -> torch.Tensor:
    """View a pool ([num_slots,row] or [num_pages,P,Hkv,D]) or a batch of new rows
    ([n,row] or [n,Hkv,D]) as 2-D rows, never copying (a copy would hide the writes)."""
    if t.dim() == 2:
        v = t
    elif pool and t.dim() == 4:
        v = t.view(t.shape[0] * t.shape[1], t.shape[2] * t.shape[3])
    elif not pool and t.dim() == 3:
        v = t.view(t.shape[0], t.shape[1] * t.shape[2])
    else:
        raise RuntimeError(f"{name}: unsupported rank {t.dim()}")
    _require(v.stride(1) == 1, f"{name}: rows must be contiguous")
    return v


def kv_store(k_pool: torch.Tensor, v_pool: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
             slot_mapping: torch.Tensor) -> None:
    """Scatter ``k_new[i]`` / ``v_new[i]`` into pool row ``slot_mapping[i]`` (in place).

    Pools: ``[num_slots, row]`` or ``[num_pages, page_size, Hkv, D]``; new rows:
    ``[n, row]`` or ``[n, Hkv, D]``.  Row strides may be anything; elements of
    a row must be contiguous."""
    _on_gpu(k_pool, v_pool, k_new, v_new, slot_mapping)
    _require(slot_mapping.dtype == torch.int32 and slot_mapping.dim() == 1 and slot_mapping.is_contiguous(),
             "slot_mapping must be a contiguous int32 vector")
    kp, vp = _rows(k_pool, "k_pool", True), _rows(v_pool, "v_pool", True)
    kn, vn = _rows(k_new, "k_new", False), _rows(v_new, "v_new", False)
    _require(kp.shape == vp.shape and kp.stride() == vp.stride(), "k_pool and v_pool must match")
    _require(kn.shape == vn.shape and kn.stride() == vn.stride(), "k_new and v_new must match")
    _require(kp.dtype == vp.dtype == kn.dtype == vn.dtype, "pool and rows must share a dtype")
    n = slot_mapping.shape[0]
    _require(kn.shape[0] == n, "one slot per new row")
    _require(kn.shape[1] == kp.shape[1], "new rows and pool rows must have the same length")
    st = lib().pkv_kv_store(kp.data_ptr(), vp.data_ptr(), kp.shape[0], kp.stride(0),
                            kn.data_ptr(), vn.data_ptr(), kn.stride(0), slot_mapping.data_ptr(), n,
                            kn.shape[1], kn.element_size(), _stream(kp))
    check(st, "pkv_kv_store")


def indexing(weight: torch.Tensor, ids: torch.Tensor, start: int = 0, out=None) -> torch.Tensor:
    """Embedding lookup in one rank's vocabulary slice: ``out[t] = weight[ids[t] - start]``,
    or a zero row when ``ids[t]`` lies outside ``[start, start + weight.shape[0])``.

    ``weight`` ``[length, row]`` contiguous (any dtype); ``ids`` int32 ``[n]``;
    returns ``[n, row]`` of ``weight``'s dtype."""
    _on_gpu(weight, ids)
    _require(weight.dim() == 2 and weight.is_contiguous(), "weight must be a contiguous 2-D table")
    _require(ids.dtype == torch.int32 and ids.dim() == 1 and ids.is_contiguous(),
             "ids must be a contiguous int32 vector")
    n, row = ids.shape[0], weight.shape[1]
    if out is None:
        out = torch.empty((n, row), dtype=weight.dtype, device=weight.device)
    _require(out.shape == (n, row) and out.dtype == weight.dtype and out.is_contiguous()
             and out.device == weight.device, "out must be contiguous [n, row] of weight's dtype")
    st = lib().pkv_indexing(out.data_ptr(), weight.data_ptr(), weight.shape[0], row,
                            weight.element_size(), ids.data_ptr(), n, start, _stream(weight))
    check(st, "pkv_indexing")
    return out


def _rope_tables(cos: torch.Tensor, sin: torch.Tensor, D: int, dev):
    _require(cos.dtype == torch.float32 and sin.dtype == torch.float32 and cos.is_contiguous()
             and sin.is_contiguous() and cos.shape == sin.shape and cos.dim() == 2
             and cos.shape[1] == D // 2, "rope tables must be contiguous fp32 [rows, D/2]")
    _require(cos.device == dev and sin.device == dev, "rope tables must be on the GPU of the data")


def kv_store_rope(k_pool, v_pool, k_new, v_new, slot_mapping, positions, rope_cos, rope_sin) -> None:
    """:func:`kv_store` of bf16 rows with every K row rotated by the rotary
    embedding of ``positions[i]`` on its way into the pool (V copied as is).

    Pools ``[num_pages, page_size, Hkv, D]``; new rows ``[n, Hkv, D]``;
    ``positions`` int32 ``[n]``; ``rope_cos``/``rope_sin`` fp32 ``[rows, D/2]``."""
    _on_gpu(k_pool, v_pool, k_new, v_new, slot_mapping, positions)
    _require(k_pool.dim() == 4 and k_new.dim() == 3, "pools [num_pages,P,Hkv,D], rows [n,Hkv,D]")
    _require(k_pool.dtype == v_pool.dtype == k_new.dtype == v_new.dtype == torch.bfloat16,
             "pools and rows must be bfloat16")
    _require(slot_mapping.dtype == torch.int32 and slot_mapping.dim() == 1 and slot_mapping.is_contiguous(),
             "slot_mapping must be a contiguous int32 vector")
    _require(positions.dtype == torch.int32 and positions.shape == slot_mapping.shape
             and positions.is_contiguous(), "positions must be contiguous int32 [n]")
    Hkv, D = k_pool.shape[2], k_pool.shape[3]
    _require(k_new.shape[1:] == (Hkv, D) and v_new.shape == k_new.shape, "rows must be [n, Hkv, D]")
    _rope_tables(rope_cos, rope_sin, D, k_pool.device)
    kp, vp = _rows(k_pool, "k_pool", True), _rows(v_pool, "v_pool", True)
    kn, vn = _rows(k_new, "k_new", False), _rows(v_new, "v_new", False)
    _require(kp.stride() == vp.stride() and kn.stride() == vn.stride(), "k and v must share strides")
    n = slot_mapping.shape[0]
    _require(kn.shape[0] == n, "one slot per new row")
    st = lib().pkv_kv_store_rope(kp.data_ptr(), vp.data_ptr(), kp.shape[0], kp.stride(0), kn.data_ptr(),
                                 vn.data_ptr(), kn.stride(0), slot_mapping.data_ptr(), n, Hkv, D,
                                 positions.data_ptr(), rope_cos.data_ptr(), rope_sin.data_ptr(),
                                 rope_cos.shape[0], _stream(kp))
    check(st, "pkv_kv_store_rope")


class PrefillPlan(NamedTuple):
    """The packed-query work map of a prefill batch (``pkv_prefill_plan``),
    on the device: ``qo_indptr`` int32 ``[B+1]``, ``tile_to_batch`` and
    ``tile_to_index`` int32 ``[num_tiles]``."""
    qo_indptr: torch.Tensor
    tile_to_batch: torch.Tensor
    tile_to_index: torch.Tensor
    num_tiles: int
    total_q: int


def prefill_plan(q_lens, device) -> PrefillPlan:
    """Build the work map for query lengths ``q_lens`` (host sequence of ints)
    with the library's host planner and copy it to ``device``."""
    ql = np.ascontiguousarray(np.asarray(q_lens, dtype=np.int32))
    B = ql.shape[0]
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    qo = np.zeros(B + 1, np.int32)
    n = lib().pkv_prefill_plan(ptr(ql), B, ptr(qo), None, None, 0)
    check(min(n, 0), "pkv_prefill_plan")
    tb, ti = np.zeros(max(n, 1), np.int32), np.zeros(max(n, 1), np.int32)
    n = lib().pkv_prefill_plan(ptr(ql), B, ptr(qo), ptr(tb), ptr(ti), tb.shape[0])
    check(min(n, 0), "pkv_prefill_plan")
    dev = lambda a: torch.from_numpy(a).to(device)
    return PrefillPlan(dev(qo), dev(tb[:max(n, 1)]), dev(ti[:max(n, 1)]), int(n), int(qo[-1]))


def paged_prefill_attn(q, k_pool, v_pool, page_table, kv_lens, plan: PrefillPlan, causal: bool = True,
                       scale: float | None = None, out=None, want_lse: bool = False):
    """Attention of packed queries ``q`` ``[total_q, Hq, D]`` bf16 over the paged
    pool; request b's rows are its last ``q_len`` positions of ``kv_lens[b]``.
    Returns ``out`` ``[total_q, Hq, D]`` bf16 (and lse fp32 ``[total_q, Hq]``)."""
    _on_gpu(q, k_pool, v_pool, page_table, kv_lens, plan.qo_indptr)
    _require(q.dtype == torch.bfloat16 and k_pool.dtype == torch.bfloat16 and v_pool.dtype == torch.bfloat16,
             "q and the pools must be bfloat16")
    _require(q.dim() == 3 and q.is_contiguous() and q.shape[0] == plan.total_q,
             "q must be contiguous [total_q, Hq, D] matching the plan")
    _require(k_pool.dim() == 4 and k_pool.is_contiguous() and v_pool.is_contiguous()
             and v_pool.shape == k_pool.shape, "pools must be contiguous [num_pages,P,Hkv,D]")
    _require(page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.is_contiguous(),
             "page_table must be contiguous int32 [B,max_pages]")
    B = page_table.shape[0]
    _require(kv_lens.dtype == torch.int32 and kv_lens.shape == (B,) and kv_lens.is_contiguous(),
             "kv_lens must be contiguous int32 [B]")
    _require(plan.qo_indptr.shape == (B + 1,), "plan built for another batch size")
    total_q, Hq, D = q.shape
    num_pages, P, Hkv, D2 = k_pool.shape
    _require(D2 == D, "head sizes differ")
    if out is None:
        out = torch.empty((total_q, Hq, D), dtype=torch.bfloat16, device=q.device)
    _require(out.shape == q.shape and out.dtype == torch.bfloat16 and out.is_contiguous(),
             "out must be contiguous bf16 like q")
    lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device) if want_lse else None
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    st = lib().pkv_paged_prefill_attn(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                      page_table.data_ptr(), kv_lens.data_ptr(), plan.qo_indptr.data_ptr(),
                                      plan.tile_to_batch.data_ptr(), plan.tile_to_index.data_ptr(),
                                      plan.num_tiles, total_q, B, Hq, Hkv, D, P, num_pages,
                                      page_table.shape[1], int(bool(causal)), scale, out.data_ptr(),
                                      lse.data_ptr() if lse is not None else None, _stream(q))
    check(st, "pkv_paged_prefill_attn")
    return (out, lse) if want_lse else out


def workspace(B: int, Hq: int, D: int, splits: int, device) -> tuple[torch.Tensor, torch.Tensor]:
    """Partial buffers for :func:`paged_decode_attn`: o ``[B,Hq,S,D]`` fp32, lse ``[B,Hq,S]`` fp32."""
    return (torch.empty((B, Hq, splits, D), dtype=torch.float32, device=device),
            torch.empty((B, Hq, splits), dtype=torch.float32, device=device))


def paged_decode_attn(q, k_pool, v_pool, page_table, seq_lens, max_seq_len: int,
                      splits: int | None = None, scale: float | None = None,
                      o_partial=None, lse_partial=None, total_tokens: int = -1,
                      q_positions=None, rope_cos=None, rope_sin=None, kernel: str = "mfma"):
    """Split-KV attention over the paged pool; returns (o_partial, lse_partial).

    q ``[B,Hq,D]`` bf16; pools ``[num_pages,P,Hkv,D]`` bf16; page_table int32
    ``[B,max_pages]``; seq_lens int32 ``[B]``; ``max_seq_len`` is a host bound
    on ``seq_lens`` (no device read); ``total_tokens`` (sum of ``seq_lens``, if
    the caller knows it) only steers the split heuristic when ``splits`` is None.
    With ``q_positions`` (int32 ``[B]``) and fp32 ``rope_cos``/``rope_sin``
    ``[rows, D/2]``, q is rotated by the rotary embedding in the kernel's
    prologue (``pkv_paged_decode_attn_rope``).  ``kernel="valu"`` calls the
    all-VALU kernel (``pkv_paged_decode_attn_valu``, no rotary prologue)."""
    _require(kernel in ("mfma", "valu"), "kernel must be 'mfma' or 'valu'")
    _require(kernel == "mfma" or q_positions is None, "the VALU kernel has no rotary prologue")
    _on_gpu(q, k_pool, v_pool, page_table, seq_lens)
    _require(q.dtype == torch.bfloat16 and k_pool.dtype == torch.bfloat16 and v_pool.dtype == torch.bfloat16,
             "q and the pools must be bfloat16")
    _require(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [B,Hq,D]")
    _require(k_pool.dim() == 4 and k_pool.is_contiguous() and v_pool.is_contiguous()
             and v_pool.shape == k_pool.shape, "pools must be contiguous [num_pages,P,Hkv,D]")
    _require(page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.is_contiguous(),
             "page_table must be contiguous int32 [B,max_pages]")
    _require(seq_lens.dtype == torch.int32 and seq_lens.is_contiguous(), "seq_lens must be int32")
    B, Hq, D = q.shape
    num_pages, P, Hkv, D2 = k_pool.shape
    _require(D2 == D and page_table.shape[0] == B and seq_lens.shape == (B,), "inconsistent shapes")
    S = num_splits(B, Hq, Hkv, max_seq_len, P, total_tokens) if splits is None else splits
    if o_partial is None or lse_partial is None:
        o_partial, lse_partial = workspace(B, Hq, D, S, q.device)
    _require(o_partial.shape == (B, Hq, S, D) and o_partial.dtype == torch.float32 and o_partial.is_contiguous(),
             "o_partial must be contiguous fp32 [B,Hq,S,D]")
    _require(lse_partial.shape == (B, Hq, S) and lse_partial.dtype == torch.float32 and lse_partial.is_contiguous(),
             "lse_partial must be contiguous fp32 [B,Hq,S]")
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    args = (q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), page_table.data_ptr(),
            seq_lens.data_ptr(), B, Hq, Hkv, D, P, num_pages, page_table.shape[1], max_seq_len, S,
            scale, o_partial.data_ptr(), lse_partial.data_ptr())
    if kernel == "valu":
        st = lib().pkv_paged_decode_attn_valu(*args, _stream(q))
        check(st, "pkv_paged_decode_attn_valu")
    elif q_positions is None:
        st = lib().pkv_paged_decode_attn(*args, _stream(q))
        check(st, "pkv_paged_decode_attn")
    else:
        _on_gpu(q, q_positions)
        _require(q_positions.dtype == torch.int32 and q_positions.shape == (B,)
                 and q_positions.is_contiguous(), "q_positions must be contiguous int32 [B]")
        _require(rope_cos is not None and rope_sin is not None, "q_positions needs rope_cos and rope_sin")
        _rope_tables(rope_cos, rope_sin, D, q.device)
        st = lib().pkv_paged_decode_attn_rope(*args, q_positions.data_ptr(), rope_cos.data_ptr(),
                                              rope_sin.data_ptr(), rope_cos.shape[0], _stream(q))
        check(st, "pkv_paged_decode_attn_rope")
    return o_partial, lse_partial


def _merged_args(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, splits, scale, out, lse_out,
                 want_lse, o_partial, lse_partial, total_tokens, partials: bool = True):
    """Checks shared by the calls that end in the merged bf16 output; returns
    the marshalled attention arguments, out and lse_out."""
    _on_gpu(q, k_pool, v_pool, page_table, seq_lens)
    _require(q.dtype == torch.bfloat16 and k_pool.dtype == torch.bfloat16 and v_pool.dtype == torch.bfloat16,
             "q and the pools must be bfloat16")
    _require(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [B,Hq,D]")
    _require(k_pool.dim() == 4 and k_pool.is_contiguous() and v_pool.is_contiguous()
             and v_pool.shape == k_pool.shape, "pools must be contiguous [num_pages,P,Hkv,D]")
    _require(page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.is_contiguous(),
             "page_table must be contiguous int32 [B,max_pages]")
    _require(seq_lens.dtype == torch.int32 and seq_lens.is_contiguous(), "seq_lens must be int32")
    B, Hq, D = q.shape
    num_pages, P, Hkv, D2 = k_pool.shape
    _require(D2 == D and page_table.shape[0] == B and seq_lens.shape == (B,), "inconsistent shapes")
    S = num_splits(B, Hq, Hkv, max_seq_len, P, total_tokens) if splits is None else splits
    if partials and S > 1 and (o_partial is None or lse_partial is None):
        o_partial, lse_partial = workspace(B, Hq, D, S, q.device)
    if o_partial is not None:
        _require(o_partial.shape == (B, Hq, S, D) and o_partial.dtype == torch.float32
                 and o_partial.is_contiguous(), "o_partial must be contiguous fp32 [B,Hq,S,D]")
    if lse_partial is not None:
        _require(lse_partial.shape == (B, Hq, S) and lse_partial.dtype == torch.float32
                 and lse_partial.is_contiguous(), "lse_partial must be contiguous fp32 [B,Hq,S]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    _require(out.shape == (B, Hq, D) and out.dtype == torch.bfloat16 and out.is_contiguous(),
             "out must be contiguous bf16 [B,Hq,D]")
    if want_lse and lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse_out is not None:
        _require(lse_out.shape == (B, Hq) and lse_out.dtype == torch.float32 and lse_out.is_contiguous(),
                 "lse_out must be contiguous fp32 [B,Hq]")
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ptr = lambda t: t.data_ptr() if t is not None else None
    tail = (page_table.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, P, num_pages, page_table.shape[1],
            max_seq_len, S, scale, ptr(o_partial), ptr(lse_partial), out.data_ptr(), ptr(lse_out))
    return tail, out, lse_out


def paged_decode_attn_merged(q, k_pool, v_pool, page_table, seq_lens, max_seq_len: int,
                             splits: int | None = None, scale: float | None = None, out=None,
                             lse_out=None, want_lse: bool = False, o_partial=None, lse_partial=None,
                             total_tokens: int = -1):
    """Attention and merge in one call (``pkv_paged_decode_attn_merged``):
    bf16 ``[B,Hq,D]`` (and fp32 lse ``[B,Hq]``), the same bits as
    :func:`paged_decode_attn` followed by :func:`decode_merge`.  With one split
    a single kernel writes the output and no partials are used; with more, the
    partials (allocated here unless given) feed a second launch."""
    tail, out, lse_out = _merged_args(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, splits, scale,
                                      out, lse_out, want_lse, o_partial, lse_partial, total_tokens)
    st = lib().pkv_paged_decode_attn_merged(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), *tail,
                                            _stream(q))
    check(st, "pkv_paged_decode_attn_merged")
    return (out, lse_out) if (want_lse or lse_out is not None) else out


def paged_decode_attn_merged_static(q, k_pool, v_pool, page_table, seq_lens, max_seq_len: int,
                                    splits: int | None = None, scale: float | None = None, out=None,
                                    lse_out=None, want_lse: bool = False, total_tokens: int = -1):
    """:func:`paged_decode_attn_merged` with the split partials in the
    library's static device scratch (``pkv_paged_decode_attn_merged_static``):
    the C call allocates nothing.  Pass ``out`` (and ``lse_out``) to allocate
    nothing here either.  Calls on one GPU share the scratch: do not let them
    overlap on different streams."""
    tail, out, lse_out = _merged_args(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, splits, scale,
                                      out, lse_out, want_lse, None, None, total_tokens, partials=False)
    st = lib().pkv_paged_decode_attn_merged_static(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                                   *tail[:12], *tail[14:], _stream(q))
    check(st, "pkv_paged_decode_attn_merged_static")
    return (out, lse_out) if (want_lse or lse_out is not None) else out


def decode_step_fused(q, k_new, v_new, k_pool, v_pool, page_table, seq_lens, slot_mapping,
                      max_seq_len: int, splits: int | None = None, scale: float | None = None, out=None,
                      lse_out=None, want_lse: bool = False, o_partial=None, lse_partial=None,
                      total_tokens: int = -1):
    """One decode step in one call (``pkv_decode_step``): the store of one new
    row per sequence fused into the attention kernel, then the merge (no
    second launch with one split).  Same pools, output and lse, bit for bit, as
    :func:`kv_store` then :func:`paged_decode_attn_merged`, provided
    ``slot_mapping[b]`` is the slot of position ``seq_lens[b] - 1``.
    ``k_new``/``v_new``: ``[B, Hkv, D]`` or ``[B, Hkv*D]`` bf16, rows contiguous."""
    _on_gpu(k_new, v_new, slot_mapping)
    kn, vn = _rows(k_new, "k_new", False), _rows(v_new, "v_new", False)
    _require(kn.shape == vn.shape and kn.stride() == vn.stride(), "k_new and v_new must match")
    _require(kn.dtype == torch.bfloat16 and vn.dtype == torch.bfloat16, "new rows must be bfloat16")
    _require(slot_mapping.dtype == torch.int32 and slot_mapping.is_contiguous()
             and slot_mapping.shape == (q.shape[0],), "slot_mapping must be contiguous int32 [B]")
    _require(kn.shape[0] == q.shape[0] and kn.shape[1] == k_pool.shape[2] * k_pool.shape[3],
             "one new row of Hkv*D values per sequence")
    tail, out, lse_out = _merged_args(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, splits, scale,
                                      out, lse_out, want_lse, o_partial, lse_partial, total_tokens)
    st = lib().pkv_decode_step(q.data_ptr(), kn.data_ptr(), vn.data_ptr(), kn.stride(0),
                               slot_mapping.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), *tail, _stream(q))
    check(st, "pkv_decode_step")
    return (out, lse_out) if (want_lse or lse_out is not None) else out


def decode_merge(o_partial, lse_partial, out=None, lse_out=None, want_lse: bool = False):
    """Log-sum-exp merge of the split partials -> bf16 ``[B,Hq,D]`` (and fp32 lse ``[B,Hq]``)."""
    _on_gpu(o_partial, lse_partial)
    _require(o_partial.dtype == torch.float32 and lse_partial.dtype == torch.float32
             and o_partial.is_contiguous() and lse_partial.is_contiguous(), "partials must be contiguous fp32")
    B, Hq, S, D = o_partial.shape
    _require(lse_partial.shape == (B, Hq, S), "lse_partial must be [B,Hq,S]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=o_partial.device)
    _require(out.shape == (B, Hq, D) and out.dtype == torch.bfloat16 and out.is_contiguous(),
             "out must be contiguous bf16 [B,Hq,D]")
    if want_lse and lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=o_partial.device)
    if lse_out is not None:
        _require(lse_out.shape == (B, Hq) and lse_out.dtype == torch.float32 and lse_out.is_contiguous(),
                 "lse_out must be contiguous fp32 [B,Hq]")
    st = lib().pkv_decode_merge(o_partial.data_ptr(), lse_partial.data_ptr(), B, Hq, D, S,
                                out.data_ptr(), lse_out.data_ptr() if lse_out is not None else None,
                                _stream(o_partial))
    check(st, "pkv_decode_merge")
    return (out, lse_out) if (want_lse or lse_out is not None) else out


def decode_step(q, k_new, v_new, k_pool, v_pool, page_table, seq_lens, slot_mapping,
                max_seq_len: int, splits: int | None = None, out=None, ws=None,
                want_lse: bool = False, total_tokens: int = -1):
    """One decode step: store the new rows, then split-KV attention and merge
    (one launch when there is one split)."""
    kv_store(k_pool, v_pool, k_new, v_new, slot_mapping)
    return paged_decode_attn_merged(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, splits,
                                    out=out, want_lse=want_lse,
                                    o_partial=None if ws is None else ws[0],
                                    lse_partial=None if ws is None else ws[1],
                                    total_tokens=total_tokens)
