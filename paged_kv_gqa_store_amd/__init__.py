"""Paged-KV grouped-query attention decode step for AMD MI355X (gfx950).

One decode step is three hand-written HIP kernels behind a C ABI
(``include/pkv.h``, ``libpkv.so``):

* ``kv_store``           scatter the step's new K/V rows into the page pool;
* ``paged_decode_attn``  split-KV attention over pages found through a page table;
* ``decode_merge``       log-sum-exp merge of the split partials;

(``paged_decode_attn_merged`` runs the last two as one call: a single kernel
when there is one split; ``paged_decode_attn_merged_static`` does the same
with its partials in a static device array, allocating nothing;
``decode_step_fused`` runs all three as one call, the store fused into the
attention kernel),

plus ``paged_prefill_attn`` (packed multi-token queries over the same pool,
with the ``prefill_plan`` work map), ``kv_store_rope`` (the store with K rotated by a rotary embedding on the
way, and ``paged_decode_attn(..., q_positions=...)`` rotating q in the
attention prologue) and ``indexing``, a row gather from one rank's slice of a
vocabulary-parallel embedding table, on the same row-move kernel design as
``kv_store``.

The binding in :mod:`paged_kv_gqa_store_amd.ops` only marshals arguments;
PyTorch provides device memory and streams.  Loading the library is lazy, and
every op raises ``RuntimeError`` if ``libpkv.so`` is missing: there is no
fallback implementation.
"""
from .ops import (  # noqa: F401
    PrefillPlan, decode_merge, decode_step, decode_step_fused, indexing, kv_store, kv_store_rope, num_splits,
    paged_decode_attn, paged_decode_attn_merged, paged_decode_attn_merged_static, paged_prefill_attn,
    prefill_plan, split_chunk, workspace,
)
