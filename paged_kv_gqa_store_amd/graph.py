"""A multi-layer decode step captured into one HIP graph.

A one-token step moves too few bytes per kernel to amortise a launch (the
mini-sglang handbook, "Custom CUDA kernels", section "Exercises", puts a
per-layer KV write at a fraction of a microsecond and sends it into a graph).
:class:`StepGraph` records ``n_layers`` x (``kv_store`` -> ``paged_decode_attn``
-> ``decode_merge``, the last two as one call that is a single kernel when
there is one split) once and replays the whole sequence with one launch.

The library's entry points are capture-safe by construction: they launch on
the current stream, never allocate, free, synchronise or memset, and take the
sequence-length bound ``max_seq_len`` from the host.  Capture and replay use
PyTorch's graph API (HIP graphs on ROCm); every kernel in the graph is the
library's own.
"""
from __future__ import annotations

import torch

from . import ops


class StepGraph:
    """``n_layers`` decode steps, one per ``(k_pool, v_pool)`` in ``pools``.

    ``q``, ``k_new`` and ``v_new`` are one tensor shared by every layer or a
    list with one tensor per layer; ``page_table``, ``seq_lens`` and
    ``slot_mapping`` are shared (the layers of one model see the same
    sequences).  All of them are static: refill them in place between
    replays.  ``max_seq_len`` and the split count are fixed at capture, so a
    server keeps one graph per length bucket.  ``outputs[l]`` is layer l's
    ``[B, Hq, D]`` bf16 result, overwritten by every replay.  With ``fused``
    (the default) each layer is one ``pkv_decode_step`` call, the store fused
    into the attention kernel; that needs one new row per sequence and
    ``slot_mapping[b]`` the slot of position ``seq_lens[b] - 1``.  Construction
    runs the layers once eagerly before capturing them (the same work a
    replay does: the new rows are stored, the outputs computed).
    """

    def __init__(self, pools, q, k_new, v_new, page_table, seq_lens, slot_mapping,
                 max_seq_len: int, splits: int | None = None, total_tokens: int = -1,
                 fused: bool = True):
        n = len(pools)
        per_layer = lambda x: list(x) if isinstance(x, (list, tuple)) else [x] * n
        self.pools = list(pools)
        self.q, self.k_new, self.v_new = per_layer(q), per_layer(k_new), per_layer(v_new)
        if not (len(self.q) == len(self.k_new) == len(self.v_new) == n) or n == 0:
            raise RuntimeError("one q / k_new / v_new per layer (or one shared)")
        self.page_table, self.seq_lens, self.slot_mapping = page_table, seq_lens, slot_mapping
        self.fused = fused
        B, Hq, D = self.q[0].shape
        P, Hkv = self.pools[0][0].shape[1], self.pools[0][0].shape[2]
        self.max_seq_len = max_seq_len
        self.splits = (ops.num_splits(B, Hq, Hkv, max_seq_len, P, total_tokens)
                       if splits is None else splits)
        # The layers run one after another inside the graph, so they share one
        # partials workspace (not needed with one split: the attention then
        # writes the merged output itself).
        self.workspace = (ops.workspace(B, Hq, D, self.splits, self.q[0].device)
                          if self.splits > 1 else (None, None))
        self.outputs = [torch.empty((B, Hq, D), dtype=torch.bfloat16, device=self.q[0].device)
                        for _ in range(n)]
        self.graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=self.q[0].device)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            # One eager pass first (it loads the kernels' code objects, which must
            # not happen under capture); it performs exactly what a replay does.
            self._record()
            side.synchronize()
            with torch.cuda.graph(self.graph, stream=side):
                self._record()
        torch.cuda.current_stream().wait_stream(side)

    def _record(self):
        o_p, l_p = self.workspace
        for layer, (k_pool, v_pool) in enumerate(self.pools):
            if self.fused:
                ops.decode_step_fused(self.q[layer], self.k_new[layer], self.v_new[layer], k_pool, v_pool,
                                      self.page_table, self.seq_lens, self.slot_mapping, self.max_seq_len,
                                      self.splits, out=self.outputs[layer], o_partial=o_p, lse_partial=l_p)
                continue
            ops.kv_store(k_pool, v_pool, self.k_new[layer], self.v_new[layer], self.slot_mapping)
            ops.paged_decode_attn_merged(self.q[layer], k_pool, v_pool, self.page_table, self.seq_lens,
                                         self.max_seq_len, self.splits, out=self.outputs[layer],
                                         o_partial=o_p, lse_partial=l_p)

    def replay(self) -> list:
        """Run every captured layer on the current stream; returns ``outputs``."""
        self.graph.replay()
        return self.outputs
