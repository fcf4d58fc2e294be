"""Seeded synthetic decode-step workloads (shared by the tests and ``bench.py``).

This module only draws and lays out inputs; it holds none of the method's
arithmetic.  Neither the CPU oracle nor the HIP binding imports the other:
both receive the byte-identical arrays this module returns.

The five workloads follow the decode configurations the pages' kernels are
sized for (grouped-query decode over a paged pool, page_size 16 or token
granular), with every value synthetic:

* q, K, V ~ N(0, 1) drawn as float32 (q scaled by ``q_std``) and rounded to
  bf16 with round-to-nearest-even (torch's CPU conversion);
* the page table is a seeded permutation of the pool's pages handed to the
  sequences in order (sequence 0 first);
* pool pages no sequence owns, and slots past a sequence's last token, hold a
  NaN canary, so a stray read shows up as NaN in the output;
* the step's new token sits at position ``L_b - 1`` (the sequence length
  counts it), its pool slot holds a NaN canary until ``kv_store`` writes it.

Random streams, for seed = 20260000 + config_id:
``numpy.random.Generator(PCG64(seed))`` draws the lengths (ragged config only)
and then the page permutation; q, K and V come from the three children of
``numpy.random.SeedSequence(seed).spawn(3)``, each cut into chunks of 2^22
values with one PCG64 stream per chunk (so the result does not depend on the
number of threads that fill it).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
SEED_BASE = 20260000


@dataclass(frozen=True)
class Config:
    seed_id: int         # the inputs are drawn from seed SEED_BASE + seed_id
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int               # page_size (tokens per page)
    num_pages: int
    seq_len: int | None  # every sequence has this length, or None for ragged
    seq_lens: tuple | None = None   # explicit lengths
    ragged_max: int | None = None   # lengths ~ U{1..ragged_max}
    q_std: float = 1.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.max_len_bound // self.P)

    @property
    def max_len_bound(self) -> int:
        if self.seq_lens is not None:
            return max(self.seq_lens)
        if self.seq_len is not None:
            return self.seq_len
        return self.ragged_max

    @property
    def row_elems(self) -> int:
        return self.Hkv * self.D

    def describe(self) -> str:
        lens = (list(self.seq_lens) if self.seq_lens is not None else
                f"{self.seq_len}" if self.seq_len is not None else f"U{{1..{self.ragged_max}}}")
        return (f"B={self.B} Hq={self.Hq} Hkv={self.Hkv} D={self.D} page_size={self.P} "
                f"pool={self.num_pages} pages seq_len={lens} q_std={self.q_std}")


WORKLOADS = {
    "tiny_gqa": Config(1, "tiny_gqa", B=2, Hq=4, Hkv=1, D=64, P=16, num_pages=32,
                       seq_len=None, seq_lens=(37, 100)),
    "llama3_8b_decode": Config(2, "llama3_8b_decode", B=32, Hq=32, Hkv=8, D=128, P=16,
                               num_pages=9000, seq_len=4096),
    "ragged_batch": Config(3, "ragged_batch", B=64, Hq=32, Hkv=8, D=128, P=16,
                           num_pages=32768, seq_len=None, ragged_max=8192),
    "long_context": Config(4, "long_context", B=4, Hq=64, Hkv=8, D=128, P=16,
                           num_pages=18432, seq_len=65536, q_std=1.5),
    "mha_page1": Config(5, "mha_page1", B=128, Hq=16, Hkv=16, D=64, P=1, num_pages=300000,
                        seq_len=2048),
}


def custom_config(seed_id=0, name="custom", **kw) -> Config:
    """A workload of any shape (parity edge cases)."""
    kw.setdefault("seq_len", None)
    return Config(seed_id, name, **kw)


@dataclass
class Inputs:
    cfg: Config
    seed: int
    q: np.ndarray             # uint16 [B, Hq, D]            (bf16 bits)
    k_pool: np.ndarray        # uint16 [num_pages, P, Hkv, D] before the store
    v_pool: np.ndarray
    page_table: np.ndarray    # int32 [B, max_pages_per_seq]
    seq_lens: np.ndarray      # int32 [B]
    slot_mapping: np.ndarray  # int32 [B]: slot of position L_b - 1
    k_new: np.ndarray         # uint16 [B, Hkv*D]
    v_new: np.ndarray
    extra: dict = field(default_factory=dict)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    def pools_after_store(self):
        """The pools with the new rows in place (what the generator drew)."""
        return self.extra["k_full"], self.extra["v_full"]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (torch CPU cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


_CHUNK = 1 << 22


def _normal_bf16(seed_seq, shape, std=1.0):
    """N(0, std^2) float32 rounded to bf16.  The array is cut into chunks of
    2^22 values; chunk i is drawn from PCG64(seed_seq.spawn(...)[i]), so the
    result does not depend on how many threads fill it."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    nchunks = -(-n // _CHUNK)
    children = seed_seq.spawn(nchunks)

    def fill(i):
        s, e = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = np.random.Generator(np.random.PCG64(children[i])).standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = to_bf16_bits(x)

    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def draw_seq_lens(cfg: Config, rng) -> np.ndarray:
    if cfg.seq_lens is not None:
        return np.asarray(cfg.seq_lens, np.int32)
    if cfg.seq_len is not None:
        return np.full(cfg.B, cfg.seq_len, np.int32)
    return rng.integers(1, cfg.ragged_max + 1, cfg.B).astype(np.int32)


def make_inputs(cfg: Config, seed: int | None = None, seq_lens=None) -> Inputs:
    """Draw one decode step's inputs for ``cfg`` (see the module docstring)."""
    seed = SEED_BASE + cfg.seed_id if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    q_ss, k_ss, v_ss = np.random.SeedSequence(seed).spawn(3)
    lens = draw_seq_lens(cfg, rng) if seq_lens is None else np.asarray(seq_lens, np.int32)
    B, P = cfg.B, cfg.P
    assert lens.shape == (B,)
    max_pages = max(1, -(-int(lens.max(initial=0)) // P), cfg.max_pages_per_seq)
    n_pages = -(-lens.astype(np.int64) // P)
    total = int(n_pages.sum())
    if total >= cfg.num_pages:
        raise ValueError(f"pool of {cfg.num_pages} pages cannot hold {total} pages plus a canary page")

    perm = rng.permutation(cfg.num_pages).astype(np.int32)
    canary_page = perm[-1]  # never owned: page-table padding points here
    page_table = np.full((B, max_pages), canary_page, np.int32)
    starts = np.concatenate([[0], np.cumsum(n_pages)])
    for b in range(B):
        page_table[b, :n_pages[b]] = perm[starts[b]:starts[b + 1]]
    used = perm[:total]

    q = _normal_bf16(q_ss, (B, cfg.Hq, cfg.D), cfg.q_std)
    shape = (cfg.num_pages, P, cfg.Hkv, cfg.D)
    k_full = np.full(shape, BF16_NAN, np.uint16)
    v_full = np.full(shape, BF16_NAN, np.uint16)
    k_full[used] = _normal_bf16(k_ss, (total, P, cfg.Hkv, cfg.D))
    v_full[used] = _normal_bf16(v_ss, (total, P, cfg.Hkv, cfg.D))
    # slots past each sequence's last token are canaries too
    for b in range(B):
        L = int(lens[b])
        if L % P:
            last = page_table[b, n_pages[b] - 1]
            k_full[last, L % P:] = BF16_NAN
            v_full[last, L % P:] = BF16_NAN

    # the new token of this step: position L_b - 1 (empty sequences have none)
    has_new = lens > 0
    pos = np.maximum(lens.astype(np.int64) - 1, 0)
    slot_mapping = (page_table[np.arange(B), pos // P].astype(np.int64) * P + pos % P).astype(np.int32)
    slot_mapping = slot_mapping[has_new]
    flat_k = k_full.reshape(cfg.num_pages * P, cfg.row_elems)
    flat_v = v_full.reshape(cfg.num_pages * P, cfg.row_elems)
    k_new = flat_k[slot_mapping].copy()
    v_new = flat_v[slot_mapping].copy()
    k_pool = k_full.copy()
    v_pool = v_full.copy()
    k_pool.reshape(-1, cfg.row_elems)[slot_mapping] = BF16_NAN
    v_pool.reshape(-1, cfg.row_elems)[slot_mapping] = BF16_NAN
    return Inputs(cfg, seed, q, k_pool, v_pool, page_table, lens, slot_mapping, k_new, v_new,
                  extra={"k_full": k_full, "v_full": v_full, "canary_page": int(canary_page)})


def contiguous_layout(inp: Inputs):
    """The same sequences re-laid contiguously: sequence b's pages in logical
    order, one after another, with an identity-like page table.  Returns
    (k_pool, v_pool, page_table) after the store."""
    k_full, v_full = inp.pools_after_store()
    B, P = inp.cfg.B, inp.cfg.P
    n_pages = -(-inp.seq_lens.astype(np.int64) // P)
    order = np.concatenate([inp.page_table[b, :n_pages[b]] for b in range(B)] + [np.zeros(0, np.int32)])
    k_c = np.concatenate([k_full[order], np.full((1,) + k_full.shape[1:], BF16_NAN, np.uint16)])
    v_c = np.concatenate([v_full[order], np.full((1,) + v_full.shape[1:], BF16_NAN, np.uint16)])
    pt = np.full(inp.page_table.shape, len(order), np.int32)
    starts = np.concatenate([[0], np.cumsum(n_pages)])
    for b in range(B):
        pt[b, :n_pages[b]] = np.arange(starts[b], starts[b + 1], dtype=np.int32)
    return k_c, v_c, pt


def bulk_fill_rows(inp: Inputs, seed: int | None = None):
    """Rows for a prefill-style bulk store of every position of every sequence
    (positions in order), the workload on which kv_store bandwidth is measured.
    Returns (k_rows uint16 [n, Hkv*D], v_rows, slots int32 [n])."""
    cfg = inp.cfg
    ss = np.random.SeedSequence((SEED_BASE + 1000 + cfg.seed_id) if seed is None else seed)
    k_ss, v_ss = ss.spawn(2)
    slots = []
    for b in range(cfg.B):
        t = np.arange(int(inp.seq_lens[b]), dtype=np.int64)
        slots.append(inp.page_table[b, t // cfg.P].astype(np.int64) * cfg.P + t % cfg.P)
    slots = np.concatenate(slots + [np.zeros(0, np.int64)]).astype(np.int32)
    n = slots.shape[0]
    k_rows = _normal_bf16(k_ss, (n, cfg.row_elems))
    v_rows = _normal_bf16(v_ss, (n, cfg.row_elems))
    return k_rows, v_rows, slots


def bulk_fill_runs(inp: Inputs):
    """The bulk fill of :func:`bulk_fill_rows` as runs of consecutive rows that
    land in consecutive slots (one run per page a sequence fills): int32
    arrays (first source row, first destination slot, rows) per run."""
    cfg = inp.cfg
    src, dst, rows = [], [], []
    r = 0
    for b in range(cfg.B):
        L = int(inp.seq_lens[b])
        for j in range(-(-L // cfg.P)):
            n = min(cfg.P, L - j * cfg.P)
            src.append(r)
            dst.append(int(inp.page_table[b, j]) * cfg.P)
            rows.append(n)
            r += n
    as32 = lambda a: np.asarray(a, np.int64).astype(np.int32)
    return as32(src), as32(dst), as32(rows)


@dataclass(frozen=True)
class PrefillConfig:
    """A paged prefill batch: request b has kv_lens[b] tokens in the pool, the
    last q_lens[b] of which are its new query rows (packed over the batch)."""
    seed_id: int
    name: str
    Hq: int
    Hkv: int
    D: int
    P: int
    num_pages: int
    q_lens: tuple
    kv_lens: tuple

    @property
    def B(self) -> int:
        return len(self.q_lens)

    def describe(self) -> str:
        return (f"B={self.B} Hq={self.Hq} Hkv={self.Hkv} D={self.D} page_size={self.P} "
                f"q_lens={list(self.q_lens)[:8]} kv_lens={list(self.kv_lens)[:8]}")


PREFILL = {
    # the page's ragged Q lengths [70, 10, 130], two of them continuing a cached context
    "ragged_chunks": PrefillConfig(101, "ragged_chunks", 8, 2, 64, 16, 64,
                                   (70, 10, 130), (70, 300, 200)),
    # Llama-3-8B-shaped chunked prefill: 1024 new tokens on top of 3072 cached, batch 4
    "llama3_8b_chunked": PrefillConfig(102, "llama3_8b_chunked", 32, 8, 128, 16, 1100,
                                       (1024,) * 4, (4096,) * 4),
    # fresh prompts, q = kv = 2048 (the size of the page's single-batch prefill figure), batch 2
    "llama3_8b_fresh": PrefillConfig(103, "llama3_8b_fresh", 32, 8, 128, 16, 300,
                                     (2048,) * 2, (2048,) * 2),
    # the same fresh prompts with one q head per kv head (32 + 32 heads)
    "mha_fresh": PrefillConfig(104, "mha_fresh", 32, 32, 128, 16, 300,
                               (2048,) * 2, (2048,) * 2),
}


def make_prefill_inputs(cfg: PrefillConfig, seed: int | None = None):
    """(q uint16 [total_q, Hq, D], k_pool, v_pool [num_pages, P, Hkv, D],
    page_table int32 [B, max_pages], kv_lens int32 [B], qo_indptr int32 [B+1]).
    The pools and page table are drawn as for a decode step over kv_lens (all
    positions stored, unowned pages NaN canaries); q ~ N(0, 1) rounded to bf16."""
    seed = SEED_BASE + cfg.seed_id if seed is None else seed
    dcfg = Config(cfg.seed_id, cfg.name, B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D, P=cfg.P,
                  num_pages=cfg.num_pages, seq_len=None, seq_lens=tuple(cfg.kv_lens))
    inp = make_inputs(dcfg, seed=seed)
    k_pool, v_pool = inp.pools_after_store()
    qo = np.concatenate([[0], np.cumsum(np.asarray(cfg.q_lens, np.int64))]).astype(np.int32)
    q = _normal_bf16(np.random.SeedSequence(seed + 7), (int(qo[-1]), cfg.Hq, cfg.D))
    return q, k_pool, v_pool, inp.page_table, np.asarray(cfg.kv_lens, np.int32), qo


def prefill_flops(q_lens, kv_lens, Hq: int, D: int, causal: bool = True) -> int:
    """Multiply-adds x 2 of QK^T and PV over the (query, position) pairs a
    query row sees: 4 * D flops per pair and q head."""
    pairs = 0
    for ql, kl in zip(q_lens, kv_lens):
        if causal:
            first = kl - ql + 1            # positions seen by the first query row
            pairs += ql * first + ql * (ql - 1) // 2
        else:
            pairs += ql * kl
    return 4 * D * Hq * pairs


@dataclass(frozen=True)
class IndexingConfig:
    """A vocabulary-parallel embedding lookup: the table is split into ``shards``
    equal slices of ``vocab / shards`` rows; one rank holds one slice."""
    name: str
    vocab: int
    hidden: int
    shards: int
    n: int            # token ids per call

    @property
    def length(self) -> int:
        return -(-self.vocab // self.shards)


INDEXING = {
    # Llama-3-8B-shaped table (128256 x 4096, bf16), 8-way vocabulary split
    "llama3_8b_embed_prefill": IndexingConfig("llama3_8b_embed_prefill", 128256, 4096, 8, 65536),
    "llama3_8b_embed_decode": IndexingConfig("llama3_8b_embed_decode", 128256, 4096, 8, 32),
}


def make_indexing_inputs(cfg: IndexingConfig, rank: int = 0, seed: int = SEED_BASE + 100):
    """(slice bf16 bits [length, hidden], ids int32 [n], start) for one rank:
    the slice holds N(0,1) rows, ids are uniform over the whole vocabulary, so
    about 1/shards of them fall into this rank's slice."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = rng.integers(0, cfg.vocab, cfg.n).astype(np.int32)
    table_ss = np.random.SeedSequence(seed + 1 + rank)
    start = rank * cfg.length
    length = min(cfg.length, cfg.vocab - start)
    return _normal_bf16(table_ss, (length, cfg.hidden)), ids, start


def indexing_bytes(ids, start: int, length: int, row_bytes: int) -> int:
    """Traffic of one lookup: read the ids and the in-slice rows, write every output row."""
    ids = np.asarray(ids, np.int64)
    valid = int(((ids >= start) & (ids < start + length)).sum())
    return 4 * ids.shape[0] + valid * row_bytes + ids.shape[0] * row_bytes


def rope_tables(rows: int, D: int, base: float = 500000.0):
    """fp32 cos/sin tables ``[rows, D/2]`` of the usual rotary frequencies
    ``theta_i = base^(-2i/D)`` (Llama-3 uses base 500000): entry (p, i) is the
    cosine / sine of ``p * theta_i``, evaluated in fp64 and rounded to fp32.
    These are inputs of the rotary step, like the weights of a model."""
    i = np.arange(D // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / D)
    ang = np.arange(rows, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def kv_bytes(seq_lens, Hkv: int, D: int, elem_bytes: int = 2) -> int:
    """K+V bytes one decode step must read: sum_b L_b * 2 * Hkv * D * elem_bytes."""
    return int(np.asarray(seq_lens, np.int64).sum()) * 2 * Hkv * D * elem_bytes


def attention_bytes(seq_lens, Hq, Hkv, D, P, num_splits, elem_bytes=2) -> dict:
    """Every term of the algorithmic traffic of attention + merge for one step."""
    lens = np.asarray(seq_lens, np.int64)
    B = lens.shape[0]
    terms = {
        "kv": kv_bytes(lens, Hkv, D, elem_bytes),
        "q": B * Hq * D * elem_bytes,
        "page_ids": int((-(-lens // P)).sum()) * 4 + B * 4,  # page ids + seq_lens
        "partials": 2 * B * Hq * num_splits * (D + 1) * 4,   # written once, read once
        "out": B * Hq * D * elem_bytes,
    }
    terms["total"] = sum(terms.values())
    return terms


def store_bytes(n_rows: int, row_bytes: int) -> int:
    """kv_store traffic: read k and v rows, write both pool rows, read the indices."""
    return 4 * n_rows * row_bytes + 4 * n_rows


def roofline_us(nbytes: int, peak_bytes_per_s: float) -> float:
    return nbytes / peak_bytes_per_s * 1e6


def sample_rows(cfg: Config, k: int, seed: int = 7) -> np.ndarray:
    """k distinct (b, h) pairs, always including the first and last row."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = cfg.B * cfg.Hq
    k = min(k, n)
    idx = set(rng.choice(n, size=k, replace=False).tolist()) | {0, n - 1}
    idx = np.array(sorted(idx), np.int64)
    return np.stack([idx // cfg.Hq, idx % cfg.Hq], axis=1)


__all__ = ["Config", "WORKLOADS", "Inputs", "make_inputs", "custom_config", "contiguous_layout",
           "bulk_fill_rows", "bulk_fill_runs", "kv_bytes", "attention_bytes", "store_bytes", "roofline_us",
           "to_bf16_bits", "bf16_bits_to_f32", "sample_rows", "IndexingConfig", "INDEXING",
           "make_indexing_inputs", "indexing_bytes", "rope_tables", "PrefillConfig", "PREFILL",
           "make_prefill_inputs", "prefill_flops"]
