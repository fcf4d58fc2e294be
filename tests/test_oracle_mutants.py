"""Plant plausible slips in a copy of the oracle (on the CPU) and check that
the pins in ``test_oracle_pins.py`` catch every one of them."""
import subprocess

import pytest

from oracle import oracle

from . import test_oracle_pins as pins

SRC = (oracle._SRC).read_text()

# (name, original text, mutated text)
MUTANTS = [
    ("scale dropped", "const double scale = 1.0 / sqrt((double)D);", "const double scale = 1.0;"),
    ("scale 1/D", "const double scale = 1.0 / sqrt((double)D);", "const double scale = 1.0 / (double)D;"),
    ("q head -> wrong kv head", "G = p->Hq / p->Hkv, g = h / G;", "G = p->Hq / p->Hkv, g = h % p->Hkv;"),
    ("slot within page off by one", "return page * page_size + t % page_size;",
     "return page * page_size + (t + 1) % page_size;"),
    ("page index ignores position", "page_table[b * max_pages + t / page_size]", "page_table[b * max_pages]"),
    ("score sign", "double s = scale * dot;", "double s = -scale * dot;"),
    ("V read from K pool", "const uint16_t *v = p->v_pool", "const uint16_t *v = p->k_pool"),
    ("weights not normalised", "double wt = exp(scores[t - t0] - m) / denom;",
     "double wt = exp(scores[t - t0] - m);"),
    ("lse misses the max", "*lse = m + log(denom);", "*lse = log(denom);"),
    ("merge weight inverted", "double ws = exp(lr[s] - M);", "double ws = exp(M - lr[s]);"),
    ("merge not normalised", "o[d] /= den;", "o[d] /= 1.0;"),
    ("merge lse misses the max", "lse[r] = M + log(den);", "lse[r] = log(den);"),
    ("store copies the wrong row", "k_new + i * in_row_stride", "k_new + (n - 1 - i) * in_row_stride"),
    ("store skips V", "memcpy(v_pool + slot * pool_row_stride", "if (0) memcpy(v_pool + slot * pool_row_stride"),
    ("split end off by one", "if (t1 > seq_lens[b]) t1 = seq_lens[b];",
     "if (t1 > seq_lens[b]) t1 = seq_lens[b] - 1;"),
    ("bf16 widened wrongly", "(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    ("chunk not page aligned", "return (per + page_size - 1) / page_size * page_size;", "return per;"),
    ("rope real part sign", "orow[2 * i] = float_to_bf16_rne(a - b);", "orow[2 * i] = float_to_bf16_rne(a + b);"),
    ("rope imaginary part sign", "orow[2 * i + 1] = float_to_bf16_rne(e + f);",
     "orow[2 * i + 1] = float_to_bf16_rne(f - e);"),
    ("rope position off by one", "const float c = cos_t[pos * half + i], sn = sin_t[pos * half + i];",
     "const int64_t pp = pos > 0 ? pos - 1 : 0; const float c = cos_t[pp * half + i], sn = sin_t[pp * half + i];"),
    ("rope cos and sin swapped", "const float c = cos_t[pos * half + i], sn = sin_t[pos * half + i];",
     "const float sn = cos_t[pos * half + i], c = sin_t[pos * half + i];"),
    ("rope pairs halves instead of neighbours", "const float x1 = (float)bf16_to_double(xr[2 * i + 1]);",
     "const float x1 = (float)bf16_to_double(xr[(2 * i + D / 2) % D]);"),
    ("prefill causal bound off by one", "const int64_t t1 = causal ? pos + 1 : L;",
     "const int64_t t1 = causal ? pos : L;"),
    ("prefill query rows aligned to the start", "const int64_t pos = L - ql + (i - qo_indptr[b]);",
     "const int64_t pos = i - qo_indptr[b];"),
    ("prefill wrong kv head", "const int64_t i = qh / Hq, h = qh % Hq, g = h / G;",
     "const int64_t i = qh / Hq, h = qh % Hq, g = h % Hkv;"),
    ("prefill lse misses the max", "lse[n] = t1 > 0 ? m + log(den) : -INFINITY;",
     "lse[n] = t1 > 0 ? log(den) : -INFINITY;"),
    ("indexing ignores the slice start", "const int64_t local = (int64_t)ids[t] - start;",
     "const int64_t local = (int64_t)ids[t];"),
    ("indexing leaves masked rows unwritten", "memset(out + t * row_bytes, 0, (size_t)row_bytes);",
     "(void)0;"),
    ("indexing reads the mirrored row", "memcpy(out + t * row_bytes, weight + local * row_bytes",
     "memcpy(out + t * row_bytes, weight + (length - 1 - local) * row_bytes"),
]

PIN_CALLS = [
    (pins.test_store_selfcheck_shapes_match_index_put, ()),
    (pins.test_store_of_generated_step_restores_the_drawn_pool, ()),
    (pins.test_softmax_weights_sum_to_one, ()),
    (pins.test_length_one_returns_that_value_row, ()),
    (pins.test_identical_keys_give_mean_of_values, ()),
    (pins.test_merge_closed_forms, ()),
    (pins.test_split_chunk_reading, ()),
    (pins.test_split_then_merge_equals_unsplit, (3,)),
    (pins.test_prefill_matches_torch_sdpa_with_an_explicit_mask, (True,)),
    (pins.test_fresh_prefill_is_torch_causal_attention, ()),
    (pins.test_prefill_single_row_requests_equal_decode, ()),
    (pins.test_prefill_lse_is_the_log_partition, ()),
    (pins.test_rope_closed_forms, ()),
    (pins.test_rope_within_one_rounding_of_the_exact_rotation, ()),
    (pins.test_rope_matches_torch_complex_multiply, ()),
    (pins.test_rope_preserves_relative_position, ()),
    (pins.test_indexing_matches_torch_embedding, ()),
    (pins.test_indexing_shards_sum_to_the_full_lookup, ()),
    (pins.test_indexing_closed_forms, ()),
    (pins.test_prefill_matches_python_loops, ()),
] + [(pins.test_attention_matches_torch_sdpa_fp64, (c,)) for c in range(4)] + [
    (pins.test_attention_matches_python_loops, (c,)) for c in (0, 2, 3)]


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, orig, mut):
    assert SRC.count(orig) == 1, f"mutation site for '{name}' not found or not unique"
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(orig, mut))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-w", str(src), "-o", str(lib), "-lm"], check=True)
    caught = []
    with oracle.use_library(lib):
        for fn, args in PIN_CALLS:
            try:
                fn(*args)
            except (AssertionError, ValueError):
                caught.append(fn.__name__)
    assert caught, f"no pin caught the mutant '{name}'"
