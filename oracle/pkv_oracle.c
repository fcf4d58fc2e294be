/*
 * CPU oracle for one decode step of grouped-query attention over a paged KV
 * cache.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg are the only callers.  It shares no code,
 * header, table or helper with the HIP library, and the library never calls it.
 *
 * Everything is the plain definition, written out:
 *   - the store is a per-row byte copy into a copy of the pools;
 *   - attention is the direct softmax formula in fp64 over the bf16 inputs,
 *     widened exactly to double;
 *   - the split mode applies the same formula to each chunk of positions and
 *     the merge combines (normalised output, log-sum-exp) pairs in fp64.
 *
 * Sources (cited by page and section):
 *   [store]  mini-sglang handbook, "Custom CUDA kernels", section "Moving
 *            whole rows by index": for each new token i, row k[i] goes to
 *            k_cache[out_loc[i]] and the same for v; the self-check in
 *            "Verifying on a machine with no GPU" takes a per-row memcpy as
 *            the reference and requires distinct destinations.
 *   [paged]  AstrAI "CUDA Kernels", section "Q Scheduling and KV Addressing":
 *            the paged KV source only translates logical KV positions into
 *            physical addresses.
 *   [gqa]    same page, "Q Scheduling and KV Addressing": the q heads of one
 *            kv-head group read the same K/V (G = q_heads / kv_heads).
 *   [scale]  same page, section "Python Wrappers" (interface): the softmax
 *            scale is always 1/sqrt(head_dim); layout blhd.
 *   [merge]  cuDNN frontend "CSA Fused Compressor", section "ratio=128": a
 *            chunked softmax keeps a (max, denominator, accumulator) triple
 *            per chunk and merges them in one fixed order.
 *   [rope]   AstrAI "CUDA Kernels", section "Rotary Embedding Kernel": the
 *            rotary embedding looks up fp32 cos/sin for the token's position
 *            and rotates each (head, dimension pair); its reference is a
 *            complex multiply, i.e. the pair (x[2i], x[2i+1]) is the complex
 *            number x[2i] + i x[2i+1], multiplied by cos + i sin.
 *   [prefill] AstrAI "CUDA Kernels", sections "Python Wrappers" (is_causal:
 *            causal mask or none) and "Q Scheduling and KV Addressing" (paged
 *            prefill over a packed [total_q, q_heads, head_dim] query tensor
 *            with qo_indptr; each request has its own KV length).  Reading:
 *            a request's query rows are its last q_len positions, so query
 *            row j of a request with kv_len tokens sits at position
 *            kv_len - q_len + j and, with the causal mask, sees positions
 *            t <= kv_len - q_len + j.
 *   [index]  mini-sglang handbook, "Custom CUDA kernels", section "Moving
 *            whole rows by index": the embedding lookup copies row
 *            ids[t] - start of this rank's vocabulary slice to output row t,
 *            and writes a row of zeros when the id lies outside the slice
 *            [start, start + length) (vocabulary parallelism).
 *
 * Readings where the pages leave a step open:
 *   pool layout [num_pages, page_size, Hkv, D] (rows of Hkv*D per slot);
 *   q head h reads kv head h / G;  split s of a sequence covers positions
 *   [s*chunk, min((s+1)*chunk, L)) with chunk = round_up(ceil(max_L/S), P);
 *   an empty position range gives o = 0 and lse = -inf.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* [store] Overwrite pool row slot_mapping[i] with input row i, byte for byte,
 * in ascending i.  Strides are in bytes.  Returns 0, or -1 on a slot outside
 * [0, num_slots). */
int oracle_kv_store(uint8_t *k_pool, uint8_t *v_pool, int64_t num_slots,
                    int64_t pool_row_stride, const uint8_t *k_new,
                    const uint8_t *v_new, int64_t in_row_stride,
                    const int32_t *slot_mapping, int64_t n, int64_t row_bytes) {
    for (int64_t i = 0; i < n; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0 || slot >= num_slots) return -1;
        memcpy(k_pool + slot * pool_row_stride, k_new + i * in_row_stride, (size_t)row_bytes);
        memcpy(v_pool + slot * pool_row_stride, v_new + i * in_row_stride, (size_t)row_bytes);
    }
    return 0;
}

/* fp32 -> bf16 bits, round to nearest, ties to even; NaN -> quiet NaN 0x7fc0. */
static uint16_t float_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* [rope] Rotate rows of n tokens, each `heads` heads of D bf16 elements at
 * row stride `stride` (elements), by the angle table row positions[t]:
 *     re = x0*c - x1*s,  im = x0*s + x1*c      (c, s = cos/sin[pos, i])
 * for every pair (x0, x1) = (x[2i], x[2i+1]).  The rounding is fixed so that
 * the result is reproducible bit for bit: each product and the sum/difference
 * is one fp32 operation in this order (no contraction: built with
 * -ffp-contract=off), then one bf16 round-to-nearest-even.  Output rows are
 * written contiguously ([n, heads*D]).  Returns 0, or -1 on a position
 * outside [0, table_rows). */
int oracle_rope(uint16_t *out, const uint16_t *x, int64_t n, int64_t heads, int64_t D,
                int64_t stride, const int32_t *positions, const float *cos_t,
                const float *sin_t, int64_t table_rows) {
    const int64_t half = D / 2;
    for (int64_t t = 0; t < n; ++t) {
        const int64_t pos = positions[t];
        if (pos < 0 || pos >= table_rows) return -1;
        for (int64_t h = 0; h < heads; ++h) {
            const uint16_t *xr = x + t * stride + h * D;
            uint16_t *orow = out + (t * heads + h) * D;
            for (int64_t i = 0; i < half; ++i) {
                const float x0 = (float)bf16_to_double(xr[2 * i]);
                const float x1 = (float)bf16_to_double(xr[2 * i + 1]);
                const float c = cos_t[pos * half + i], sn = sin_t[pos * half + i];
                const float a = x0 * c, b = x1 * sn, e = x0 * sn, f = x1 * c;
                orow[2 * i] = float_to_bf16_rne(a - b);
                orow[2 * i + 1] = float_to_bf16_rne(e + f);
            }
        }
    }
    return 0;
}

/* [index] Row gather with the vocabulary-slice mask: out row t is weight row
 * ids[t] - start when start <= ids[t] < start + length, else all zero bytes.
 * out is [n, row_bytes], weight is [length, row_bytes], both contiguous. */
void oracle_indexing(uint8_t *out, const uint8_t *weight, int64_t length, int64_t row_bytes,
                     const int32_t *ids, int64_t n, int64_t start) {
    for (int64_t t = 0; t < n; ++t) {
        const int64_t local = (int64_t)ids[t] - start;
        if (local >= 0 && local < length)
            memcpy(out + t * row_bytes, weight + local * row_bytes, (size_t)row_bytes);
        else
            memset(out + t * row_bytes, 0, (size_t)row_bytes);
    }
}

/* [paged] Physical slot of logical position t of sequence b. */
static int64_t physical_slot(const int32_t *page_table, int64_t max_pages, int64_t b,
                             int64_t t, int64_t page_size) {
    int64_t page = page_table[b * max_pages + t / page_size];
    return page * page_size + t % page_size;
}

typedef struct {
    const uint16_t *q, *k_pool, *v_pool;
    const int32_t *page_table, *seq_lens;
    int64_t B, Hq, Hkv, D, P, max_pages;
} problem;

/* Softmax attention of query row (b, h) over positions [t0, t1).
 * scores[] must hold t1 - t0 doubles.  Writes o[D] (normalised output) and
 * *lse (natural log of the sum of exp(score)); optionally the weights w[].
 * An empty range writes o = 0, lse = -inf. */
static void attend(const problem *p, int64_t b, int64_t h, int64_t t0, int64_t t1,
                   double *scores, double *o, double *lse, double *w) {
    const int64_t D = p->D, G = p->Hq / p->Hkv, g = h / G;   /* [gqa] */
    const int64_t row = p->Hkv * D;                           /* elements per slot */
    const uint16_t *qv = p->q + (b * p->Hq + h) * D;
    const double scale = 1.0 / sqrt((double)D);               /* [scale] */
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    if (t1 <= t0) { *lse = -INFINITY; return; }

    double m = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
        const uint16_t *k = p->k_pool + physical_slot(p->page_table, p->max_pages, b, t, p->P) * row + g * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(qv[d]) * bf16_to_double(k[d]);
        double s = scale * dot;
        scores[t - t0] = s;
        if (s > m) m = s;
    }
    double denom = 0.0;
    for (int64_t t = t0; t < t1; ++t) denom += exp(scores[t - t0] - m);
    for (int64_t t = t0; t < t1; ++t) {
        double wt = exp(scores[t - t0] - m) / denom;
        if (w) w[t - t0] = wt;
        const uint16_t *v = p->v_pool + physical_slot(p->page_table, p->max_pages, b, t, p->P) * row + g * D;
        for (int64_t d = 0; d < D; ++d) o[d] += wt * bf16_to_double(v[d]);
    }
    *lse = m + log(denom);
}

static int check_problem(const problem *p) {
    if (p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->D <= 0 || p->P <= 0 || p->max_pages < 0) return -2;
    if (p->Hq % p->Hkv) return -2;
    for (int64_t b = 0; b < p->B; ++b)
        if (p->seq_lens[b] < 0 || p->seq_lens[b] > p->max_pages * p->P) return -2;
    return 0;
}

static int64_t longest(const problem *p) {
    int64_t L = 0;
    for (int64_t b = 0; b < p->B; ++b) if (p->seq_lens[b] > L) L = p->seq_lens[b];
    return L;
}

/* Full (unsplit) attention for every (b, h): out[B,Hq,D], lse[B,Hq]. */
int oracle_paged_decode(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                        const int32_t *page_table, const int32_t *seq_lens,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t P,
                        int64_t max_pages, double *out, double *lse) {
    problem p = {q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D, P, max_pages};
    int rc = check_problem(&p);
    if (rc) return rc;
    const int64_t Lmax = longest(&p);
    int failed = 0;
#pragma omp parallel
    {
        double *scores = malloc((size_t)(Lmax > 0 ? Lmax : 1) * sizeof(double));
        if (!scores) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * Hq; ++bh) {
            if (!scores) continue;
            int64_t b = bh / Hq, h = bh % Hq;
            attend(&p, b, h, 0, seq_lens[b], scores, out + bh * D, lse + bh, NULL);
        }
        free(scores);
    }
    return failed ? -5 : 0;
}

/* [prefill] Attention of every packed query row.  q [total_q, Hq, D] bf16 with
 * total_q = qo_indptr[B]; kv_lens[b] tokens of request b in the paged pools.
 * out [total_q, Hq, D] fp64, lse [total_q, Hq] (natural log).  Returns 0,
 * -2 on inconsistent sizes (q_len > kv_len, decreasing qo_indptr). */
int oracle_paged_prefill(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                         const int32_t *page_table, const int32_t *kv_lens,
                         const int32_t *qo_indptr, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                         int64_t P, int64_t max_pages, int causal, const int64_t *rows,
                         int64_t n_rows, double *out, double *lse) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0 || Hq % Hkv || qo_indptr[0] != 0) return -2;
    int64_t Lmax = 1;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t ql = qo_indptr[b + 1] - qo_indptr[b];
        if (ql < 0 || ql > kv_lens[b] || kv_lens[b] > max_pages * P) return -2;
        if (kv_lens[b] > Lmax) Lmax = kv_lens[b];
    }
    const int64_t total_q = qo_indptr[B], G = Hq / Hkv, row = Hkv * D;
    const double qk_scale = 1.0 / sqrt((double)D);   /* [scale] */
    int failed = 0;
#pragma omp parallel
    {
        double *scores = malloc((size_t)Lmax * sizeof(double));
        if (!scores) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < (rows ? n_rows : total_q * Hq); ++n) {
            if (!scores) continue;
            /* output slot n holds packed row i, head h (all of them in order, or rows[n]) */
            const int64_t qh = rows ? rows[2 * n] * Hq + rows[2 * n + 1] : n;
            if (qh < 0 || qh >= total_q * Hq) continue;
            const int64_t i = qh / Hq, h = qh % Hq, g = h / G;
            int64_t b = 0;
            while (qo_indptr[b + 1] <= i) ++b;          /* the request of packed row i */
            const int64_t ql = qo_indptr[b + 1] - qo_indptr[b], L = kv_lens[b];
            const int64_t pos = L - ql + (i - qo_indptr[b]);
            const int64_t t1 = causal ? pos + 1 : L;    /* positions [0, t1) are seen */
            const uint16_t *qv = q + (i * Hq + h) * D;
            double *o = out + n * D;
            double m = -INFINITY;
            for (int64_t t = 0; t < t1; ++t) {
                const uint16_t *k = k_pool + physical_slot(page_table, max_pages, b, t, P) * row + g * D;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(qv[d]) * bf16_to_double(k[d]);
                scores[t] = qk_scale * dot;
                if (scores[t] > m) m = scores[t];
            }
            double den = 0.0;
            for (int64_t t = 0; t < t1; ++t) den += exp(scores[t] - m);
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t t = 0; t < t1; ++t) {
                const double w = exp(scores[t] - m) / den;
                const uint16_t *v = v_pool + physical_slot(page_table, max_pages, b, t, P) * row + g * D;
                for (int64_t d = 0; d < D; ++d) o[d] += w * bf16_to_double(v[d]);
            }
            lse[n] = t1 > 0 ? m + log(den) : -INFINITY;
        }
        free(scores);
    }
    return failed ? -5 : 0;
}

/* Attention for a chosen list of (b, h) rows only: rows[2*i] = b, rows[2*i+1] = h.
 * out[n_rows, D], lse[n_rows].  Used to check single outputs of very large
 * problems one by one. */
int oracle_paged_decode_rows(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *page_table, const int32_t *seq_lens,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t P,
                             int64_t max_pages, const int64_t *rows, int64_t n_rows,
                             double *out, double *lse) {
    problem p = {q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D, P, max_pages};
    int rc = check_problem(&p);
    if (rc) return rc;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[2 * i] < 0 || rows[2 * i] >= B || rows[2 * i + 1] < 0 || rows[2 * i + 1] >= Hq) return -2;
    const int64_t Lmax = longest(&p);
    int failed = 0;
#pragma omp parallel
    {
        double *scores = malloc((size_t)(Lmax > 0 ? Lmax : 1) * sizeof(double));
        if (!scores) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (!scores) continue;
            int64_t b = rows[2 * i], h = rows[2 * i + 1];
            attend(&p, b, h, 0, seq_lens[b], scores, out + i * D, lse + i, NULL);
        }
        free(scores);
    }
    return failed ? -5 : 0;
}

/* Softmax weights of row (b, h) over its L = seq_lens[b] positions: w[L]. */
int oracle_softmax_weights(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                           const int32_t *page_table, const int32_t *seq_lens,
                           int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t P,
                           int64_t max_pages, int64_t b, int64_t h, double *w) {
    problem p = {q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D, P, max_pages};
    int rc = check_problem(&p);
    if (rc) return rc;
    if (b < 0 || b >= B || h < 0 || h >= Hq) return -2;
    int64_t L = seq_lens[b];
    double *scores = malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
    double *o = malloc((size_t)D * sizeof(double));
    if (!scores || !o) { free(scores); free(o); return -5; }
    double lse;
    attend(&p, b, h, 0, L, scores, o, &lse, w);
    free(scores);
    free(o);
    return 0;
}

/* Reading of the split plan: chunk = round_up(ceil(max_seq_len / S), P). */
int64_t oracle_split_chunk(int64_t max_seq_len, int64_t num_splits, int64_t page_size) {
    if (max_seq_len <= 0 || num_splits <= 0 || page_size <= 0) return 0;
    int64_t per = (max_seq_len + num_splits - 1) / num_splits;
    return (per + page_size - 1) / page_size * page_size;
}

/* Split mode: for every (b, h, s), attention over positions
 * [s*chunk, min((s+1)*chunk, L_b)).  o_part[B,Hq,S,D], lse_part[B,Hq,S]. */
int oracle_paged_decode_split(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                              const int32_t *page_table, const int32_t *seq_lens,
                              int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t P,
                              int64_t max_pages, int64_t chunk, int64_t S,
                              double *o_part, double *lse_part) {
    problem p = {q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D, P, max_pages};
    int rc = check_problem(&p);
    if (rc) return rc;
    if (chunk <= 0 || S <= 0) return -2;
    int failed = 0;
#pragma omp parallel
    {
        double *scores = malloc((size_t)chunk * sizeof(double));
        if (!scores) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < B * Hq * S; ++i) {
            if (!scores) continue;
            int64_t s = i % S, bh = i / S, b = bh / Hq, h = bh % Hq;
            int64_t t0 = s * chunk, t1 = (s + 1) * chunk;
            if (t1 > seq_lens[b]) t1 = seq_lens[b];
            attend(&p, b, h, t0, t1, scores, o_part + i * D, lse_part + i, NULL);
        }
        free(scores);
    }
    return failed ? -5 : 0;
}

/* [merge] Combine S partials per row in ascending s:
 *   M = max_s lse_s,  w_s = exp(lse_s - M),
 *   out = sum_s w_s o_s / sum_s w_s,  lse = M + log(sum_s w_s).
 * A row whose partials are all empty (M = -inf) gives out = 0, lse = -inf.
 * o_part[rows,S,D], lse_part[rows,S] -> out[rows,D], lse[rows]. */
void oracle_merge(const double *o_part, const double *lse_part, int64_t rows, int64_t S,
                  int64_t D, double *out, double *lse) {
    for (int64_t r = 0; r < rows; ++r) {
        const double *lr = lse_part + r * S;
        double *o = out + r * D;
        double M = -INFINITY;
        for (int64_t s = 0; s < S; ++s) if (lr[s] > M) M = lr[s];
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
        double den = 0.0;
        for (int64_t s = 0; s < S; ++s) {
            double ws = exp(lr[s] - M);
            den += ws;
            const double *os = o_part + (r * S + s) * D;
            for (int64_t d = 0; d < D; ++d) o[d] += ws * os[d];
        }
        for (int64_t d = 0; d < D; ++d) o[d] /= den;
        lse[r] = M + log(den);
    }
}

/* Number of threads the parallel regions use (for reporting). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
