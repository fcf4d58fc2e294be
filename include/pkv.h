/*
 * pkv.h -- C ABI of libpkv.so: one decode step of grouped-query attention
 * over a paged KV cache, on AMD MI355X (gfx950).
 *
 *   pkv_kv_store          scatter the step's new K/V rows into the page pool
 *   pkv_kv_store_rope     the store with K rows rotated by a rotary embedding on the way
 *   pkv_paged_decode_attn_rope  the attention with q rotated in its prologue
 *   pkv_paged_prefill_attn  attention of packed multi-token queries (prefill)
 *   pkv_prefill_plan      the Q-tile work map of a prefill batch (host only)
 *   pkv_indexing          row gather from a vocabulary slice (embedding lookup)
 *   pkv_paged_decode_attn split-KV attention through the page table -> partials
 *   pkv_paged_decode_attn_valu  the same on the vector ALUs only (measured alternative)
 *   pkv_decode_merge      log-sum-exp merge of the partials -> bf16 output
 *   pkv_paged_decode_attn_merged  the attention and the merge in one call
 *   pkv_paged_decode_attn_merged_static  the same without workspace or allocation
 *   pkv_decode_step       store, attention and merge in one call (one kernel at S = 1)
 *   pkv_num_splits        split-count heuristic (host only)
 *   pkv_num_splits_batch  the same, given the group size and token count (host only)
 *   pkv_split_chunk       positions per split for a split count (host only)
 *   pkv_status_str        text of a status code
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers unless stated; every buffer belongs to the
 *     caller.  The library never allocates, frees or synchronises (its one
 *     static array is described at pkv_paged_decode_attn_merged_static): each call
 *     validates its arguments on the host, enqueues its kernels on `stream`
 *     (a hipStream_t; NULL = the default stream) and returns.
 *   - A negative status means that nothing was launched (except PKV_ERR_HIP,
 *     reported when the launch itself failed).
 *   - Device-side preconditions are not checked on the host (that would need a
 *     synchronisation); the kernels never access memory outside the buffers
 *     the sizes describe, whatever the index contents (see each call).
 *
 * Layouts (bf16 = 2-byte IEEE bfloat16 bit patterns, row-major):
 *   q            [B, Hq, D]                      contiguous
 *   k_pool/v_pool[num_pages, page_size, Hkv, D]  == [num_slots, Hkv*D] rows
 *   page_table   int32 [B, max_pages_per_seq]    page ids of each sequence, in order
 *   seq_lens     int32 [B]                       tokens of each sequence, the new one included
 *   slot_mapping int32 [n]                       destination slot of each new row
 *   o_partial    fp32 [B, Hq, num_splits, D]     normalised per-split outputs
 *   lse_partial  fp32 [B, Hq, num_splits]        per-split natural-log sum-exp
 *   out          bf16 [B, Hq, D];  lse_out fp32 [B, Hq] (optional)
 */
#ifndef PKV_H
#define PKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;

#define PKV_OK 0
#define PKV_ERR_NULL (-1)        /* a required pointer is NULL                       */
#define PKV_ERR_SHAPE (-2)       /* a size is out of range or inconsistent           */
#define PKV_ERR_UNSUPPORTED (-3) /* head_dim / group size / page size not supported  */
#define PKV_ERR_ALIGN (-4)       /* a base pointer or stride is not 16-byte aligned  */
#define PKV_ERR_HIP (-5)         /* the HIP runtime reported a launch failure        */
#define PKV_ERR_SCRATCH (-6)     /* the partials do not fit the static scratch buffer */

/*
 * pkv_kv_store -- write n new rows into the K and V pools by slot index.
 *
 * Follows: mini-sglang handbook, "Custom CUDA kernels", section "Moving whole
 * rows by index" (k_cache[out_loc[i]] <- k[i], same for v; a pure row move)
 * and section "Hooking into PyTorch" (int32 indices, rows contiguous, free row
 * strides, n == 0 returns at once, the stream handed in by the caller).
 *
 *   k_pool, v_pool    device, num_slots rows of pool_row_stride elements
 *   k_new, v_new      device, n rows of in_row_stride elements
 *   slot_mapping      device int32 [n]; row i goes to slot slot_mapping[i]
 *   row_elems         elements copied per row (Hkv*D); <= both strides
 *   elem_bytes        1, 2, 4 or 8 (2 for bf16)
 * Strides are in elements.  Rows move in 16-byte units when both bases, both
 * strides and the row length are 16-byte multiples, otherwise in the largest
 * unit (8, 4, 2, 1 bytes) that divides all of them; the bytes written are
 * identical either way.
 * Preconditions (device): slots distinct.  A slot outside [0, num_slots) is
 * skipped, never written.  Two rows naming one slot race.
 * Returns PKV_OK (n == 0: nothing launched), PKV_ERR_NULL, PKV_ERR_SHAPE,
 * PKV_ERR_UNSUPPORTED (elem_bytes), PKV_ERR_HIP.
 */
pkv_status pkv_kv_store(void *k_pool, void *v_pool, int64_t num_slots, int64_t pool_row_stride,
                        const void *k_new, const void *v_new, int64_t in_row_stride,
                        const int32_t *slot_mapping, int64_t n, int64_t row_elems,
                        int32_t elem_bytes, void *stream);

/*
 * Rotary embedding (both entry points below).
 *
 * Follows: AstrAI "CUDA Kernels", section "Rotary Embedding Kernel" (fp32
 * cos/sin of a token's position rotate every (head, dimension pair); the
 * reference is a complex multiply).  Rows are bf16; within each head of D
 * elements the pair (x[2i], x[2i+1]) is the complex number x[2i] + i x[2i+1],
 * multiplied by cos[pos, i] + i sin[pos, i]:
 *     x'[2i]   = x[2i] * c - x[2i+1] * s
 *     x'[2i+1] = x[2i] * s + x[2i+1] * c
 * each product and the difference/sum one fp32 operation in this order (no
 * fused multiply-add), then one bf16 round-to-nearest-even per element (NaN ->
 * 0x7fc0).  Tables: rope_cos, rope_sin fp32 [rope_rows, D/2], contiguous,
 * 16-byte aligned (else PKV_ERR_ALIGN); the caller fills them (for example
 * with theta_i = base^(-2i/D) and angle = pos * theta_i).  A position outside
 * [0, rope_rows) rotates nothing: the affected row comes out NaN.
 */

/*
 * pkv_kv_store_rope -- pkv_kv_store for bf16 rows of Hkv heads x D, with every
 * K row rotated by the rotary embedding of positions[i] before it is written
 * (V rows are copied unchanged).  The rotated K goes straight to the pool: no
 * separate pass over K.
 *   positions  device int32 [n]: position of new row i (its table row)
 *   Hkv, D     heads per row and head size (D a multiple of 8); rows are
 *              Hkv*D bf16 elements, strides in elements
 * Both pool and input bases and strides must be 16-byte multiples (else
 * PKV_ERR_ALIGN).  Slots as for pkv_kv_store (outside the pool: skipped).
 * Returns PKV_OK (n == 0: nothing launched), PKV_ERR_NULL, PKV_ERR_SHAPE,
 * PKV_ERR_ALIGN, PKV_ERR_HIP.
 */
pkv_status pkv_kv_store_rope(void *k_pool, void *v_pool, int64_t num_slots,
                             int64_t pool_row_stride, const void *k_new, const void *v_new,
                             int64_t in_row_stride, const int32_t *slot_mapping, int64_t n,
                             int32_t Hkv, int32_t D, const int32_t *positions,
                             const float *rope_cos, const float *rope_sin, int32_t rope_rows,
                             void *stream);

/*
 * pkv_paged_prefill_attn -- attention of packed multi-token queries (a prefill
 * or a prefill chunk) over the paged pool.
 *
 * Follows: AstrAI "CUDA Kernels", section "Q Scheduling and KV Addressing"
 * (packed queries, the Q tile work map of pkv_prefill_plan, paged KV
 * addressing, GQA head packing) and section "Python Wrappers" (is_causal; scale
 * 1/sqrt(head_dim)).  Request b has kv_lens[b] tokens in the pool (its new ones
 * already stored) and query rows qo_indptr[b] .. qo_indptr[b+1]-1, which are
 * its last q_len = qo_indptr[b+1] - qo_indptr[b] positions: row j of the
 * request sits at position p_j = kv_lens[b] - q_len + j.  For q head h
 * (kv head g = h / (Hq/Hkv)):
 *     x_t = scale * <q[row, h, :], K[phys(b, t), g, :]>   over t in T_j
 *     out[row, h, :] = sum_{t in T_j} softmax(x)_t V[phys(b, t), g, :]
 *     lse[row, h] = ln sum_{t in T_j} exp(x_t)          (if lse != NULL)
 * with T_j = [0, p_j] when causal != 0, else [0, kv_lens[b]).  fp32 softmax
 * statistics and accumulation; the probabilities enter the P.V product as
 * bf16 (the matrix-core operand); out is bf16 (RNE).
 *   q            device bf16 [total_q, Hq, D], 16-byte aligned
 *   qo_indptr    device int32 [B + 1];  q_tile_to_batch / q_tile_to_index
 *                device int32 [num_q_tiles], as built by pkv_prefill_plan
 *   kv_lens      device int32 [B];  pools and page_table as for decode
 *   out          device bf16 [total_q, Hq, D], 8-byte aligned
 *   D in {64, 128}; Hq/Hkv in {1, 2, 4, 8}; page_size a power of two <= 1024.
 * Preconditions (device): q_len <= kv_lens[b] <= max_pages_per_seq*page_size
 * and a work map built for these qo_indptr.  Rows and positions outside
 * total_q and the page table are never touched; a row that sees no position
 * comes out NaN, and so does a row that would use a page id outside the pool.
 */
pkv_status pkv_paged_prefill_attn(const void *q, const void *k_pool, const void *v_pool,
                                  const int32_t *page_table, const int32_t *kv_lens,
                                  const int32_t *qo_indptr, const int32_t *q_tile_to_batch,
                                  const int32_t *q_tile_to_index, int32_t num_q_tiles,
                                  int32_t total_q, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t page_size, int32_t num_pages, int32_t max_pages_per_seq,
                                  int32_t causal, float scale, void *out, float *lse,
                                  void *stream);

/*
 * pkv_paged_decode_attn_rope -- pkv_paged_decode_attn with q rotated by the
 * rotary embedding of q_positions[b] (device int32 [B]) in the kernel's
 * prologue; the rotated q is rounded to bf16 exactly as a separately rotated
 * q would be, so the result equals pkv_paged_decode_attn on that q, bit for
 * bit.  Other arguments, layouts and status codes as pkv_paged_decode_attn.
 */
pkv_status pkv_paged_decode_attn_rope(const void *q, const void *k_pool, const void *v_pool,
                                      const int32_t *page_table, const int32_t *seq_lens,
                                      int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                      int32_t page_size, int32_t num_pages,
                                      int32_t max_pages_per_seq, int32_t max_seq_len,
                                      int32_t num_splits, float scale, float *o_partial,
                                      float *lse_partial, const int32_t *q_positions,
                                      const float *rope_cos, const float *rope_sin,
                                      int32_t rope_rows, void *stream);

/*
 * pkv_indexing -- row gather from one rank's slice of a vocabulary-parallel
 * embedding table.
 *
 * Follows: mini-sglang handbook, "Custom CUDA kernels", section "Moving whole
 * rows by index" (the embedding lookup: output row t is the table row of
 * token ids[t], or a row of zeros when the id falls outside this rank's slice
 * of the vocabulary, so that an all-reduce over the ranks yields the lookup in
 * the whole table).
 *
 *   out      device, [n, row_elems] contiguous; every row is written
 *   weight   device, [length, row_elems] contiguous: vocabulary rows
 *            start .. start + length - 1 (may be NULL when length == 0)
 *   ids      device int32 [n]
 *   elem_bytes 1, 2, 4 or 8
 *     out[t] = weight[ids[t] - start]  if start <= ids[t] < start + length
 *            = 0 (all bytes)           otherwise
 * Rows move in the largest unit (16, 8, 4, 2, 1 bytes) dividing the row length
 * and both base addresses.  Any id is safe: only in-slice rows are read.
 * Returns PKV_OK (n == 0: nothing launched), PKV_ERR_NULL, PKV_ERR_SHAPE,
 * PKV_ERR_UNSUPPORTED (elem_bytes), PKV_ERR_HIP.
 */
pkv_status pkv_indexing(void *out, const void *weight, int64_t length, int64_t row_elems,
                        int32_t elem_bytes, const int32_t *ids, int64_t n, int64_t start,
                        void *stream);

/*
 * pkv_paged_decode_attn -- split-KV decode attention over the paged pool.
 *
 * Follows: AstrAI "CUDA Kernels", section "Overview" (split-KV GQA decode, the
 * paged source shares the kernel body), section "Q Scheduling and KV
 * Addressing" (the paged source turns a logical position into a physical
 * address; the q heads of one kv-head group share each K/V tile), section
 * "Python Wrappers" (scale 1/sqrt(head_dim)).
 *
 * For every sequence b, q head h (kv head g = h / (Hq/Hkv)) and split s, over
 * positions t in [s*chunk, min((s+1)*chunk, seq_lens[b])) with
 * chunk = pkv_split_chunk(max_seq_len, num_splits, page_size) and slot
 * r(t) = page_table[b, t / page_size] * page_size + t % page_size:
 *     x_t = scale * <q[b,h,:], K[r(t), g, :]>
 *     o_partial[b,h,s,:]  = sum_t softmax(x)_t V[r(t), g, :]
 *     lse_partial[b,h,s]  = ln sum_t exp(x_t)
 * fp32 arithmetic on the bf16 inputs.  An empty range writes o = 0 and
 * lse = -inf.  Every element of o_partial / lse_partial is written.
 *
 *   head_dim D in {64, 128}; group Hq/Hkv in {1, 2, 4, 8}; page_size a power of
 *   two in [1, 1024]; num_splits in [1, 1024]; max_seq_len in [0, max_pages_per_seq*page_size];
 *   num_splits * Hkv * B < 2^31 (the workgroup count).
 *   q, k_pool, v_pool 16-byte aligned (else PKV_ERR_ALIGN).
 * Preconditions (device): seq_lens[b] <= max_seq_len.  Positions past
 * num_splits*chunk are not visited.  A page id outside [0, num_pages) makes
 * that row's output NaN instead of being read.
 */
pkv_status pkv_paged_decode_attn(const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *page_table, const int32_t *seq_lens, int32_t B,
                                 int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                                 int32_t num_pages, int32_t max_pages_per_seq,
                                 int32_t max_seq_len, int32_t num_splits, float scale,
                                 float *o_partial, float *lse_partial, void *stream);

/*
 * pkv_paged_decode_attn_valu -- pkv_paged_decode_attn computed by the all-VALU
 * kernel instead of the matrix-core one: the same contract, arguments, status
 * codes and results (up to fp32 summation order), plus num_splits <= 65535.
 * Kept as the measured alternative of the choice to run QK^T on the matrix
 * cores (AstrAI "CUDA Kernels", section "File Layout", runs decode on mma
 * tiles; here the fp32 dot products run on the vector ALUs, one online-softmax
 * state per token slot, merged at the end).  It is roughly half as fast on
 * grouped heads and is selected only by calling it.
 */
pkv_status pkv_paged_decode_attn_valu(const void *q, const void *k_pool, const void *v_pool,
                                      const int32_t *page_table, const int32_t *seq_lens,
                                      int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                      int32_t page_size, int32_t num_pages,
                                      int32_t max_pages_per_seq, int32_t max_seq_len,
                                      int32_t num_splits, float scale, float *o_partial,
                                      float *lse_partial, void *stream);

/*
 * pkv_decode_merge -- combine the split partials of every (b, h) row.
 *
 * Follows: cuDNN frontend "CSA Fused Compressor", section "ratio=128" (chunked
 * softmax: per-chunk (max, denominator, accumulator) triples merged in one
 * fixed order) and section "Numerics" (fp32 throughout, one final bf16
 * rounding, bitwise run-to-run determinism).
 *     M = max_s lse_s,  w_s = exp(lse_s - M)
 *     out = bf16_rne( sum_s w_s o_s / sum_s w_s )   (s ascending)
 *     lse_out = M + ln sum_s w_s                    (if lse_out != NULL)
 * A row whose splits are all empty gives out = 0 and lse_out = -inf.
 *   D in {64, 128}; num_splits in [1, 1024]; out 16-byte aligned.
 */
pkv_status pkv_decode_merge(const float *o_partial, const float *lse_partial, int32_t B,
                            int32_t Hq, int32_t D, int32_t num_splits, void *out, float *lse_out,
                            void *stream);

/*
 * pkv_paged_decode_attn_merged -- pkv_paged_decode_attn followed by
 * pkv_decode_merge, in one call, with the same results bit for bit.
 *
 * Follows the same passages as those two calls (AstrAI "CUDA Kernels",
 * "Q Scheduling and KV Addressing"; cuDNN frontend "CSA Fused Compressor",
 * "ratio=128" and "Numerics").  With num_splits == 1 the merge of a single
 * split is its own output (weight exp(0) = 1): one kernel writes out (and
 * lse_out) directly, without partials, and o_partial / lse_partial may be
 * NULL.  With num_splits > 1 the attention writes the partials (required)
 * and the merge runs as a second launch on the same stream.
 *   Arguments as pkv_paged_decode_attn, plus
 *   out      device bf16 [B, Hq, D], 16-byte aligned
 *   lse_out  device fp32 [B, Hq] or NULL
 * Status codes as the two calls; nothing is launched on an error.
 */
pkv_status pkv_paged_decode_attn_merged(const void *q, const void *k_pool, const void *v_pool,
                                        const int32_t *page_table, const int32_t *seq_lens,
                                        int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t page_size, int32_t num_pages,
                                        int32_t max_pages_per_seq, int32_t max_seq_len,
                                        int32_t num_splits, float scale, float *o_partial,
                                        float *lse_partial, void *out, float *lse_out,
                                        void *stream);

/*
 * pkv_paged_decode_attn_merged_static -- pkv_paged_decode_attn_merged with no
 * workspace argument and no allocation of any kind, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  With num_splits > 1 the split partials go
 * to a static device array of the library (16 MiB, one copy per GPU, held
 * until the process ends) instead of caller buffers; the kernels, and so the
 * out / lse_out bits, are those of pkv_paged_decode_attn_merged.
 *   Arguments as pkv_paged_decode_attn_merged without o_partial / lse_partial.
 *   Limit: B * Hq * num_splits * D floats, rounded up to a multiple of 64,
 *   plus B * Hq * num_splits floats must not exceed 4 Mi (16 MiB); otherwise
 *   PKV_ERR_SCRATCH and nothing is launched.  num_splits == 1 uses no scratch.
 *   The array of a GPU is found (hipGetSymbolAddress) on the first call on
 *   that GPU, which must be the GPU current on the calling thread and the
 *   stream's; later calls only launch.
 *   Every call on one GPU shares that GPU's array, and the attention writes
 *   every partial before the merge reads it, so nothing needs clearing between
 *   calls; calls whose kernels overlap on one GPU (other streams, other
 *   threads) race on it and must be serialised by the caller.
 * Status codes as pkv_paged_decode_attn_merged, plus PKV_ERR_SCRATCH.
 */
pkv_status pkv_paged_decode_attn_merged_static(const void *q, const void *k_pool,
                                               const void *v_pool, const int32_t *page_table,
                                               const int32_t *seq_lens, int32_t B, int32_t Hq,
                                               int32_t Hkv, int32_t D, int32_t page_size,
                                               int32_t num_pages, int32_t max_pages_per_seq,
                                               int32_t max_seq_len, int32_t num_splits,
                                               float scale, void *out, float *lse_out,
                                               void *stream);

/*
 * pkv_decode_step -- one whole decode step: pkv_kv_store of one new row per
 * sequence, then pkv_paged_decode_attn_merged, in one call, with the same
 * pools, output and lse bit for bit.
 *
 * Follows the passages of those calls (mini-sglang handbook, "Custom CUDA
 * kernels", "Moving whole rows by index"; AstrAI "CUDA Kernels", "Q
 * Scheduling and KV Addressing"; cuDNN frontend "CSA Fused Compressor",
 * "ratio=128").  The store is fused into the attention kernel: the workgroup
 * of head g whose split holds position seq_lens[b] - 1 copies head g of row b
 * of k_new / v_new to pool slot slot_mapping[b], and the attention takes that
 * position from the new row itself.  With num_splits == 1 the whole step is
 * one kernel and o_partial / lse_partial may be NULL; otherwise the merge
 * runs as a second launch.
 *   k_new, v_new   device bf16 [B, new_row_stride], 16-byte aligned; row b is
 *                  the new token of sequence b, Hkv*D values per row
 *   new_row_stride elements between rows, >= Hkv*D, a multiple of 8
 *   slot_mapping   device int32 [B]; slots outside [0, num_pages*page_size)
 *                  are not written (as pkv_kv_store)
 *   k_pool, v_pool written (one row per sequence); other arguments as
 *                  pkv_paged_decode_attn_merged
 * Preconditions (device, as in the unfused step): seq_lens[b] >= 1 counts the
 * new token, and slot_mapping[b] is the slot of its position seq_lens[b] - 1
 * (page_table[b][(L-1)/P]*P + (L-1)%P); the slots are distinct.
 */
pkv_status pkv_decode_step(const void *q, const void *k_new, const void *v_new,
                           int64_t new_row_stride, const int32_t *slot_mapping, void *k_pool,
                           void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                           int32_t num_pages, int32_t max_pages_per_seq, int32_t max_seq_len,
                           int32_t num_splits, float scale, float *o_partial, float *lse_partial,
                           void *out, float *lse_out, void *stream);

/*
 * pkv_num_splits -- split count for a batch (host only, no GPU call).
 *
 * The pages only say the launcher does the split-K arithmetic and that small
 * batches underfill the GPU despite split-KV (AstrAI "CUDA Kernels", sections
 * "File Layout" and "Known Optimization Targets"); the rule is a reading,
 * tuned by measurement on MI355X.  This form knows neither the group size nor
 * the lengths, so it counts one workgroup per (sequence, kv head, split) and
 * takes the batch as ragged:
 *     S = clamp(max(ceil(num_cus / (B * Hkv)), ceil(max_seq_len / 2048)),
 *               1, min(1024, max(1, ceil(max_seq_len / 256))))
 * pkv_num_splits_batch is the form for callers that know the group size and
 * the token count.
 * Returns >= 1 for valid arguments, PKV_ERR_SHAPE otherwise (B, Hkv or num_cus
 * below 1, max_seq_len negative, page_size not a power of two).
 */
int32_t pkv_num_splits(int32_t B, int32_t Hkv, int32_t max_seq_len, int32_t page_size,
                       int32_t num_cus);

/*
 * pkv_num_splits_batch -- pkv_num_splits for a batch whose group size and
 * token count the caller knows (a serving scheduler does); host only.
 *     streams = B * Hkv / hb                    workgroups per split: hb = 1, or
 *               with one q head per kv head (Hq == Hkv) the row kernel's heads
 *               per workgroup, counted as 8 when Hkv % 8 == 0, else 4 when
 *               Hkv % 4 == 0 (512 / D is 8 at D = 64 and 4 at D = 128)
 *     S_fill  = ceil(w * num_cus / streams)     w = 2 if Hq/Hkv >= 8, else 1
 *     ragged  = total_tokens < 0 (unknown) or total_tokens < 0.9 * B * max_seq_len
 *     S       = ragged ? max(S_fill, ceil(max_seq_len / 2048)) : S_fill
 *     S       = clamp(S, 1, min(1024, max(1, ceil(max_seq_len / 256))))
 * total_tokens is the sum of the batch's sequence lengths, or any negative
 * value when unknown.  Uniform batches keep one split per workgroup stream
 * while that fills the GPU; ragged ones are cut into splits of at most 2048
 * positions, so that the workgroups of long sequences are not the last to
 * finish.  Returns as pkv_num_splits (also PKV_ERR_SHAPE when Hq is not a
 * multiple of Hkv).
 */
int32_t pkv_num_splits_batch(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_seq_len,
                             int64_t total_tokens, int32_t page_size, int32_t num_cus);

/*
 * pkv_prefill_plan -- the packed-query work map of a prefill batch (host only).
 *
 * Follows: AstrAI "CUDA Kernels", section "Q Scheduling and KV Addressing" (a
 * packed [total_q, q_heads, head_dim] query tensor is cut into Q tiles of 64
 * rows per request; each tile knows its request and its tile index within the
 * request, so a workgroup finds its rows in O(1): for Q lengths [70, 10, 130]
 * the page prints qo_indptr [0, 70, 80, 210], tile->request [0, 0, 1, 2, 2, 2]
 * and tile->index [0, 1, 0, 0, 1, 2]).
 *   q_lens            host int32 [B]: query rows of each request (>= 0)
 *   qo_indptr         host int32 [B + 1]: exclusive prefix sums of q_lens
 *   q_tile_to_batch   host int32 [capacity]: request of each tile
 *   q_tile_to_index   host int32 [capacity]: tile index within its request
 * Tiles are PKV_PREFILL_TILE_ROWS rows.  Returns the number of tiles; with
 * either tile array NULL only that number (a size query); PKV_ERR_SHAPE if it
 * exceeds capacity or a length is negative, PKV_ERR_NULL for missing arrays.
 */
#define PKV_PREFILL_TILE_ROWS 64
int32_t pkv_prefill_plan(const int32_t *q_lens, int32_t B, int32_t *qo_indptr,
                         int32_t *q_tile_to_batch, int32_t *q_tile_to_index, int32_t capacity);

/* pkv_split_chunk -- positions covered by one split: the smallest multiple of
 * page_size >= ceil(max_seq_len / num_splits).  0 if max_seq_len == 0,
 * PKV_ERR_SHAPE for invalid arguments.  Host only. */
int32_t pkv_split_chunk(int32_t max_seq_len, int32_t num_splits, int32_t page_size);

/* pkv_status_str -- static text for a status code (never NULL). */
const char *pkv_status_str(pkv_status s);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
