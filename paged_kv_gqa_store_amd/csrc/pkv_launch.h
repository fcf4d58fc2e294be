// Host-side launchers of the libpkv kernels (internal header; the exported
// C ABI lives in include/pkv.h and validates every argument before these run).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Arguments of one split-KV decode launch, already validated.
struct DecodeParams {
  const uint16_t *q;         // [B, Hq, D] bf16
  const uint16_t *k_pool;    // [num_pages, P, Hkv, D] bf16
  const uint16_t *v_pool;
  const int32_t *page_table; // [B, max_pages]
  const int32_t *seq_lens;   // [B]
  float *o_partial;          // [B, Hq, S, D]
  float *lse_partial;        // [B, Hq, S]
  int B, Hq, Hkv, D, G;
  int page_log2;             // page_size = 1 << page_log2
  int num_pages, max_pages;
  int num_splits, chunk;     // split s covers [s*chunk, (s+1)*chunk)
  int longest_first;         // workgroups take the (sequence, split) pairs longest first
  float scale_log2;          // softmax scale * log2(e)
  // rotary embedding of q (all NULL / 0 when q is used as given)
  const int32_t *q_pos;      // [B] position of each sequence's query token
  const float *rope_cos;     // [rope_rows, D/2] fp32
  const float *rope_sin;
  int rope_rows;
  // with one split, the merged result written directly (NULL: write partials)
  uint16_t *out;             // [B, Hq, D] bf16
  float *lse_out;            // [B, Hq] or NULL
  // the step's kv_store fused in (k_new NULL when not): row b of k_new / v_new
  // goes to pool slot slots[b], and is position seq_lens[b] - 1
  const uint16_t *k_new;
  const uint16_t *v_new;
  int64_t new_stride;        // elements between rows of k_new / v_new
  const int32_t *slots;      // [B]
  int64_t num_slots;         // num_pages * page_size
};

hipError_t launch_kv_store(void *k_pool, void *v_pool, int64_t num_slots, int64_t pool_stride_b,
                           const void *k_new, const void *v_new, int64_t in_stride_b,
                           const int32_t *slots, int64_t n, int64_t row_b, int unit_b,
                           hipStream_t stream);

hipError_t launch_kv_store_rope(void *k_pool, void *v_pool, int64_t num_slots,
                               int64_t pool_stride_b, const void *k_new, const void *v_new,
                               int64_t in_stride_b, const int32_t *slots, int64_t n, int Hkv,
                               int D, const int32_t *positions, const float *rope_cos,
                               const float *rope_sin, int rope_rows, hipStream_t stream);

hipError_t launch_gather_rows(void *out, const void *weight, int64_t length, const int32_t *ids,
                              int64_t n, int64_t start, int64_t row_b, int unit_b,
                              hipStream_t stream);

// Split-KV decode: the matrix-core kernel, the row kernel for one q head per
// kv head, and the all-VALU kernel (only pkv_paged_decode_attn_valu, the
// measured alternative of the matrix-core choice); all honour the same contract.
hipError_t launch_paged_decode_valu(const DecodeParams &p, hipStream_t stream);
hipError_t launch_paged_decode_mfma(const DecodeParams &p, hipStream_t stream);
// One q head per kv head: the kernel that reads whole token rows (512 / D heads
// per workgroup), when Hkv is a multiple of 512 / D.
bool paged_decode_rows_applies(const DecodeParams &p);
hipError_t launch_paged_decode_rows(const DecodeParams &p, hipStream_t stream);
// The decode attention behind every decode entry point: the row kernel where
// it applies, the matrix-core kernel otherwise.
hipError_t launch_paged_decode(const DecodeParams &p, hipStream_t stream);

hipError_t launch_decode_merge(const float *o_partial, const float *lse_partial, int rows, int D,
                               int num_splits, uint16_t *out, float *lse_out, hipStream_t stream);

}  // namespace pkv
