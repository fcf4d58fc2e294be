// Host-side launcher of the paged prefill kernel (internal header; the
// exported C ABI lives in include/pkv.h and validates every argument first).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Arguments of one paged prefill launch, already validated.
struct PrefillParams {
  const uint16_t *q;             // [total_q, Hq, D] bf16
  const uint16_t *k_pool;        // [num_pages, P, Hkv, D] bf16
  const uint16_t *v_pool;
  const int32_t *page_table;     // [B, max_pages]
  const int32_t *kv_lens;        // [B]
  const int32_t *qo_indptr;      // [B + 1]
  const int32_t *tile_to_batch;  // [num_q_tiles]
  const int32_t *tile_to_index;  // [num_q_tiles]
  uint16_t *out;                 // [total_q, Hq, D] bf16
  float *lse;                    // [total_q, Hq] or NULL
  int num_q_tiles, total_q, B, Hq, Hkv, D, G;
  int page_log2, num_pages, max_pages;
  int causal;
  float scale_log2;              // softmax scale * log2(e)
  int interleave;                // set by the launcher: groups of one XCD interleave their q chunks
};

hipError_t launch_paged_prefill(const PrefillParams &p, hipStream_t stream);

}  // namespace pkv
