// The exported C ABI of libpkv.so (declared in include/pkv.h): argument
// validation on the host, then one launch per kernel on the caller's stream.
// Nothing here allocates, frees or synchronises.
#include <math.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "pkv.h"
#include "pkv_launch.h"
#include "pkv_prefill_launch.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2_exact(int64_t x) {
  int k = 0;
  while ((int64_t(1) << k) < x) ++k;
  return k;
}
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest copy unit (16, 8, 4, 2 or 1 bytes) dividing every address and length.
int copy_unit(std::initializer_list<uint64_t> vals) {
  for (int u = 16; u > 1; u >>= 1) {
    bool ok = true;
    for (uint64_t v : vals) ok = ok && (v % uint64_t(u) == 0);
    if (ok) return u;
  }
  return 1;
}

constexpr int kMaxSplits = 1024;
// (sequence, split) pairs the decode kernels rank longest first: every
// workgroup ranks all of them, one pair per thread of its 256.  (With a rank
// taken by comparing every pair's key with every other, 512 pairs, the ragged
// batch at 8 splits, cost more than the finer split saved: 251 against 194 us.)
constexpr int64_t kMaxRankedPairs = 256;


// Validates the arguments shared by both attention entry points and fills the
// launch parameters; PKV_OK with p.B == 0 means "nothing to launch".
pkv_status attention_params(const void *q, const void *k_pool, const void *v_pool,
                            const int32_t *page_table, const int32_t *seq_lens, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                            int32_t num_pages, int32_t max_pages_per_seq, int32_t max_seq_len,
                            int32_t num_splits, float scale, float *o_partial,
                            float *lse_partial, pkv::DecodeParams &p,
                            bool need_partials = true) {
  if (B < 0 || Hq < 1 || Hkv < 1 || num_pages < 1 || max_pages_per_seq < 1 || max_seq_len < 0 ||
      num_splits < 1 || num_splits > kMaxSplits)
    return PKV_ERR_SHAPE;
  if (Hq % Hkv) return PKV_ERR_SHAPE;
  const int G = Hq / Hkv;
  if (D != 64 && D != 128) return PKV_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PKV_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size > 1024) return PKV_ERR_UNSUPPORTED;
  if (int64_t(max_seq_len) > int64_t(max_pages_per_seq) * page_size) return PKV_ERR_SHAPE;
  if (B > 65535 || Hkv > 65535) return PKV_ERR_SHAPE;
  if (int64_t(num_splits) * Hkv * B > int64_t(INT32_MAX)) return PKV_ERR_SHAPE;   // grid size
  if (int64_t(num_pages) * page_size > (int64_t(1) << 31)) return PKV_ERR_SHAPE;
  if (int64_t(max_pages_per_seq) * page_size > (int64_t(1) << 30)) return PKV_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return PKV_ERR_SHAPE;
  p = pkv::DecodeParams{};
  p.B = B;
  if (B == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens) return PKV_ERR_NULL;
  if (need_partials && (!o_partial || !lse_partial)) return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return PKV_ERR_ALIGN;
  p.q = static_cast<const uint16_t *>(q);
  p.k_pool = static_cast<const uint16_t *>(k_pool);
  p.v_pool = static_cast<const uint16_t *>(v_pool);
  p.page_table = page_table;
  p.seq_lens = seq_lens;
  p.o_partial = o_partial;
  p.lse_partial = lse_partial;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.G = G;
  p.page_log2 = log2_exact(page_size);
  p.num_pages = num_pages;
  p.max_pages = max_pages_per_seq;
  p.num_splits = num_splits;
  p.chunk = max_seq_len == 0 ? page_size : pkv_split_chunk(max_seq_len, num_splits, page_size);
  // few (sequence, split) pairs and several splits: the kernel ranks the pairs
  // by length (one per thread of a workgroup) and runs them longest first
  p.longest_first = num_splits > 1 && int64_t(B) * num_splits <= kMaxRankedPairs && p.chunk < (1 << 21);
  p.scale_log2 = scale * 1.4426950408889634f;
  return PKV_OK;
}

// fp32 cos/sin tables of rope_rows rows of D/2 values, 16-byte aligned
pkv_status rope_table_check(const float *rope_cos, const float *rope_sin, int32_t rope_rows) {
  if (rope_rows < 1) return PKV_ERR_SHAPE;
  if (!rope_cos || !rope_sin) return PKV_ERR_NULL;
  if (!aligned16(rope_cos) || !aligned16(rope_sin)) return PKV_ERR_ALIGN;
  return PKV_OK;
}

// Split partials of pkv_paged_decode_attn_merged_static, for callers that
// cannot allocate: one copy of this array per GPU, alive until the process
// ends.  Host code never uses the array's name as an address (on the host it
// is a stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device, on that entry point's first call there.
constexpr int64_t kScratchFloats = int64_t(4) << 20;   // 16 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
float *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this GPU's scratch (the GPU current on the calling thread).
hipError_t scratch_of_current_device(float **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void *a = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? static_cast<float *>(a) : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  if (!g_scratch_ptr[dev]) return hipErrorInvalidSymbol;
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// The attention and, with several splits, the merge of the partials p points
// to; out and lse_out already validated.
pkv_status launch_merged(pkv::DecodeParams &p, void *out, float *lse_out, hipStream_t s) {
  if (p.num_splits == 1) {
    p.out = static_cast<uint16_t *>(out);
    p.lse_out = lse_out;
    p.o_partial = nullptr;
    p.lse_partial = nullptr;
    return pkv::launch_paged_decode(p, s) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
  }
  if (pkv::launch_paged_decode(p, s) != hipSuccess) return PKV_ERR_HIP;
  const hipError_t e = pkv::launch_decode_merge(p.o_partial, p.lse_partial, p.B * p.Hq, p.D,
                                                p.num_splits, static_cast<uint16_t *>(out),
                                                lse_out, s);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

extern "C" {

const char *pkv_status_str(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "pkv: a required pointer is NULL";
    case PKV_ERR_SHAPE: return "pkv: a size is out of range or inconsistent";
    case PKV_ERR_UNSUPPORTED: return "pkv: head_dim, group size or page size not supported";
    case PKV_ERR_ALIGN: return "pkv: a base pointer or stride is not 16-byte aligned";
    case PKV_ERR_HIP: return "pkv: HIP launch failed";
    case PKV_ERR_SCRATCH:
      return "pkv: the split partials exceed the 16 MiB static scratch buffer "
             "(B * Hq * num_splits * (D + 1) floats, plus alignment)";
    default: return "pkv: unknown status";
  }
}

int32_t pkv_split_chunk(int32_t max_seq_len, int32_t num_splits, int32_t page_size) {
  if (max_seq_len < 0 || num_splits < 1 || !is_pow2(page_size)) return PKV_ERR_SHAPE;
  if (max_seq_len == 0) return 0;
  const int64_t per = ceil_div(max_seq_len, num_splits);
  return int32_t(ceil_div(per, page_size) * page_size);
}

int32_t pkv_prefill_plan(const int32_t *q_lens, int32_t B, int32_t *qo_indptr,
                         int32_t *q_tile_to_batch, int32_t *q_tile_to_index, int32_t capacity) {
  if (B < 0 || capacity < 0) return PKV_ERR_SHAPE;
  if (B > 0 && (!q_lens || !qo_indptr)) return PKV_ERR_NULL;
  int64_t total = 0, tiles = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (q_lens[b] < 0) return PKV_ERR_SHAPE;
    total += q_lens[b];
    tiles += ceil_div(q_lens[b], PKV_PREFILL_TILE_ROWS);
  }
  if (total > INT32_MAX || tiles > INT32_MAX) return PKV_ERR_SHAPE;
  if (!q_tile_to_batch || !q_tile_to_index) return int32_t(tiles);   // size query
  if (tiles > capacity) return PKV_ERR_SHAPE;
  int32_t off = 0, t = 0;
  if (qo_indptr) qo_indptr[0] = 0;
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t i = 0; i * PKV_PREFILL_TILE_ROWS < q_lens[b]; ++i, ++t) {
      q_tile_to_batch[t] = b;
      q_tile_to_index[t] = i;
    }
    off += q_lens[b];
    qo_indptr[b + 1] = off;
  }
  return t;
}

int32_t pkv_num_splits_batch(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_seq_len,
                             int64_t total_tokens, int32_t page_size, int32_t num_cus) {
  if (B < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv || max_seq_len < 0 || !is_pow2(page_size) ||
      num_cus < 1)
    return PKV_ERR_SHAPE;
  // workgroups per split: one per (sequence, kv head), or with one q head per
  // kv head one per (sequence, block of 512 / D kv heads): 8 heads at D = 64,
  // 4 at D = 128 (D is not an argument: counted as 8, which errs towards more
  // splits)
  const int64_t hb = Hq == Hkv ? (Hkv % 8 == 0 ? 8 : (Hkv % 4 == 0 ? 4 : 1)) : 1;
  const int64_t streams = int64_t(B) * Hkv / hb;
  const int64_t wg_per_cu = Hq / Hkv >= 8 ? 2 : 1;   // workgroups that keep one CU busy
  int64_t s = ceil_div(wg_per_cu * num_cus, streams);
  const bool uniform = total_tokens >= 0 && total_tokens * 10 >= int64_t(B) * max_seq_len * 9;
  if (!uniform) {
    const int64_t s_bal = ceil_div(max_seq_len, 2048);
    if (s_bal > s) s = s_bal;
  }
  int64_t cap = ceil_div(max_seq_len, 256);
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s > kMaxSplits) s = kMaxSplits;
  return int32_t(s < 1 ? 1 : s);
}

int32_t pkv_num_splits(int32_t B, int32_t Hkv, int32_t max_seq_len, int32_t page_size,
                       int32_t num_cus) {
  // group size and token count unknown: one workgroup per (sequence, kv head)
  // and split, lengths ragged
  if (B < 1 || Hkv < 1 || max_seq_len < 0 || !is_pow2(page_size) || num_cus < 1) return PKV_ERR_SHAPE;
  int64_t s = ceil_div(num_cus, int64_t(B) * Hkv);
  const int64_t s_bal = ceil_div(max_seq_len, 2048);
  if (s_bal > s) s = s_bal;
  int64_t cap = ceil_div(max_seq_len, 256);
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s > kMaxSplits) s = kMaxSplits;
  return int32_t(s < 1 ? 1 : s);
}

pkv_status pkv_kv_store(void *k_pool, void *v_pool, int64_t num_slots, int64_t pool_row_stride,
                        const void *k_new, const void *v_new, int64_t in_row_stride,
                        const int32_t *slot_mapping, int64_t n, int64_t row_elems,
                        int32_t elem_bytes, void *stream) {
  if (n < 0 || num_slots < 0 || row_elems < 0) return PKV_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return PKV_ERR_UNSUPPORTED;
  if (n == 0 || row_elems == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PKV_ERR_NULL;
  if (row_elems > pool_row_stride || row_elems > in_row_stride) return PKV_ERR_SHAPE;
  const int64_t row_b = row_elems * elem_bytes;
  const int64_t pool_stride_b = pool_row_stride * elem_bytes;
  const int64_t in_stride_b = in_row_stride * elem_bytes;
  if (num_slots > (int64_t(1) << 31) || n > (int64_t(1) << 40)) return PKV_ERR_SHAPE;
  const int unit = copy_unit({uint64_t(row_b), uint64_t(pool_stride_b), uint64_t(in_stride_b),
                              reinterpret_cast<uintptr_t>(k_pool), reinterpret_cast<uintptr_t>(v_pool),
                              reinterpret_cast<uintptr_t>(k_new), reinterpret_cast<uintptr_t>(v_new)});
  hipError_t e = pkv::launch_kv_store(k_pool, v_pool, num_slots, pool_stride_b, k_new, v_new,
                                      in_stride_b, slot_mapping, n, row_b, unit,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_kv_store_rope(void *k_pool, void *v_pool, int64_t num_slots,
                             int64_t pool_row_stride, const void *k_new, const void *v_new,
                             int64_t in_row_stride, const int32_t *slot_mapping, int64_t n,
                             int32_t Hkv, int32_t D, const int32_t *positions,
                             const float *rope_cos, const float *rope_sin, int32_t rope_rows,
                             void *stream) {
  if (n < 0 || num_slots < 0 || Hkv < 1 || D < 8 || D % 8) return PKV_ERR_SHAPE;
  const int64_t row_elems = int64_t(Hkv) * D;
  if (row_elems > pool_row_stride || row_elems > in_row_stride) return PKV_ERR_SHAPE;
  if (num_slots > (int64_t(1) << 31) || n > (int64_t(1) << 40)) return PKV_ERR_SHAPE;
  const pkv_status st = rope_table_check(rope_cos, rope_sin, rope_rows);
  if (st != PKV_OK) return st;
  if (n == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping || !positions) return PKV_ERR_NULL;
  if (copy_unit({uint64_t(pool_row_stride * 2), uint64_t(in_row_stride * 2),
                 reinterpret_cast<uintptr_t>(k_pool), reinterpret_cast<uintptr_t>(v_pool),
                 reinterpret_cast<uintptr_t>(k_new), reinterpret_cast<uintptr_t>(v_new)}) != 16)
    return PKV_ERR_ALIGN;
  hipError_t e = pkv::launch_kv_store_rope(k_pool, v_pool, num_slots, pool_row_stride * 2, k_new,
                                           v_new, in_row_stride * 2, slot_mapping, n, Hkv, D,
                                           positions, rope_cos, rope_sin, rope_rows,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_indexing(void *out, const void *weight, int64_t length, int64_t row_elems,
                        int32_t elem_bytes, const int32_t *ids, int64_t n, int64_t start,
                        void *stream) {
  if (n < 0 || length < 0 || row_elems < 0) return PKV_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return PKV_ERR_UNSUPPORTED;
  if (n == 0 || row_elems == 0) return PKV_OK;
  if (!out || !ids || (length > 0 && !weight)) return PKV_ERR_NULL;
  if (length > (int64_t(1) << 40) || n > (int64_t(1) << 40)) return PKV_ERR_SHAPE;
  const int64_t row_b = row_elems * elem_bytes;
  const int unit = copy_unit({uint64_t(row_b), reinterpret_cast<uintptr_t>(out),
                              reinterpret_cast<uintptr_t>(weight)});
  hipError_t e = pkv::launch_gather_rows(out, weight, length, ids, n, start, row_b, unit,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}


pkv_status pkv_paged_decode_attn(const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *page_table, const int32_t *seq_lens, int32_t B,
                                 int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                                 int32_t num_pages, int32_t max_pages_per_seq,
                                 int32_t max_seq_len, int32_t num_splits, float scale,
                                 float *o_partial, float *lse_partial, void *stream) {
  pkv::DecodeParams p;
  const pkv_status st = attention_params(q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D,
                                         page_size, num_pages, max_pages_per_seq, max_seq_len,
                                         num_splits, scale, o_partial, lse_partial, p);
  if (st != PKV_OK || p.B == 0) return st;
  hipError_t e = pkv::launch_paged_decode(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_paged_decode_attn_valu(const void *q, const void *k_pool, const void *v_pool,
                                      const int32_t *page_table, const int32_t *seq_lens,
                                      int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                      int32_t page_size, int32_t num_pages,
                                      int32_t max_pages_per_seq, int32_t max_seq_len,
                                      int32_t num_splits, float scale, float *o_partial,
                                      float *lse_partial, void *stream) {
  pkv::DecodeParams p;
  const pkv_status st = attention_params(q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D,
                                         page_size, num_pages, max_pages_per_seq, max_seq_len,
                                         num_splits, scale, o_partial, lse_partial, p);
  if (st != PKV_OK || p.B == 0) return st;
  if (num_splits > 65535) return PKV_ERR_SHAPE;   // grid (splits, kv heads, sequences)
  hipError_t e = pkv::launch_paged_decode_valu(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_paged_decode_attn_rope(const void *q, const void *k_pool, const void *v_pool,
                                      const int32_t *page_table, const int32_t *seq_lens,
                                      int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                      int32_t page_size, int32_t num_pages,
                                      int32_t max_pages_per_seq, int32_t max_seq_len,
                                      int32_t num_splits, float scale, float *o_partial,
                                      float *lse_partial, const int32_t *q_positions,
                                      const float *rope_cos, const float *rope_sin,
                                      int32_t rope_rows, void *stream) {
  pkv::DecodeParams p;
  pkv_status st = attention_params(q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D,
                                   page_size, num_pages, max_pages_per_seq, max_seq_len,
                                   num_splits, scale, o_partial, lse_partial, p);
  if (st != PKV_OK) return st;
  st = rope_table_check(rope_cos, rope_sin, rope_rows);
  if (st != PKV_OK) return st;
  if (p.B == 0) return PKV_OK;
  if (!q_positions) return PKV_ERR_NULL;
  p.q_pos = q_positions;
  p.rope_cos = rope_cos;
  p.rope_sin = rope_sin;
  p.rope_rows = rope_rows;
  hipError_t e = pkv::launch_paged_decode(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_paged_prefill_attn(const void *q, const void *k_pool, const void *v_pool,
                                  const int32_t *page_table, const int32_t *kv_lens,
                                  const int32_t *qo_indptr, const int32_t *q_tile_to_batch,
                                  const int32_t *q_tile_to_index, int32_t num_q_tiles,
                                  int32_t total_q, int32_t B,
                                  int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                                  int32_t num_pages, int32_t max_pages_per_seq, int32_t causal,
                                  float scale, void *out, float *lse, void *stream) {
  if (B < 0 || num_q_tiles < 0 || total_q < 0 || Hq < 1 || Hkv < 1 || num_pages < 1 ||
      max_pages_per_seq < 1)
    return PKV_ERR_SHAPE;
  if (Hq % Hkv) return PKV_ERR_SHAPE;
  const int G = Hq / Hkv;
  if (D != 64 && D != 128) return PKV_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PKV_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size > 1024) return PKV_ERR_UNSUPPORTED;
  // one workgroup per (q tile, row chunk <= 4, kv head, head half <= 2)
  if (B > 65535 || Hkv > 65535 || int64_t(num_q_tiles) * 4 * Hkv * 2 > int64_t(INT32_MAX))
    return PKV_ERR_SHAPE;
  if (int64_t(num_pages) * page_size > (int64_t(1) << 31)) return PKV_ERR_SHAPE;
  if (int64_t(max_pages_per_seq) * page_size > (int64_t(1) << 30)) return PKV_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return PKV_ERR_SHAPE;
  if (B == 0 || num_q_tiles == 0 || total_q == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !page_table || !kv_lens || !qo_indptr || !q_tile_to_batch ||
      !q_tile_to_index || !out)
    return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      (reinterpret_cast<uintptr_t>(out) & 7u))
    return PKV_ERR_ALIGN;
  pkv::PrefillParams p;
  p.q = static_cast<const uint16_t *>(q);
  p.k_pool = static_cast<const uint16_t *>(k_pool);
  p.v_pool = static_cast<const uint16_t *>(v_pool);
  p.page_table = page_table;
  p.kv_lens = kv_lens;
  p.qo_indptr = qo_indptr;
  p.tile_to_batch = q_tile_to_batch;
  p.tile_to_index = q_tile_to_index;
  p.out = static_cast<uint16_t *>(out);
  p.lse = lse;
  p.num_q_tiles = num_q_tiles;
  p.total_q = total_q;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.G = G;
  p.page_log2 = log2_exact(page_size);
  p.num_pages = num_pages;
  p.max_pages = max_pages_per_seq;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = pkv::launch_paged_prefill(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_paged_decode_attn_merged(const void *q, const void *k_pool, const void *v_pool,
                                        const int32_t *page_table, const int32_t *seq_lens,
                                        int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t page_size, int32_t num_pages,
                                        int32_t max_pages_per_seq, int32_t max_seq_len,
                                        int32_t num_splits, float scale, float *o_partial,
                                        float *lse_partial, void *out, float *lse_out,
                                        void *stream) {
  pkv::DecodeParams p;
  const bool one = num_splits == 1;
  pkv_status st = attention_params(q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D,
                                   page_size, num_pages, max_pages_per_seq, max_seq_len,
                                   num_splits, scale, o_partial, lse_partial, p, !one);
  if (st != PKV_OK || p.B == 0) return st;
  if (!out) return PKV_ERR_NULL;
  if (!aligned16(out)) return PKV_ERR_ALIGN;
  if (int64_t(B) * Hq > (int64_t(1) << 30)) return PKV_ERR_SHAPE;
  if (!one && !aligned16(o_partial)) return PKV_ERR_ALIGN;
  return launch_merged(p, out, lse_out, static_cast<hipStream_t>(stream));
}

pkv_status pkv_paged_decode_attn_merged_static(const void *q, const void *k_pool,
                                               const void *v_pool, const int32_t *page_table,
                                               const int32_t *seq_lens, int32_t B, int32_t Hq,
                                               int32_t Hkv, int32_t D, int32_t page_size,
                                               int32_t num_pages, int32_t max_pages_per_seq,
                                               int32_t max_seq_len, int32_t num_splits,
                                               float scale, void *out, float *lse_out,
                                               void *stream) {
  pkv::DecodeParams p;
  pkv_status st = attention_params(q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D,
                                   page_size, num_pages, max_pages_per_seq, max_seq_len,
                                   num_splits, scale, nullptr, nullptr, p, false);
  if (st != PKV_OK || p.B == 0) return st;
  if (!out) return PKV_ERR_NULL;
  if (!aligned16(out)) return PKV_ERR_ALIGN;
  if (int64_t(B) * Hq > (int64_t(1) << 30)) return PKV_ERR_SHAPE;
  if (num_splits > 1) {
    // o [B, Hq, S, D] from the start of the array, lse [B, Hq, S] from the next
    // 256-byte boundary after it
    const int64_t rows = int64_t(B) * Hq * num_splits;
    const int64_t lse_off = (rows * D + 63) / 64 * 64;
    if (lse_off + rows > kScratchFloats) return PKV_ERR_SCRATCH;
    float *base = nullptr;
    if (scratch_of_current_device(&base) != hipSuccess) return PKV_ERR_HIP;
    p.o_partial = base;
    p.lse_partial = base + lse_off;
  }
  return launch_merged(p, out, lse_out, static_cast<hipStream_t>(stream));
}

pkv_status pkv_decode_step(const void *q, const void *k_new, const void *v_new,
                           int64_t new_row_stride, const int32_t *slot_mapping, void *k_pool,
                           void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                           int32_t num_pages, int32_t max_pages_per_seq, int32_t max_seq_len,
                           int32_t num_splits, float scale, float *o_partial, float *lse_partial,
                           void *out, float *lse_out, void *stream) {
  pkv::DecodeParams p;
  const bool one = num_splits == 1;
  pkv_status st = attention_params(q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D,
                                   page_size, num_pages, max_pages_per_seq, max_seq_len,
                                   num_splits, scale, o_partial, lse_partial, p, !one);
  if (st != PKV_OK || p.B == 0) return st;
  if (!out || !k_new || !v_new || !slot_mapping) return PKV_ERR_NULL;
  if (new_row_stride < int64_t(Hkv) * D) return PKV_ERR_SHAPE;
  if (!aligned16(out) || !aligned16(k_new) || !aligned16(v_new) || (new_row_stride * 2) % 16)
    return PKV_ERR_ALIGN;
  if (int64_t(B) * Hq > (int64_t(1) << 30)) return PKV_ERR_SHAPE;
  if (!one && !aligned16(o_partial)) return PKV_ERR_ALIGN;
  p.k_new = static_cast<const uint16_t *>(k_new);
  p.v_new = static_cast<const uint16_t *>(v_new);
  p.new_stride = new_row_stride;
  p.slots = slot_mapping;
  p.num_slots = int64_t(num_pages) * page_size;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (one) {
    p.out = static_cast<uint16_t *>(out);
    p.lse_out = lse_out;
    return pkv::launch_paged_decode(p, s) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
  }
  if (pkv::launch_paged_decode(p, s) != hipSuccess) return PKV_ERR_HIP;
  const hipError_t e = pkv::launch_decode_merge(o_partial, lse_partial, B * Hq, D, num_splits,
                                                static_cast<uint16_t *>(out), lse_out, s);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_decode_merge(const float *o_partial, const float *lse_partial, int32_t B,
                            int32_t Hq, int32_t D, int32_t num_splits, void *out, float *lse_out,
                            void *stream) {
  if (B < 0 || Hq < 1 || num_splits < 1 || num_splits > kMaxSplits) return PKV_ERR_SHAPE;
  if (D != 64 && D != 128) return PKV_ERR_UNSUPPORTED;
  if (int64_t(B) * Hq > (int64_t(1) << 30)) return PKV_ERR_SHAPE;
  if (B == 0) return PKV_OK;
  if (!o_partial || !lse_partial || !out) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(o_partial)) return PKV_ERR_ALIGN;
  hipError_t e = pkv::launch_decode_merge(o_partial, lse_partial, B * Hq, D, num_splits,
                                          static_cast<uint16_t *>(out), lse_out,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
