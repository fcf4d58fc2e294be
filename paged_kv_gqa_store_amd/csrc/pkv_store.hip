// kv_store: scatter the step's new K/V rows into the page pool by slot index.
//
// Follows the mini-sglang handbook, "Custom CUDA kernels", section "Moving
// whole rows by index": a pure row move, bound by memory bandwidth, copied in
// 16-byte vectors when the row and its strides allow it.  The gfx950 design:
//   - wave64; a row gets 2^k lanes (k chosen on the host so a 2 KB row is one
//     wave and a 128 B row is 8 lanes: several short rows share a wave);
//   - a lane loads the row's slot index together with all of its K and V
//     data (the data loads do not wait for the index), and stores only after
//     the index is known to lie in the pool: each wave keeps
//     2 * units_per_lane 16-byte loads in flight;
//   - rows are read and written exactly once, so both directions carry the
//     non-temporal hint (measured 2-7% faster on gfx950);
//   - a slot outside the pool is skipped, so a bad index cannot fault.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// Native vector types: the non-temporal builtins take no HIP struct vectors.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Copies rows with UNITS (compile-time) copy units per lane, unit type U.
// Row r of the inputs goes to pool row slots[r]; lanes_log2 lanes per row.
template <typename U, int UNITS>
__global__ __launch_bounds__(256) void store_rows_kernel(
    U *__restrict__ k_pool, U *__restrict__ v_pool, int64_t num_slots, int64_t pool_stride,
    const U *__restrict__ k_new, const U *__restrict__ v_new, int64_t in_stride,
    const int32_t *__restrict__ slots, int64_t n, int64_t row_units, int lanes_log2) {
  const int64_t lanes = int64_t(1) << lanes_log2;
  const int64_t rows_per_grid = (int64_t(gridDim.x) * blockDim.x) >> lanes_log2;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t lane = gid & (lanes - 1);
  for (int64_t r = gid >> lanes_log2; r < n; r += rows_per_grid) {
    const int64_t slot = __builtin_nontemporal_load(slots + r);
    const U *ks = k_new + r * in_stride;
    const U *vs = v_new + r * in_stride;
    for (int64_t base = 0; base < row_units; base += UNITS * lanes) {
      U kb[UNITS], vb[UNITS];
#pragma unroll
      for (int u = 0; u < UNITS; ++u) {
        const int64_t i = base + u * lanes + lane;
        if (i < row_units) {
          kb[u] = __builtin_nontemporal_load(ks + i);
          vb[u] = __builtin_nontemporal_load(vs + i);
        }
      }
      if (slot < 0 || slot >= num_slots) continue;
      U *kd = k_pool + slot * pool_stride;
      U *vd = v_pool + slot * pool_stride;
#pragma unroll
      for (int u = 0; u < UNITS; ++u) {
        const int64_t i = base + u * lanes + lane;
        if (i < row_units) {
          __builtin_nontemporal_store(kb[u], kd + i);
          __builtin_nontemporal_store(vb[u], vd + i);
        }
      }
    }
  }
}

// kv_store with rotary embedding (AstrAI "CUDA Kernels", section "Rotary
// Embedding Kernel": fp32 cos/sin of the token's position rotate every
// (head, dimension pair)).  K rows are rotated while they are scattered, so the
// rotated K never makes a separate round trip through memory; V rows are
// copied as by store_rows_kernel.  bf16 rows of heads*D elements moved in
// 16-byte units (4 pairs); a unit's pairs need 4 cos and 4 sin values, read
// as one 16-byte vector each (the table row is shared by the token's heads and
// stays in cache).  A position outside the table writes a NaN K row.
__global__ __launch_bounds__(256) void store_rope_kernel(
    u32x4 *__restrict__ k_pool, u32x4 *__restrict__ v_pool, int64_t num_slots, int64_t pool_stride,
    const u32x4 *__restrict__ k_new, const u32x4 *__restrict__ v_new, int64_t in_stride,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ positions,
    const float *__restrict__ rope_cos, const float *__restrict__ rope_sin, int rope_rows,
    int64_t n, int64_t row_units, int d_units, int lanes_log2) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int64_t lanes = int64_t(1) << lanes_log2;
  const int64_t rows_per_grid = (int64_t(gridDim.x) * blockDim.x) >> lanes_log2;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t lane = gid & (lanes - 1);
  const int half = d_units * 4;                 // D / 2 pairs per head
  for (int64_t r = gid >> lanes_log2; r < n; r += rows_per_grid) {
    const int64_t slot = __builtin_nontemporal_load(slots + r);
    const int pos = __builtin_nontemporal_load(positions + r);
    const bool pos_ok = pos >= 0 && pos < rope_rows;
    const float *cr = rope_cos + int64_t(pos_ok ? pos : 0) * half;
    const float *sr = rope_sin + int64_t(pos_ok ? pos : 0) * half;
    const u32x4 *ks = k_new + r * in_stride;
    const u32x4 *vs = v_new + r * in_stride;
    for (int64_t i = lane; i < row_units; i += lanes) {
      u32x4 kb = __builtin_nontemporal_load(ks + i);
      const u32x4 vb = __builtin_nontemporal_load(vs + i);
      const int p4 = 4 * int(i % d_units);      // first pair of this unit within its head
      const f32x4 c = *reinterpret_cast<const f32x4 *>(cr + p4);
      const f32x4 sn = *reinterpret_cast<const f32x4 *>(sr + p4);
#pragma unroll
      for (int k = 0; k < 4; ++k) kb[k] = pos_ok ? rope_pair(kb[k], c[k], sn[k]) : 0x7fc07fc0u;
      if (slot < 0 || slot >= num_slots) continue;
      __builtin_nontemporal_store(kb, k_pool + slot * pool_stride + i);
      __builtin_nontemporal_store(vb, v_pool + slot * pool_stride + i);
    }
  }
}

// indexing: vocabulary-slice row gather (mini-sglang handbook, "Custom CUDA
// kernels", section "Moving whole rows by index").  Output row r is row
// ids[r] - start of the slice, or zeros when the id lies outside
// [start, start + length).  Same lane layout as the store; the slice rows may
// repeat across tokens, so they are loaded with the default cache policy,
// while the output (written once) is stored non-temporally.
template <typename U, int UNITS>
__global__ __launch_bounds__(256) void gather_rows_kernel(
    U *__restrict__ out, const U *__restrict__ weight, int64_t length,
    const int32_t *__restrict__ ids, int64_t n, int64_t start, int64_t row_units,
    int lanes_log2) {
  const int64_t lanes = int64_t(1) << lanes_log2;
  const int64_t rows_per_grid = (int64_t(gridDim.x) * blockDim.x) >> lanes_log2;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t lane = gid & (lanes - 1);
  for (int64_t r = gid >> lanes_log2; r < n; r += rows_per_grid) {
    const int64_t local = int64_t(__builtin_nontemporal_load(ids + r)) - start;
    const bool valid = local >= 0 && local < length;
    const U *src = weight + (valid ? local : 0) * row_units;
    U *dst = out + r * row_units;
    for (int64_t base = 0; base < row_units; base += UNITS * lanes) {
      U buf[UNITS];
#pragma unroll
      for (int u = 0; u < UNITS; ++u) {
        const int64_t i = base + u * lanes + lane;
        buf[u] = U{};
        if (valid && i < row_units) buf[u] = src[i];
      }
#pragma unroll
      for (int u = 0; u < UNITS; ++u) {
        const int64_t i = base + u * lanes + lane;
        if (i < row_units) __builtin_nontemporal_store(buf[u], dst + i);
      }
    }
  }
}

// lanes per row (a power of two covering the row, at most one wave), copy units
// per lane and grid size for n rows of row_units units
struct RowLaunch {
  int lanes_log2;
  int64_t units_per_lane;
  dim3 grid;
};
RowLaunch plan_rows(int64_t n, int64_t row_units) {
  RowLaunch r;
  r.lanes_log2 = 0;
  while ((int64_t(1) << r.lanes_log2) < row_units && r.lanes_log2 < 6) ++r.lanes_log2;
  const int64_t lanes = int64_t(1) << r.lanes_log2;
  r.units_per_lane = (row_units + lanes - 1) / lanes;
  const int64_t rows_per_block = 256 / lanes;
  int64_t blocks = (n + rows_per_block - 1) / rows_per_block;
  // enough blocks to fill 256 CUs many times over; the grid-stride loop does the rest
  if (blocks > 65536) blocks = 65536;
  r.grid = dim3{unsigned(blocks)};
  return r;
}

template <typename U>
hipError_t launch_gather(void *out, const void *weight, int64_t length, const int32_t *ids,
                         int64_t n, int64_t start, int64_t row_b, hipStream_t stream) {
  const int64_t row_units = row_b / int64_t(sizeof(U));
  const RowLaunch L = plan_rows(n, row_units);
  U *o = static_cast<U *>(out);
  const U *w = static_cast<const U *>(weight);
  if (L.units_per_lane >= 2)
    hipLaunchKernelGGL((gather_rows_kernel<U, 2>), L.grid, dim3{256}, 0, stream, o, w, length, ids,
                       n, start, row_units, L.lanes_log2);
  else
    hipLaunchKernelGGL((gather_rows_kernel<U, 1>), L.grid, dim3{256}, 0, stream, o, w, length, ids,
                       n, start, row_units, L.lanes_log2);
  return hipGetLastError();
}

template <typename U>
hipError_t launch_unit(void *k_pool, void *v_pool, int64_t num_slots, int64_t pool_stride_b,
                       const void *k_new, const void *v_new, int64_t in_stride_b,
                       const int32_t *slots, int64_t n, int64_t row_b, hipStream_t stream) {
  const int64_t row_units = row_b / int64_t(sizeof(U));
  const RowLaunch L = plan_rows(n, row_units);
  const int lanes_log2 = L.lanes_log2;
  const int64_t units_per_lane = L.units_per_lane;
  const dim3 grid = L.grid, block{256};
  U *kp = static_cast<U *>(k_pool);
  U *vp = static_cast<U *>(v_pool);
  const U *kn = static_cast<const U *>(k_new);
  const U *vn = static_cast<const U *>(v_new);
  const int64_t ps = pool_stride_b / int64_t(sizeof(U)), is = in_stride_b / int64_t(sizeof(U));
  if (units_per_lane >= 2)
    hipLaunchKernelGGL((store_rows_kernel<U, 2>), grid, block, 0, stream, kp, vp, num_slots, ps,
                       kn, vn, is, slots, n, row_units, lanes_log2);
  else
    hipLaunchKernelGGL((store_rows_kernel<U, 1>), grid, block, 0, stream, kp, vp, num_slots, ps,
                       kn, vn, is, slots, n, row_units, lanes_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_rows(void *out, const void *weight, int64_t length, const int32_t *ids,
                              int64_t n, int64_t start, int64_t row_b, int unit_b,
                              hipStream_t stream) {
  switch (unit_b) {
    case 16: return launch_gather<u32x4>(out, weight, length, ids, n, start, row_b, stream);
    case 8: return launch_gather<u32x2>(out, weight, length, ids, n, start, row_b, stream);
    case 4: return launch_gather<uint32_t>(out, weight, length, ids, n, start, row_b, stream);
    case 2: return launch_gather<uint16_t>(out, weight, length, ids, n, start, row_b, stream);
    default: return launch_gather<uint8_t>(out, weight, length, ids, n, start, row_b, stream);
  }
}

hipError_t launch_kv_store_rope(void *k_pool, void *v_pool, int64_t num_slots,
                               int64_t pool_stride_b, const void *k_new, const void *v_new,
                               int64_t in_stride_b, const int32_t *slots, int64_t n, int Hkv,
                               int D, const int32_t *positions, const float *rope_cos,
                               const float *rope_sin, int rope_rows, hipStream_t stream) {
  const int64_t row_units = int64_t(Hkv) * D / 8;
  const RowLaunch L = plan_rows(n, row_units);
  hipLaunchKernelGGL(store_rope_kernel, L.grid, dim3{256}, 0, stream,
                     static_cast<u32x4 *>(k_pool), static_cast<u32x4 *>(v_pool), num_slots,
                     pool_stride_b / 16, static_cast<const u32x4 *>(k_new),
                     static_cast<const u32x4 *>(v_new), in_stride_b / 16, slots, positions,
                     rope_cos, rope_sin, rope_rows, n, row_units, D / 8, L.lanes_log2);
  return hipGetLastError();
}

hipError_t launch_kv_store(void *k_pool, void *v_pool, int64_t num_slots, int64_t pool_stride_b,
                           const void *k_new, const void *v_new, int64_t in_stride_b,
                           const int32_t *slots, int64_t n, int64_t row_b, int unit_b,
                           hipStream_t stream) {
  switch (unit_b) {
    case 16: return launch_unit<u32x4>(k_pool, v_pool, num_slots, pool_stride_b, k_new, v_new, in_stride_b, slots, n, row_b, stream);
    case 8: return launch_unit<u32x2>(k_pool, v_pool, num_slots, pool_stride_b, k_new, v_new, in_stride_b, slots, n, row_b, stream);
    case 4: return launch_unit<uint32_t>(k_pool, v_pool, num_slots, pool_stride_b, k_new, v_new, in_stride_b, slots, n, row_b, stream);
    case 2: return launch_unit<uint16_t>(k_pool, v_pool, num_slots, pool_stride_b, k_new, v_new, in_stride_b, slots, n, row_b, stream);
    default: return launch_unit<uint8_t>(k_pool, v_pool, num_slots, pool_stride_b, k_new, v_new, in_stride_b, slots, n, row_b, stream);
  }
}

}  // namespace pkv
