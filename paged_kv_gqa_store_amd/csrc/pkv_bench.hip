// Copy kernels that bound the store on the same GPU (libpkv_bench.so, see
// include/pkv_bench.h): a linear 16-byte copy, and the same rows moved to the
// same destinations one page run per workgroup.  Measurement only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_bench.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_linear_kernel(u32x4 *__restrict__ dst,
                                                          const u32x4 *__restrict__ src,
                                                          int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// 4 units per lane in flight per pool (K and V): 16 KB per workgroup and pass
__global__ __launch_bounds__(256) void copy_runs_kernel(
    u32x4 *__restrict__ kd, u32x4 *__restrict__ vd, int64_t dst_rows, const u32x4 *__restrict__ ks,
    const u32x4 *__restrict__ vs, int64_t src_rows, const int32_t *__restrict__ run_src,
    const int32_t *__restrict__ run_dst, const int32_t *__restrict__ run_len, int64_t n_runs,
    int64_t row_units) {
  for (int64_t r = blockIdx.x; r < n_runs; r += gridDim.x) {
    const int64_t s0 = run_src[r], d0 = run_dst[r], len = run_len[r];
    if (s0 < 0 || d0 < 0 || len < 0 || s0 + len > src_rows || d0 + len > dst_rows) continue;
    const int64_t n = len * row_units;
    const u32x4 *ksr = ks + s0 * row_units, *vsr = vs + s0 * row_units;
    u32x4 *kdr = kd + d0 * row_units, *vdr = vd + d0 * row_units;
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += 256 * 4) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * 256;
        if (i < n) {
          a[u] = __builtin_nontemporal_load(ksr + i);
          b[u] = __builtin_nontemporal_load(vsr + i);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * 256;
        if (i < n) {
          __builtin_nontemporal_store(a[u], kdr + i);
          __builtin_nontemporal_store(b[u], vdr + i);
        }
      }
    }
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int32_t pkvb_copy_linear(void *dst, const void *src, int64_t bytes, void *stream) {
  if (bytes < 0 || bytes % 16) return -2;
  if (bytes == 0) return 0;
  if (!dst || !src) return -1;
  if (!aligned16(dst) || !aligned16(src)) return -4;
  const int64_t n = bytes / 16;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_linear_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4 *>(dst),
                     static_cast<const u32x4 *>(src), n);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int32_t pkvb_copy_page_runs(void *k_dst, void *v_dst, int64_t dst_rows, const void *k_src,
                            const void *v_src, int64_t src_rows, const int32_t *run_src_row,
                            const int32_t *run_dst_slot, const int32_t *run_rows, int64_t n_runs,
                            int64_t row_bytes, void *stream) {
  if (n_runs < 0 || row_bytes <= 0 || row_bytes % 16 || dst_rows < 0 || src_rows < 0) return -2;
  if (n_runs == 0) return 0;
  if (!k_dst || !v_dst || !k_src || !v_src || !run_src_row || !run_dst_slot || !run_rows) return -1;
  if (!aligned16(k_dst) || !aligned16(v_dst) || !aligned16(k_src) || !aligned16(v_src)) return -4;
  const int64_t blocks = n_runs < 65536 ? n_runs : 65536;
  hipLaunchKernelGGL(copy_runs_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4 *>(k_dst),
                     static_cast<u32x4 *>(v_dst), dst_rows, static_cast<const u32x4 *>(k_src),
                     static_cast<const u32x4 *>(v_src), src_rows, run_src_row, run_dst_slot,
                     run_rows, n_runs, row_bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
