// Device helpers shared by the gfx950 kernels of libpkv (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 -> fp32 is exact: a bf16 is the top half of a binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4 &v, float f[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Rotary embedding of one 32-bit word holding the pair (x[2i], x[2i+1]) of
// bf16 values (x[2i] in the low half): the pair is the complex number
// x[2i] + i x[2i+1], multiplied by c + i s.  Each product and the
// sum/difference is one fp32 operation (contraction off, so the bits do not
// depend on FMA formation), then each half rounds once to bf16 (RNE).
__device__ __forceinline__ uint32_t rope_pair(uint32_t w, float c, float s) {
#pragma clang fp contract(off)
  const float x0 = bf16_lo(w), x1 = bf16_hi(w);
  const float a = x0 * c, b = x1 * s, e = x0 * s, f = x1 * c;
  return f32_to_bf16_rne(a - b) | (f32_to_bf16_rne(e + f) << 16);
}

// 2^x on the hardware transcendental unit (v_exp_f32): 2^-inf = 0, 2^0 = 1.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Longest-first order of the (sequence, split) pairs of a decode launch: the
// workgroups of pair rank r (r-th longest; equal lengths in index order) come
// r-th in the grid.  Every workgroup ranks all n <= 4 * blockDim.x pairs
// (thread i the pairs i, i + blockDim.x, ...) in LDS and returns the pair
// whose rank is `target` (pair index i = b + B * s) and its length.  Key of
// pair i: length * 2048 + (2047 - i) (unique, ordered as length then lower
// index; lengths < 2^21, checked on the host), compared four at a time;
// padding keys are 0, below every pair's.
// sm_key: 4 * blockDim.x unsigned, 16-byte aligned.
__device__ __forceinline__ int2 pick_longest_first(const int32_t *seq_lens, int B, int num_splits,
                                                   int chunk, int max_len, int target,
                                                   unsigned *sm_key, int *sm_pick) {
  const int n = B * num_splits;
  const int nt = blockDim.x;
  unsigned key[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = threadIdx.x + u * nt;
    key[u] = 0u;
    if (i < n) {
      const int Li = min(max(seq_lens[i % B], 0), max_len);
      const int len = max(0, min(chunk, Li - (i / B) * chunk));
      key[u] = unsigned(len) * 2048u + unsigned(2047 - i);
    }
    sm_key[i] = key[u];
  }
  __syncthreads();
  const int nq = (n + 3) / 4;
  const uint4 *k4 = reinterpret_cast<const uint4 *>(sm_key);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = threadIdx.x + u * nt;
    if (i < n) {
      int r = 0;
      for (int j = 0; j < nq; ++j) {
        const uint4 k = k4[j];
        r += (k.x > key[u]) + (k.y > key[u]) + (k.z > key[u]) + (k.w > key[u]);
      }
      if (r == target) *sm_pick = i;
    }
  }
  __syncthreads();
  const int pick = *sm_pick;
  return make_int2(pick, int(sm_key[pick] >> 11));
}

}  // namespace pkv
