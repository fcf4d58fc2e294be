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
// r-th in the grid.  Every workgroup ranks the n <= blockDim.x pairs (thread i
// holds pair i = b + B * s; the host caps n) and returns the pair of rank
// `target` and its length.
//
// A pair is full (length = chunk), partial (0 < length < chunk: at most one
// per sequence, the split holding its last position) or empty.  In the order
// above, the full pairs come first, in index order, then the partial pairs by
// key length * 2048 + (2047 - i) (unique, length then lower index), then the
// empty pairs in index order.  A ballot per class and the per-wave counts
// give every full and empty pair its rank directly; a partial pair counts the
// partial keys above its own, compacted in LDS (at most B of them, read four
// at a time, zero-padded: every key is above zero).
// sm: blockDim.x + 3 * (waves) + 2 unsigned, 16-byte aligned (kRankScratch).
template <int kWaves>
constexpr int kRankScratch = kWaves * 64 + 3 * kWaves + 2;

__device__ __forceinline__ int2 pick_longest_first(const int32_t *seq_lens, int B, int num_splits,
                                                   int chunk, int max_len, int target, unsigned *sm) {
  const int n = B * num_splits;
  const int nt = blockDim.x, nw = nt / 64;
  const int i = threadIdx.x, lane = i & 63, wave = i >> 6;
  unsigned *cnt = sm + nt;            // [wave][class]: full, partial, empty
  unsigned *res = sm + nt + 3 * nw;   // the pick and its length
  int len = 0, cls = 3;           // class 3: no pair
  if (i < n) {
    const int Li = min(max(seq_lens[i % B], 0), max_len);
    len = max(0, min(chunk, Li - (i / B) * chunk));
    cls = len == chunk ? 0 : (len > 0 ? 1 : 2);
  }
  const unsigned long long bf = __ballot(cls == 0), bp = __ballot(cls == 1), be = __ballot(cls == 2);
  const unsigned long long mine = cls == 0 ? bf : (cls == 1 ? bp : be);
  const int below = int(__builtin_amdgcn_mbcnt_hi(unsigned(mine >> 32),
                                                  __builtin_amdgcn_mbcnt_lo(unsigned(mine), 0u)));
  if (lane == 0) {
    cnt[3 * wave] = unsigned(__popcll(bf));
    cnt[3 * wave + 1] = unsigned(__popcll(bp));
    cnt[3 * wave + 2] = unsigned(__popcll(be));
  }
  if (i == 0) {   // a valid pair even if no thread matched (cannot happen with n <= blockDim.x)
    res[0] = unsigned(min(target, n - 1));
    res[1] = 0u;
  }
  __syncthreads();
  int nF = 0, nP = 0, off = 0;
  for (int w = 0; w < nw; ++w) {
    nF += int(cnt[3 * w]);
    nP += int(cnt[3 * w + 1]);
    if (w < wave && cls < 3) off += int(cnt[3 * w + cls]);
  }
  const int idx = off + below;    // position within the pair's class, in index order
  const unsigned key = unsigned(len) * 2048u + unsigned(2047 - i);
  if (cls == 1) sm[idx] = key;
  if (i < 3 && nP + i < ((nP + 3) & ~3)) sm[nP + i] = 0u;
  __syncthreads();
  if (cls < 3) {
    int r;
    if (cls == 0) {
      r = idx;
    } else if (cls == 2) {
      r = nF + nP + idx;
    } else {
      r = nF;
      const uint4 *k4 = reinterpret_cast<const uint4 *>(sm);
      for (int q = 0; q < (nP + 3) / 4; ++q) {
        const uint4 k = k4[q];
        r += (k.x > key) + (k.y > key) + (k.z > key) + (k.w > key);
      }
    }
    if (r == target) {
      res[0] = unsigned(i);
      res[1] = unsigned(len);
    }
  }
  __syncthreads();
  return make_int2(int(res[0]), int(res[1]));
}

}  // namespace pkv
