// Split-KV paged decode attention and the log-sum-exp merge of its partials.
//
// Follows AstrAI "CUDA Kernels": section "Overview" (GQA decode split over the
// KV sequence; the paged variant shares the kernel body and only changes the
// KV source), section "Q Scheduling and KV Addressing" (the paged source turns
// a logical position into a physical address; all q heads of a kv-head group
// are served by one pass over that head's K/V), section "Python Wrappers"
// (scale 1/sqrt(head_dim)).  The merge follows cuDNN frontend "CSA Fused
// Compressor", sections "ratio=128" and "Numerics" (per-chunk softmax state
// merged in one fixed order; fp32 math with a single final bf16 rounding).
//
// One workgroup per (split, kv head, sequence).  Scores are kept in the log2
// domain: q is pre-multiplied by scale*log2(e), so exp is one v_exp_f32.
#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;

// ---------------------------------------------------------------------------
// VALU kernel: 16-byte lanes, D/8 lanes per token, 64/(D/8) tokens per wave
// step.  Every token slot of every wave keeps its own online-softmax state;
// the states are merged through cross-lane shuffles and LDS at the end.
template <int D, int G>
__global__ __launch_bounds__(256) void paged_decode_valu_kernel(DecodeParams p) {
  constexpr int LPT = D / 8;      // lanes per token
  constexpr int TPW = 64 / LPT;   // tokens per wave step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPT, slot = lane / LPT;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int page_mask = (1 << p.page_log2) - 1;

  int L = p.seq_lens[b];
  L = min(max(L, 0), p.max_pages << p.page_log2);
  const int t0 = s * p.chunk;
  const int t1 = min(t0 + p.chunk, L);

  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 w = *reinterpret_cast<const uint4 *>(
        p.q + (size_t(b) * p.Hq + size_t(g) * G + h) * D + sub * 8);
    unpack8(w, qf[h]);
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[h][i] *= p.scale_log2;
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
  }

  const int32_t *pt = p.page_table + size_t(b) * p.max_pages;
  const size_t row_elems = size_t(p.Hkv) * D;
  const uint16_t *kbase = p.k_pool + size_t(g) * D + sub * 8;
  const uint16_t *vbase = p.v_pool + size_t(g) * D + sub * 8;

  for (int tb = t0 + wave * TPW; tb < t1; tb += kWaves * TPW) {
    const int t = tb + slot;
    const bool valid = t < t1;
    bool bad = false;
    float kf[8], vf[8];
    if (valid) {
      int pid = pt[t >> p.page_log2];
      bad = unsigned(pid) >= unsigned(p.num_pages);
      if (bad) pid = 0;
      const size_t r = (size_t(pid) << p.page_log2) + (t & page_mask);
      unpack8(*reinterpret_cast<const uint4 *>(kbase + r * row_elems), kf);
      unpack8(*reinterpret_cast<const uint4 *>(vbase + r * row_elems), vf);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) kf[i] = vf[i] = 0.f;
    }
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaf(qf[h][i], kf[i], a);
      sc[h] = a;
    }
#pragma unroll
    for (int off = LPT / 2; off > 0; off >>= 1)
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] += __shfl_xor(sc[h], off);
    if (valid) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float x = bad ? NAN : sc[h];
        const float mn = fmaxf(m[h], x);
        const float alpha = (m[h] == mn) ? 1.f : fast_exp2(m[h] - mn);
        const float pr = fast_exp2(x - mn);
        l[h] = fmaf(l[h], alpha, pr);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(acc[h][i], alpha, pr * vf[i]);
        m[h] = mn;
      }
    }
  }

  // merge the token slots of this wave (lane bits above the token's lanes)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mw = m[h];
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
    const float f = (m[h] == mw) ? 1.f : fast_exp2(m[h] - mw);
    l[h] *= f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] *= f;
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
      l[h] += __shfl_xor(l[h], off);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] += __shfl_xor(acc[h][i], off);
    }
    m[h] = mw;
  }

  // merge the waves through LDS, in ascending wave order
  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
  __shared__ float sm_acc[kWaves][G][D];
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) sm_acc[wave][h][sub * 8 + i] = acc[h][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wave][h] = m[h];
      sm_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      M = fmaxf(M, sm_m[w][h]);
      nan |= sm_l[w][h] != sm_l[w][h];
    }
    const size_t orow = (size_t(b) * p.Hq + size_t(g) * G + h) * p.num_splits + s;
    // Empty split: no position seen.  A split whose every score was NaN also
    // leaves the running max at -inf (fmaxf drops NaN) but its sum is NaN, and
    // it must come out NaN, so it takes the general path (NaN * 0 stays NaN).
    if (M == -INFINITY && !nan) {
      p.o_partial[orow * D + d] = 0.f;
      if (d == 0) p.lse_partial[orow] = -INFINITY;
      continue;
    }
    float ls = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][h];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      ls = fmaf(sm_l[w][h], f, ls);
      o = fmaf(sm_acc[w][h][d], f, o);
    }
    p.o_partial[orow * D + d] = o / ls;
    if (d == 0) p.lse_partial[orow] = (M + __builtin_amdgcn_logf(ls)) * kLn2;
  }
}

template <int D, int G>
hipError_t launch_valu(const DecodeParams &p, hipStream_t stream) {
  dim3 grid(p.num_splits, p.Hkv, p.B), block(256);
  hipLaunchKernelGGL((paged_decode_valu_kernel<D, G>), grid, block, 0, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge: one wave per (b, h) row, D/64 dims per lane.  Lane s reads split s's
// lse (64 splits per pass), the wave takes their max; then each split's
// weight is broadcast from its lane and the splits are accumulated in
// ascending order (the fixed order of the fp32 sums), with the o loads of
// several splits in flight.
__device__ __forceinline__ float wave_max(float x) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float *__restrict__ o_part,
                                                           const float *__restrict__ lse_part,
                                                           int rows, int S,
                                                           uint16_t *__restrict__ out,
                                                           float *__restrict__ lse_out) {
  constexpr int DPL = D / 64;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float *lp = lse_part + size_t(row) * S;
  float M = -INFINITY;
  bool nan = false;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const float x = s0 + lane < S ? lp[s0 + lane] : -INFINITY;
    nan |= (x != x);
    M = (x > M) ? x : M;
  }
  M = wave_max(M);
  nan = __any(nan);
  float num[DPL], den = 0.f;
#pragma unroll
  for (int j = 0; j < DPL; ++j) num[j] = 0.f;
  if (M != -INFINITY) {
    const float *orow = o_part + size_t(row) * S * D + lane * DPL;
    for (int s0 = 0; s0 < S; s0 += 64) {
      const float x = s0 + lane < S ? lp[s0 + lane] : -INFINITY;
      const float wl = fast_exp2((x - M) * kLog2e);
      const int n = min(64, S - s0);
      int i = 0;
      for (; i + 8 <= n; i += 8) {   // eight splits' loads in flight, then their sums in order
        float ov[8][DPL];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int j = 0; j < DPL; ++j) ov[u][j] = orow[size_t(s0 + i + u) * D + j];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i + u));
          den += w;
#pragma unroll
          for (int j = 0; j < DPL; ++j) num[j] = fmaf(w, ov[u][j], num[j]);
        }
      }
      for (; i < n; ++i) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
        den += w;
#pragma unroll
        for (int j = 0; j < DPL; ++j) num[j] = fmaf(w, orow[size_t(s0 + i) * D + j], num[j]);
      }
    }
  }
  uint32_t bits[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    const float o = nan ? NAN : (M == -INFINITY ? 0.f : num[j] / den);
    bits[j] = f32_to_bf16_rne(o);
  }
  if constexpr (DPL == 2) {
    reinterpret_cast<uint32_t *>(out + size_t(row) * D)[lane] = bits[0] | (bits[1] << 16);
  } else {
    out[size_t(row) * D + lane] = uint16_t(bits[0]);
  }
  if (lse_out && lane == 0)
    lse_out[row] = nan ? NAN : (M == -INFINITY ? -INFINITY : M + __builtin_amdgcn_logf(den) * kLn2);
}

}  // namespace

hipError_t launch_paged_decode_valu(const DecodeParams &p, hipStream_t stream) {
#define PKV_CASE(DD, GG) \
  if (p.D == DD && p.G == GG) return launch_valu<DD, GG>(p, stream);
  PKV_CASE(64, 1) PKV_CASE(64, 2) PKV_CASE(64, 4) PKV_CASE(64, 8)
  PKV_CASE(128, 1) PKV_CASE(128, 2) PKV_CASE(128, 4) PKV_CASE(128, 8)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const float *o_partial, const float *lse_partial, int rows, int D,
                               int num_splits, uint16_t *out, float *lse_out, hipStream_t stream) {
  dim3 grid((rows + 3) / 4), block(256);
  if (D == 64)
    hipLaunchKernelGGL((decode_merge_kernel<64>), grid, block, 0, stream, o_partial, lse_partial,
                       rows, num_splits, out, lse_out);
  else if (D == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), grid, block, 0, stream, o_partial, lse_partial,
                       rows, num_splits, out, lse_out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
