// Split-KV paged decode attention, matrix-core variant for gfx950.
//
// Same contract as the VALU kernel (see pkv_decode.hip and include/pkv.h):
// one workgroup per (split, kv head, sequence), the q heads of the kv-head
// group served by one pass over that head's K/V (AstrAI "CUDA Kernels",
// section "Q Scheduling and KV Addressing"), split-KV partials merged later.
//
// What runs where, per 16-token tile and per wave:
//   QK^T   one v_mfma_f32_16x16x32_bf16 per 32 dims: A = the group's q rows
//          (heads on M, zero-padded to 16), B = K^T (tokens on N).  Each lane
//          loads its 8-dim K slice straight from HBM into the B operand: no
//          conversion and no LDS staging of K.
//   softmax   scores stay in the MFMA output layout (lane = token, register
//          = head); tile max by DPP row rotations within the 16-lane row;
//          exp2 on v_exp_f32 (q scale folded with log2 e).
//   P.V    on the VALU in fp32: a lane owns 8 dims of one token's V row per
//          load, p is broadcast from the score layout through a small LDS
//          slot; the accumulator is rescaled only when a head's max moved.
//   K/V of the next tile are in flight while a tile is computed; page ids
//   are loaded one tile further ahead.
#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kTile = 16;  // tokens per tile = N of one 16x16x32 MFMA

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) { return __builtin_bit_cast(bf16x8, v); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// reductions over the 16 lanes of a DPP row (row_ror:8, 4, 2, 1)
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0x128>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x122>(x));
  return fmaxf(x, dpp<0x121>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0x128>(x);
  x += dpp<0x124>(x);
  x += dpp<0x122>(x);
  return x + dpp<0x121>(x);
}

// Orders this wave's LDS writes before its following LDS reads (the LDS
// executes one wave's operations in order; this stops the compiler moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int D, int G, bool kPageTile>
__global__ __launch_bounds__(kWaves * 64) void paged_decode_mfma_kernel(DecodeParams p) {
  constexpr int KS = D / 32;      // MFMA k-steps per tile = V loads per lane per tile
  constexpr int LPV = D / 8;      // lanes per token in the V layout
  constexpr int TPV = 64 / LPV;   // tokens per V load instruction
  static_assert(TPV * KS == kTile, "tile shape");
  constexpr int HG = (G + 3) / 4; // 16-lane rows that hold real heads in the score layout

  __shared__ float4 sm_p[kWaves][HG][kTile];
  __shared__ float4 sm_alpha[kWaves][HG];
  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
  __shared__ float sm_acc[kWaves][G][D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int log2P = p.page_log2;
  const int pmask = (1 << log2P) - 1;

  int L = p.seq_lens[b];
  L = min(max(L, 0), p.max_pages << log2P);
  const int t0 = s * p.chunk;
  const int t1 = min(t0 + p.chunk, L);
  const int ntiles = t1 > t0 ? (t1 - t0 + kTile - 1) / kTile : 0;
  const int my_tiles = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;

  // q rows of the group as the MFMA A operand: lane = head (lane & 15), dims 32j + 8(lane >> 4)
  const int qh = lane & 15, qk = lane >> 4;
  bf16x8 qa[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (qh < G)
      w = *reinterpret_cast<const uint4 *>(p.q + (size_t(b) * p.Hq + size_t(g) * G + qh) * D + 32 * j + 8 * qk);
    qa[j] = as_bf16x8(w);
  }

  float m[4], ls[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    ls[r] = 0.f;
  }
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;

  const int32_t *pt = p.page_table + size_t(b) * p.max_pages;
  const size_t row_stride = size_t(p.Hkv) * D;
  const uint16_t *kbase = p.k_pool + size_t(g) * D + 8 * qk;
  const uint16_t *vbase = p.v_pool + size_t(g) * D + 8 * (lane % LPV);
  const int vt = lane / LPV;
  const int last = t1 - 1;

  struct Pids { int k; int v[KS]; };
  struct Regs { uint4 k[KS]; uint4 v[KS]; };

  auto tile_base = [&](int k) { return t0 + kTile * (wave + kWaves * k); };

  auto load_pids = [&](int k, Pids &pi) {
    const int tb = tile_base(k);
    pi.k = pt[min(tb + (lane & 15), last) >> log2P];
    if constexpr (!kPageTile) {
#pragma unroll
      for (int i = 0; i < KS; ++i) pi.v[i] = pt[min(tb + TPV * i + vt, last) >> log2P];
    }
  };

  auto load_kv = [&](int k, const Pids &pi, Regs &rg) {
    const int tb = tile_base(k);
    {
      const int pid = unsigned(pi.k) < unsigned(p.num_pages) ? pi.k : 0;
      const size_t row = (size_t(pid) << log2P) + (min(tb + (lane & 15), last) & pmask);
      const uint4 *kp = reinterpret_cast<const uint4 *>(kbase + row * row_stride);
#pragma unroll
      for (int j = 0; j < KS; ++j) rg.k[j] = kp[4 * j];
    }
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int raw = kPageTile ? pi.k : pi.v[i];
      const int pid = unsigned(raw) < unsigned(p.num_pages) ? raw : 0;
      const size_t row = (size_t(pid) << log2P) + (min(tb + TPV * i + vt, last) & pmask);
      rg.v[i] = *reinterpret_cast<const uint4 *>(vbase + row * row_stride);
    }
  };

  auto compute = [&](int k, const Pids &pi, const Regs &rg) {
    const int tb = tile_base(k);
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], as_bf16x8(rg.k[j]), c, 0, 0, 0);
    // this lane: token tb + (lane & 15), heads 4 * (lane >> 4) + r
    const bool valid = tb + (lane & 15) < t1;
    const bool bad = unsigned(pi.k) >= unsigned(p.num_pages);
    float alpha[4], pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = !valid ? -INFINITY : (bad ? NAN : c[r] * p.scale_log2);
      const float mn = fmaxf(m[r], row_max16(x));
      alpha[r] = (m[r] == mn) ? 1.f : fast_exp2(m[r] - mn);
      pr[r] = fast_exp2(x - mn);
      ls[r] = fmaf(ls[r], alpha[r], pr[r]);
      m[r] = mn;
    }
    // hand p (and the rescale factors) over to the V layout
    wave_lds_sync();
    if (lane < 16 * HG) {
      sm_p[wave][lane >> 4][lane & 15] = make_float4(pr[0], pr[1], pr[2], pr[3]);
      if ((lane & 15) == 0) sm_alpha[wave][lane >> 4] = make_float4(alpha[0], alpha[1], alpha[2], alpha[3]);
    }
    wave_lds_sync();
    float al[HG * 4];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      const float4 a = sm_alpha[wave][hg];
      al[4 * hg] = a.x; al[4 * hg + 1] = a.y; al[4 * hg + 2] = a.z; al[4 * hg + 3] = a.w;
    }
    bool moved = false;
#pragma unroll
    for (int h = 0; h < G; ++h) moved |= (al[h] != 1.f);
    if (moved) {   // wave-uniform: every lane read the same factors
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[h][d] *= al[h];
    }
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      float ph[HG * 4];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const float4 q4 = sm_p[wave][hg][TPV * i + vt];
        ph[4 * hg] = q4.x; ph[4 * hg + 1] = q4.y; ph[4 * hg + 2] = q4.z; ph[4 * hg + 3] = q4.w;
      }
      float vf[8];
      unpack8(rg.v[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[h][d] = fmaf(ph[h], vf[d], acc[h][d]);
    }
  };

  if (my_tiles > 0) {
    Pids pa, pb;
    Regs ra, rb;
    load_pids(0, pa);
    load_kv(0, pa, ra);
    if (my_tiles > 1) load_pids(1, pb);
    for (int k = 0; k < my_tiles; k += 2) {
      // tile k is in ra; pids of tile k + 1 are in pb
      if (k + 1 < my_tiles) {
        load_kv(k + 1, pb, rb);
        if (k + 2 < my_tiles) load_pids(k + 2, pa);
      }
      compute(k, pa, ra);
      if (k + 1 < my_tiles) {
        if (k + 2 < my_tiles) {
          load_kv(k + 2, pa, ra);
          if (k + 3 < my_tiles) load_pids(k + 3, pb);
        }
        compute(k + 1, pb, rb);
      }
    }
  }

  // ---- per-wave totals: sums over the score rows and over the V token slots
#pragma unroll
  for (int r = 0; r < 4; ++r) ls[r] = row_sum16(ls[r]);
#pragma unroll
  for (int off = LPV; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] += __shfl_xor(acc[h][d], off);
  if (lane < LPV) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int d = 0; d < 8; ++d) sm_acc[wave][h][8 * lane + d] = acc[h][d];
  }
  if (lane < 16 * HG && (lane & 15) == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * (lane >> 4) + r;
      if (h < G) {
        sm_m[wave][h] = m[r];
        sm_l[wave][h] = ls[r];
      }
    }
  }
  __syncthreads();

  // ---- merge the waves (ascending order) and write this split's partial
  for (int idx = threadIdx.x; idx < G * D; idx += kWaves * 64) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    const size_t orow = (size_t(b) * p.Hq + size_t(g) * G + h) * p.num_splits + s;
    if (M == -INFINITY) {
      p.o_partial[orow * D + d] = 0.f;
      if (d == 0) p.lse_partial[orow] = -INFINITY;
      continue;
    }
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][h];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      l = fmaf(sm_l[w][h], f, l);
      o = fmaf(sm_acc[w][h][d], f, o);
    }
    p.o_partial[orow * D + d] = o / l;
    if (d == 0) p.lse_partial[orow] = (M + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

template <int D, int G>
hipError_t launch_mfma(const DecodeParams &p, hipStream_t stream) {
  const dim3 grid{unsigned(p.num_splits), unsigned(p.Hkv), unsigned(p.B)}, block{kWaves * 64};
  if (p.page_log2 >= 4)
    hipLaunchKernelGGL((paged_decode_mfma_kernel<D, G, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((paged_decode_mfma_kernel<D, G, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode_mfma(const DecodeParams &p, hipStream_t stream) {
#define PKV_CASE(DD, GG) \
  if (p.D == DD && p.G == GG) return launch_mfma<DD, GG>(p, stream);
  PKV_CASE(64, 1) PKV_CASE(64, 2) PKV_CASE(64, 4) PKV_CASE(64, 8)
  PKV_CASE(128, 1) PKV_CASE(128, 2) PKV_CASE(128, 4) PKV_CASE(128, 8)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
