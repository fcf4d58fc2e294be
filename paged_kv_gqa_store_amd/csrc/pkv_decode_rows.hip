// Split-KV paged decode attention for one q head per kv head (multi-head
// attention), reading whole token rows.
//
// Same contract as the matrix-core kernel (include/pkv.h,
// pkv_paged_decode_attn): AstrAI "CUDA Kernels", section "Q Scheduling and
// KV Addressing" (the paged source turns a logical position into a physical
// address), section "Python Wrappers" (scale 1/sqrt(head_dim)); split-KV
// partials merged as in cuDNN frontend "CSA Fused Compressor", "ratio=128".
//
// With one q head per kv head there is no group to share a K/V tile, and a
// workgroup per kv head would gather each token's head slice (128 or 256 B) at
// a random slot while the other heads' workgroups gather the rest of the same
// row at other times.  On gfx950 that pattern sustains ~68% of HBM bandwidth;
// the same bytes read as contiguous 1 KB pieces of each token's row sustain
// ~81%.  So one workgroup serves NH = 512 / D consecutive heads of a sequence:
//   - one wave instruction loads one token's NH head slices (64 lanes x 16 B,
//     lane = 8 dims of one head) from K, one from V; the token is
//     wave-uniform, so its slot (page id staged in LDS) is a scalar and each
//     load is a scalar base plus a constant lane offset;
//   - scores are fp32 dot products on the VALU (q pre-scaled by
//     scale * log2 e), summed over the head's D/8 lanes by DPP;
//   - each wave streams a contiguous range of KS-token tiles through a ring of
//     NBUF register tiles, with one online-softmax update per tile (a lane
//     keeps its head's running max and sum, and 8 accumulators);
//   - the four waves merge through LDS in ascending order and write the
//     split's normalised o and lse (or, with one split, the bf16 output).
// Workgroup order: head block fastest, then sequence, then split; with several
// splits and at most 256 (sequence, split) pairs, the pairs go longest first.
#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSegPagesRows = 2048;   // page ids held in LDS at a time

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the LPH lanes of one head (aligned groups of 8 or 16 lanes):
// quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2), row_half_mirror
// (lane i <-> 7 - i within 8), and for 16 lanes row_ror:8.
template <int LPH>
__device__ __forceinline__ float head_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  if constexpr (LPH == 16) x += dpp_f<0x128>(x);
  return x;
}

template <int D, int NBUF, int kMode>
__global__ __launch_bounds__(256) void paged_decode_rows_kernel(DecodeParams p) {
  constexpr bool kRope = kMode == 1, kFuse = kMode == 2;
  constexpr int kWaves = 4;
  constexpr int NH = 512 / D;   // heads per workgroup: 1 KB of every token's row
  constexpr int LPH = D / 8;    // lanes per head, 8 dims (16 B) each
  constexpr int KS = 8;         // tokens per tile: one K and one V load per token and lane
  static_assert(NH * LPH == 64, "one token per wave instruction");

  __shared__ int sm_pid[kSegPagesRows];
  __shared__ float sm_m[kWaves][NH], sm_l[kWaves][NH];
  __shared__ float sm_acc[kWaves][NH * D];
  [[maybe_unused]] __shared__ u32x4 sm_new[2][64];   // fused store: this head block of the new row

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nhb = p.Hkv / NH;
  const int hb = blockIdx.x % nhb;
  int b, s;
  bool empty_pair = false;
  if (p.longest_first) {
    __shared__ __attribute__((aligned(16))) unsigned sm_key[kRankScratch<kWaves>];
    const int2 pk = pick_longest_first(p.seq_lens, p.B, p.num_splits, p.chunk, p.max_pages << p.page_log2,
                                       blockIdx.x / nhb, sm_key);
    b = pk.x % p.B;
    s = pk.x / p.B;
    empty_pair = pk.y == 0;
  } else {
    b = (blockIdx.x / nhb) % p.B;
    s = blockIdx.x / (nhb * p.B);
  }

  const int h = lane / LPH;                    // head within the block
  auto write_empty = [&]() {
    // an empty split: o = 0, lse = -inf (one split: out = 0, lse_out = -inf)
    for (int idx = threadIdx.x; idx < NH * D; idx += kWaves * 64) {
      const size_t fr = size_t(b) * p.Hq + hb * NH + idx / D;
      const int d = idx % D;
      if (p.out) {
        p.out[fr * D + d] = 0;
        if (d == 0 && p.lse_out) p.lse_out[fr] = -INFINITY;
      } else {
        const size_t orow = fr * p.num_splits + s;
        p.o_partial[orow * D + d] = 0.f;
        if (d == 0) p.lse_partial[orow] = -INFINITY;
      }
    }
  };
  if (empty_pair && (!kFuse || s > 0)) {
    write_empty();   // without any load: in a ragged batch these pairs are many
    return;
  }

  const int log2P = p.page_log2;
  const int pmask = (1 << log2P) - 1;
  const int32_t *pt = p.page_table + size_t(b) * p.max_pages;
  const int t0 = s * p.chunk;
  const int pg0 = t0 >> log2P;
  auto fetch_pids = [&](int pga, int npg) {
    for (int i = threadIdx.x; i < npg; i += kWaves * 64) sm_pid[i] = pt[min(pga + i, p.max_pages - 1)];
  };
  fetch_pids(pg0, min((p.chunk + pmask) >> log2P, kSegPagesRows));

  int L = p.seq_lens[b];
  L = min(max(L, 0), p.max_pages << log2P);
  const int t1 = min(t0 + p.chunk, L);

  // byte offset of this lane's 16 bytes within a token row (and within q's row
  // of the sequence, which has the same [heads, D] layout since Hq == Hkv)
  const int row_bytes = p.Hkv * D * 2;
  const unsigned lane_off = unsigned(hb * NH * D + 8 * lane) * 2u;
  const char *kpool = reinterpret_cast<const char *>(p.k_pool);
  const char *vpool = reinterpret_cast<const char *>(p.v_pool);
  const char *qrow = reinterpret_cast<const char *>(p.q) + size_t(b) * p.Hq * D * 2;

  if constexpr (kFuse) {
    // The step's store, fused (as in the matrix-core kernel): the split
    // holding position L - 1 (split 0 of an empty sequence) copies this head
    // block of the new K / V row to its pool slot, and keeps it in LDS, where
    // the tile holding position L - 1 takes it from (ordered by the barrier
    // that opens the first page-id segment).  A slot outside the pool is not
    // written.
    const int sw = L > 0 ? min((L - 1) / p.chunk, p.num_splits - 1) : 0;
    if (s == sw && wave < 2) {
      const int64_t slot = p.slots[b];
      const uint16_t *src = (wave == 0 ? p.k_new : p.v_new) + size_t(b) * p.new_stride;
      const u32x4 row = ld16(reinterpret_cast<const char *>(src) + lane_off);
      sm_new[wave][lane] = row;
      if (slot >= 0 && slot < p.num_slots) {
        char *dst = const_cast<char *>(wave == 0 ? kpool : vpool) + slot * int64_t(row_bytes) + lane_off;
        *reinterpret_cast<u32x4 *>(dst) = row;
      }
    }
  }

  // this lane's 8 dims of q, as fp32 scaled by scale * log2(e) (rotated first
  // for kMode 1: 4 whole pairs, rounded to bf16 like a separately rotated q)
  float qf[8];
  {
    u32x4 w = ld16(qrow + lane_off);
    if constexpr (kRope) {
      const int pos = p.q_pos[b];
      const bool pos_ok = pos >= 0 && pos < p.rope_rows;
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      const size_t trow = size_t(pos_ok ? pos : 0) * (D / 2) + 4 * (lane % LPH);
      const f32x4 c = *reinterpret_cast<const f32x4 *>(p.rope_cos + trow);
      const f32x4 sn = *reinterpret_cast<const f32x4 *>(p.rope_sin + trow);
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = pos_ok ? rope_pair(w[k], c[k], sn[k]) : 0x7fc07fc0u;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qf[2 * k] = bf16_lo(w[k]) * p.scale_log2;
      qf[2 * k + 1] = bf16_hi(w[k]) * p.scale_log2;
    }
  }

  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = 0.f;

  struct Regs { u32x4 k[KS]; u32x4 v[KS]; unsigned bad; };

  for (int sa = t0; sa < t1;) {
    const int pga = sa >> log2P;
    const int sb = min(t1, (pga + kSegPagesRows) << log2P);
    if (sa != t0) {
      __syncthreads();
      fetch_pids(pga, min(((sb - 1) >> log2P) - pga + 1, kSegPagesRows));
    }
    __syncthreads();

    const int nst = (sb - sa + KS - 1) / KS;
    const int tpw = (nst + kWaves - 1) / kWaves;
    const int first = min(wave * tpw, nst);
    const int my_tiles = min(tpw, nst - first);
    const int last = sb - 1;
    const int tw0 = sa + KS * first;

    // Loads tile k: one token per load, its slot a scalar.  Positions past
    // `last` load `last` again (their scores are masked); a prefetch past the
    // range (real == false) reads q's row instead, an L2 hit, and is never
    // computed.
    auto load_kv = [&](int k, Regs &rg, bool real) {
      const int tb = tw0 + KS * k;
      rg.bad = 0u;
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        const int t = min(tb + i, last);
        const int raw = __builtin_amdgcn_readfirstlane(sm_pid[(t >> log2P) - pga]);
        const bool ok = unsigned(raw) < unsigned(p.num_pages);
        rg.bad |= ok ? 0u : (1u << i);
        const int64_t slot = (int64_t(ok ? raw : 0) << log2P) + (t & pmask);
        const char *kb = real ? kpool + slot * row_bytes : qrow;
        const char *vb = real ? vpool + slot * row_bytes : qrow;
        rg.k[i] = ld16_stream(kb + lane_off);
        rg.v[i] = ld16_stream(vb + lane_off);
      }
    };

    auto compute = [&](int k, Regs rg) {
      const int tb = tw0 + KS * k;
      if constexpr (kFuse) {
        // the tile that reaches position L - 1 (wave-uniform tests) takes it
        // from the new row, also where a load past `last` was clamped onto it
        // (masked, but 0 * NaN would not be 0)
        if (last == L - 1 && tb + KS > last) {
          const u32x4 kn = sm_new[0][lane], vn = sm_new[1][lane];
#pragma unroll
          for (int i = 0; i < KS; ++i)
            if (tb + i >= last) {
              rg.k[i] = kn;
              rg.v[i] = vn;
            }
        }
      }
      float x[KS];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dot = fmaf(qf[2 * j], bf16_lo(rg.k[i][j]), dot);
          dot = fmaf(qf[2 * j + 1], bf16_hi(rg.k[i][j]), dot);
        }
        dot = head_sum<LPH>(dot);
        const bool valid = tb + i <= last;
        x[i] = !valid ? -INFINITY : (((rg.bad >> i) & 1u) ? NAN : dot);
        mt = fmaxf(mt, x[i]);
      }
      const float mn = fmaxf(m, mt);
      const float alpha = (m == mn) ? 1.f : fast_exp2(m - mn);
      float ps = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] *= alpha;
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        const float pr = fast_exp2(x[i] - mn);
        ps += pr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] = fmaf(pr, bf16_lo(rg.v[i][j]), acc[2 * j]);
          acc[2 * j + 1] = fmaf(pr, bf16_hi(rg.v[i][j]), acc[2 * j + 1]);
        }
      }
      l = fmaf(l, alpha, ps);
      m = mn;
    };

    // Ring of NBUF register tiles: whole passes in the steady state, then the
    // remaining (already loaded) tiles.
    if (my_tiles > 0) {
      const int lt = my_tiles - 1;
      Regs rg[NBUF];
#pragma unroll
      for (int j = 0; j < NBUF - 1; ++j) load_kv(min(j, lt), rg[j], j <= lt);
      int k = 0;
      for (; k + NBUF <= my_tiles; k += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          load_kv(min(k + u + NBUF - 1, lt), rg[(u + NBUF - 1) % NBUF], k + u + NBUF - 1 <= lt);
          asm volatile("" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
          compute(k + u, rg[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < NBUF - 1; ++u)
        if (k + u < my_tiles) compute(k + u, rg[u]);
    }
    sa = sb;
  }

  // ---- merge the four waves (ascending order = ascending positions)
  if (lane % LPH == 0) {
    sm_m[wave][h] = m;
    sm_l[wave][h] = l;
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) sm_acc[wave][h * D + 8 * (lane % LPH) + d] = acc[d];
  __syncthreads();
  for (int idx = threadIdx.x; idx < NH * D; idx += kWaves * 64) {
    const int hh = idx / D, d = idx % D;
    float M = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      M = fmaxf(M, sm_m[w][hh]);
      nan |= sm_l[w][hh] != sm_l[w][hh];
    }
    const size_t fr = size_t(b) * p.Hq + hb * NH + hh;
    const size_t orow = fr * p.num_splits + s;
    // Empty split: no position seen.  A split whose every score was NaN also
    // leaves the running max at -inf (fmaxf drops NaN) but its sum is NaN, and
    // it must come out NaN, so it takes the general path (NaN * 0 stays NaN).
    if (M == -INFINITY && !nan) {
      if (p.out) {
        p.out[fr * D + d] = 0;
        if (d == 0 && p.lse_out) p.lse_out[fr] = -INFINITY;
      } else {
        p.o_partial[orow * D + d] = 0.f;
        if (d == 0) p.lse_partial[orow] = -INFINITY;
      }
      continue;
    }
    float ls = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][hh];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      ls = fmaf(sm_l[w][hh], f, ls);
      o = fmaf(sm_acc[w][hh * D + d], f, o);
    }
    const float lse = (M + __builtin_amdgcn_logf(ls)) * kLn2;
    if (p.out) {
      const bool badl = lse != lse;
      p.out[fr * D + d] = uint16_t(f32_to_bf16_rne(badl ? NAN : o / ls));
      if (d == 0 && p.lse_out) p.lse_out[fr] = badl ? NAN : lse;
    } else {
      p.o_partial[orow * D + d] = o / ls;
      if (d == 0) p.lse_partial[orow] = lse;
    }
  }
}

template <int D, int kMode>
hipError_t launch_rows(const DecodeParams &p, hipStream_t stream) {
  constexpr int NH = 512 / D;
  constexpr int NBUF = 2;
  const dim3 grid{unsigned(p.num_splits * (p.Hkv / NH) * p.B)}, block{256};
  hipLaunchKernelGGL((paged_decode_rows_kernel<D, NBUF, kMode>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool paged_decode_rows_applies(const DecodeParams &p) {
  return p.G == 1 && (p.D == 64 || p.D == 128) && p.Hkv % (512 / p.D) == 0;
}

hipError_t launch_paged_decode_rows(const DecodeParams &p, hipStream_t stream) {
  const int mode = p.q_pos ? 1 : (p.k_new ? 2 : 0);
#define PKV_CASE(DD, MM) \
  if (p.D == DD && mode == MM) return launch_rows<DD, MM>(p, stream);
  PKV_CASE(64, 0) PKV_CASE(64, 1) PKV_CASE(64, 2)
  PKV_CASE(128, 0) PKV_CASE(128, 1) PKV_CASE(128, 2)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
