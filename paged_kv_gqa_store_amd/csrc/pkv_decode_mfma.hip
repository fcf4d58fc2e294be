// Split-KV paged decode attention, matrix-core variant for gfx950.
//
// Same contract as the VALU kernel (see pkv_decode.hip and include/pkv.h):
// one workgroup per (split, kv head, sequence), the q heads of the kv-head
// group served by one pass over that head's K/V (AstrAI "CUDA Kernels",
// section "Q Scheduling and KV Addressing"), split-KV partials merged later.
//
// What runs where, per 16-token tile and per wave:
//   QK^T   one v_mfma_f32_16x16x32_bf16 per 32 dims: A = the group's q rows
//          (heads on M, zero-padded to 16), B = K^T (tokens on N).  K is read
//          from HBM as whole rows (every load instruction covers 4 or 8 full
//          rows: instructions that touch 16 rows x 64 B each measured ~25%
//          slower on gfx950) and re-laid into the B operand through a padded
//          per-wave LDS tile.
//   softmax   scores stay in the MFMA output layout (lane = token, register
//          = head); tile max by DPP row rotations within the 16-lane row;
//          exp2 on v_exp_f32 (q scale folded with log2 e).
//   P.V    on the VALU in fp32: a lane owns 8 dims of one token's V row per
//          load, p is broadcast from the score layout through a small LDS
//          slot; the accumulator is rescaled only when a head's max moved.
//   Page ids of a split are staged in LDS (fetched together with the
//   sequence length); each wave streams a contiguous range of tiles through
//   a ring of register buffers, with two (D=128) or three (D=64) tiles in
//   flight while one is computed (one with 8 q heads at D=128, which keeps
//   the kernel within 256 registers: two workgroups per CU).
//   K and V are read once, so their loads carry the non-temporal hint: on
//   gfx950 this measured ~10% faster than default-policy loads of the same
//   addresses (the lines are not kept in L2 / the memory-side cache).
//   With pages of >= 16 tokens a tile is one page's run of 16 slots: each
//   tile's loads go through one buffer descriptor per pool (scalar base at
//   the tile's first slot, a range that ends at the split's last position)
//   and constant per-lane offsets, so they need no vector address arithmetic,
//   and the slots past the range read zeros without touching memory.  The
//   ring's steady state runs whole passes of NBUF tiles; the remaining tiles,
//   already loaded, are computed after it, so no dummy tile is ever computed.
//   Workgroup order: kv head fastest, then sequence, then split.  With one
//   split this keeps the kv heads of a sequence (which read the same pages)
//   launched together; with several, every sequence's first split is
//   dispatched before any second split, so long ragged sequences start early.
//   With several splits and at most 256 (sequence, split) pairs, the pairs
//   go longest first (ranked in LDS by every workgroup).
#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// Native vector types only in the hot loop: HIP's uint4/float4 are structs,
// and a struct copy into LDS becomes a memcpy that pins its source to scratch.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;  // tokens per tile = N of one 16x16x32 MFMA
constexpr int kSegPages = 2048;  // page ids held in LDS at a time

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// streaming (non-temporal) 16-byte load for K/V rows, which are read exactly once
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
// Buffer descriptors (V#): base, no stride, a byte range; lanes whose offset
// falls outside the range read zeros and touch no memory.  Dword 3 of a gfx9
// descriptor: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), short(0), bytes, kRsrcWord3);
}
// streaming 16-byte load through a descriptor (cache policy nt)
__device__ __forceinline__ u32x4 ld16_buf_stream(__amdgpu_buffer_rsrc_t r, int voffset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 2);
}
__device__ __forceinline__ void unpack8v(const u32x4 &v, float f[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}

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

// Keeps the prefetch loads issued before it where they are: a compiler memory
// barrier (no instruction, no wait) stops IR passes sinking a load next to its
// use, and the scheduling barrier stops the machine scheduler doing the same.
__device__ __forceinline__ void pin_issue_order() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// kMode: 0 plain; 1 q rotated in the prologue; 2 the step's kv_store fused in
template <int D, int G, bool kPageTile, int NBUF, int kWaves, int kMode>
__global__ __launch_bounds__(kWaves * 64) void paged_decode_mfma_kernel(DecodeParams p) {
  constexpr bool kRope = kMode == 1, kFuse = kMode == 2;
  constexpr int KS = D / 32;      // MFMA k-steps per tile = V loads per lane per tile
  constexpr int LPV = D / 8;      // lanes per token in the V layout
  constexpr int TPV = 64 / LPV;   // tokens per V load instruction
  static_assert(TPV * KS == kTile, "tile shape");
  constexpr int HG = (G + 3) / 4; // 16-lane rows that hold real heads in the score layout

  constexpr int KPITCH = D * 2 + 16;   // bytes per K row in LDS (16-B pad: conflict-free MFMA reads)
  __shared__ int sm_pid[kSegPages];
  __shared__ __attribute__((aligned(16))) unsigned char sm_k[kWaves][kTile * KPITCH];
  __shared__ f32x4 sm_p[kWaves][HG][kTile];
  __shared__ f32x4 sm_alpha[kWaves][HG];
  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
  __shared__ float sm_acc[kWaves][G][D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // one-dimensional grid: kv head fastest, then the (sequence, split) pairs,
  // sequence before split; with few pairs and several splits (a ragged batch)
  // the pairs go longest first instead.  Either order is a function of the
  // arguments only, and a pair's result does not depend on its workgroup.
  int g = blockIdx.x % p.Hkv, b, s;
  bool empty_pair = false;        // a split past its sequence's end (known in the longest-first order)
  if (p.longest_first) {
    __shared__ __attribute__((aligned(16))) unsigned sm_key[kRankScratch<kWaves>];
    const int2 pk = pick_longest_first(p.seq_lens, p.B, p.num_splits, p.chunk, p.max_pages << p.page_log2,
                                       blockIdx.x / p.Hkv, sm_key);
    b = pk.x % p.B;
    s = pk.x / p.B;
    empty_pair = pk.y == 0;
  } else {
    b = (blockIdx.x / p.Hkv) % p.B;
    s = blockIdx.x / (p.Hkv * p.B);
  }
  if (empty_pair && (!kFuse || s > 0)) {
    // the result of an empty split (as in the epilogue), without its loads:
    // in a ragged batch these pairs are many, and they run last.  (A later
    // split never holds position L - 1; split 0 of an empty sequence takes the
    // full path, which stores the step's row as the unfused step would.)
    for (int idx = threadIdx.x; idx < G * D; idx += kWaves * 64) {
      const int h = idx / D, d = idx % D;
      const size_t frow = size_t(b) * p.Hq + size_t(g) * G + h;
      if (p.out) {
        p.out[frow * D + d] = 0;
        if (d == 0 && p.lse_out) p.lse_out[frow] = -INFINITY;
      } else {
        const size_t orow = frow * p.num_splits + s;
        p.o_partial[orow * D + d] = 0.f;
        if (d == 0) p.lse_partial[orow] = -INFINITY;
      }
    }
    return;
  }
  const int log2P = p.page_log2;
  const int pmask = (1 << log2P) - 1;
  const int32_t *pt = p.page_table + size_t(b) * p.max_pages;
  const int t0 = s * p.chunk;

  // Page ids of the first segment are fetched together with the sequence
  // length (the chunk is known on the host; entries past the sequence's end
  // are read but never used).
  const int pg0 = t0 >> log2P;
  auto fetch_pids = [&](int pga, int npg) {
    for (int i = threadIdx.x; i < npg; i += kWaves * 64) sm_pid[i] = pt[min(pga + i, p.max_pages - 1)];
  };
  const int chunk_pages = (p.chunk + pmask) >> log2P;
  fetch_pids(pg0, min(chunk_pages, kSegPages));

  int L = p.seq_lens[b];
  L = min(max(L, 0), p.max_pages << log2P);
  const int t1 = min(t0 + p.chunk, L);
  // fused store: head g of the new K / V row (8 dims per entry), for the tile
  // that holds position L - 1
  [[maybe_unused]] __shared__ u32x4 sm_new[2][D / 8];
  if constexpr (kFuse) {
    // The step's store, fused: the split holding position L - 1 (split 0 for
    // an empty sequence) copies head g of the new K/V row to its pool slot,
    // 16 bytes per lane (the store's contract: an index outside the pool is
    // not written).  The attention takes position L - 1 from the new row
    // itself, kept in LDS (ordered before its use by the barrier that opens
    // the first page-id segment), so no ordering with the pool writes is needed.
    const int sw = L > 0 ? min((L - 1) / p.chunk, p.num_splits - 1) : 0;
    constexpr int LPR = D / 8;
    if (s == sw && wave == 0 && lane < 2 * LPR) {
      const int64_t slot = p.slots[b];
      const size_t c = size_t(g) * D + 8 * (lane % LPR);
      const uint16_t *src = (lane < LPR ? p.k_new : p.v_new) + size_t(b) * p.new_stride + c;
      const u32x4 row = ld16(src);
      sm_new[lane / LPR][lane % LPR] = row;
      if (slot >= 0 && slot < p.num_slots) {
        uint16_t *dst = const_cast<uint16_t *>(lane < LPR ? p.k_pool : p.v_pool) + size_t(slot) * p.Hkv * D + c;
        *reinterpret_cast<u32x4 *>(dst) = row;
      }
    }
  }

  // q rows of the group as the MFMA A operand: lane = head (lane & 15), dims 32j + 8(lane >> 4)
  const int qh = lane & 15, qk = lane >> 4;
  bf16x8 qa[KS];
  [[maybe_unused]] const float *rc = nullptr, *rs = nullptr;
  [[maybe_unused]] bool pos_ok = true;
  if constexpr (kRope) {
    // rotary embedding of q (AstrAI "CUDA Kernels", section "Rotary Embedding
    // Kernel"): a lane's 8 dims are 4 whole pairs, rotated by the cos/sin row of
    // this sequence's query position and rounded to bf16 like the stored K.
    const int pos = p.q_pos[b];
    pos_ok = pos >= 0 && pos < p.rope_rows;
    rc = p.rope_cos + size_t(pos_ok ? pos : 0) * (D / 2);
    rs = p.rope_sin + size_t(pos_ok ? pos : 0) * (D / 2);
  }
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qh < G) {
      w = ld16(p.q + (size_t(b) * p.Hq + size_t(g) * G + qh) * D + 32 * j + 8 * qk);
      if constexpr (kRope) {
        const f32x4 c = *reinterpret_cast<const f32x4 *>(rc + 16 * j + 4 * qk);
        const f32x4 sn = *reinterpret_cast<const f32x4 *>(rs + 16 * j + 4 * qk);
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = pos_ok ? rope_pair(w[k], c[k], sn[k]) : 0x7fc07fc0u;
      }
    }
    qa[j] = as_bf16x8(w);
  }
  // Make q resident now: otherwise the first use inside the pipelined loop
  // would make the compiler wait for every load in flight.
#pragma unroll
  for (int j = 0; j < KS; ++j) asm volatile("" ::"v"(qa[j]));

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

  const size_t row_stride = size_t(p.Hkv) * D;
  // K and V are both read as whole rows: lane = 8 dims (lane % LPV) of token
  // slot lane / LPV; 4 (D=128) or 8 (D=64) full rows per load instruction.
  const uint16_t *kbase = p.k_pool + size_t(g) * D + 8 * (lane % LPV);
  const uint16_t *vbase = p.v_pool + size_t(g) * D + 8 * (lane % LPV);
  const uint16_t *qrow = p.q + (size_t(b) * p.Hq + size_t(g) * G) * D + 8 * (lane % LPV);
  const int vt = lane / LPV;
  // with whole-page tiles: byte offset of this lane's 16 bytes within the tile
  // for each load i (token slot TPV * i + vt, head g, dims 8 * (lane % LPV))
  const int row_bytes = int(row_stride) * 2;
  [[maybe_unused]] int voff[KS];
#pragma unroll
  for (int i = 0; i < KS; ++i) voff[i] = (TPV * i + vt) * row_bytes + (g * D + 8 * (lane % LPV)) * 2;

  struct Regs { u32x4 k[KS]; u32x4 v[KS]; int pid; };

  // Segments of at most kSegPages pages: their page ids sit in LDS while the
  // four waves stream the segment's tiles (each wave a contiguous range).
  for (int sa = t0; sa < t1;) {
    const int pga = sa >> log2P;
    const int sb = min(t1, (pga + kSegPages) << log2P);
    if (sa != t0) {
      __syncthreads();
      fetch_pids(pga, min(((sb - 1) >> log2P) - pga + 1, kSegPages));
    }
    __syncthreads();

    const int nst = (sb - sa + kTile - 1) / kTile;
    const int tpw = (nst + kWaves - 1) / kWaves;
    const int first = min(wave * tpw, nst);
    const int my_tiles = min(tpw, nst - first);
    const int last = sb - 1;
    const int tw0 = sa + kTile * first;   // first token of this wave's range

    // Loads tile k (clamped into the range by the caller); when `real` is
    // false the tile lies past the range and every lane reads the group's
    // first q row instead: an L2 hit, where repeating a K/V tile would go to
    // HBM again (lines loaded with the non-temporal hint are not retained).
    auto load_kv = [&](int k, Regs &rg, bool real) {
      const int tb = tw0 + kTile * k;
      if constexpr (kPageTile) {
        // A tile lies inside one page (tiles start on multiples of 16 within
        // pages of >= 16 tokens): one descriptor per tile and pool, based at
        // the tile's first slot and spanning its positions up to `last`.  The
        // lanes of positions past `last` read zeros, as does every lane of a
        // prefetch past the range (an empty span), and no load needs VALU
        // address arithmetic.
        const int raw = __builtin_amdgcn_readfirstlane(sm_pid[(tb >> log2P) - pga]);
        rg.pid = raw;
        const int pid = unsigned(raw) < unsigned(p.num_pages) ? raw : 0;
        const int64_t first_slot = (int64_t(pid) << log2P) + (tb & pmask);
        const int span = real ? min(last - tb + 1, kTile) * row_bytes : 0;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_pool + first_slot * int64_t(row_stride), span);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_pool + first_slot * int64_t(row_stride), span);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          rg.k[i] = ld16_buf_stream(rk, voff[i]);
          rg.v[i] = ld16_buf_stream(rv, voff[i]);
        }
      } else {
        const uint16_t *kb = real ? kbase : qrow;
        const uint16_t *vb = real ? vbase : qrow;
        const size_t rs = real ? row_stride : 0;
        rg.pid = sm_pid[(min(tb + (lane & 15), last) >> log2P) - pga];   // page of this lane's score token
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          const int tv = min(tb + TPV * i + vt, last);
          const int rv = sm_pid[(tv >> log2P) - pga];
          const int pv = unsigned(rv) < unsigned(p.num_pages) ? rv : 0;
          const size_t row = (size_t(pv) << log2P) + (tv & pmask);
          rg.k[i] = ld16_stream(kb + row * rs);
          rg.v[i] = ld16_stream(vb + row * rs);
        }
      }
    };

    auto compute = [&](int k, Regs rg) {
      const int tb = tw0 + kTile * k;
      if constexpr (kFuse) {
        // the one tile that holds position L - 1 (a wave-uniform test): the
        // lanes that loaded that position's pool slot take the new row instead
        if (L - 1 >= tb && L - 1 < tb + kTile) {
          const u32x4 kn = sm_new[0][lane % LPV], vn = sm_new[1][lane % LPV];
#pragma unroll
          for (int i = 0; i < KS; ++i) {
            const bool fresh = min(tb + TPV * i + vt, last) == L - 1;
            rg.k[i] = fresh ? kn : rg.k[i];
            rg.v[i] = fresh ? vn : rg.v[i];
          }
        }
      }
      // re-lay K from whole rows into the B operand (lane = token, 8 dims per k-step)
      unsigned char *kt = sm_k[wave];
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < KS; ++i)
        *reinterpret_cast<u32x4 *>(kt + (TPV * i + vt) * KPITCH + 16 * (lane % LPV)) = rg.k[i];
      wave_lds_sync();
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const u32x4 kb = ld16(kt + (lane & 15) * KPITCH + 16 * (4 * j + qk));
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], as_bf16x8(kb), c, 0, 0, 0);
      }
      // this lane: token tb + (lane & 15), heads 4 * (lane >> 4) + r
      const bool valid = tb + (lane & 15) <= last;
      const bool bad = unsigned(rg.pid) >= unsigned(p.num_pages);
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
        sm_p[wave][lane >> 4][lane & 15] = f32x4{pr[0], pr[1], pr[2], pr[3]};
        if ((lane & 15) == 0) sm_alpha[wave][lane >> 4] = f32x4{alpha[0], alpha[1], alpha[2], alpha[3]};
      }
      wave_lds_sync();
      float al[HG * 4];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const f32x4 a = sm_alpha[wave][hg];
        al[4 * hg] = a[0]; al[4 * hg + 1] = a[1]; al[4 * hg + 2] = a[2]; al[4 * hg + 3] = a[3];
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
          const f32x4 q4 = sm_p[wave][hg][TPV * i + vt];
          ph[4 * hg] = q4[0]; ph[4 * hg + 1] = q4[1]; ph[4 * hg + 2] = q4[2]; ph[4 * hg + 3] = q4[3];
        }
        float vf[8];
        unpack8v(rg.v[i], vf);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[h][d] = fmaf(ph[h], vf[d], acc[h][d]);
      }
    };

    // Ring of NBUF register tiles: NBUF-1 tiles are in flight while one is
    // computed.  The steady-state body is branch-free: loads past the range
    // read a q row (an L2 hit) and are never computed, so the compiler can
    // neither sink a prefetch next to its use nor merge waits across paths.
    // The last my_tiles % NBUF tiles, already loaded, are computed after it.
    if (my_tiles > 0) {
      const int lt = my_tiles - 1;
      Regs rg[NBUF];
#pragma unroll
      for (int j = 0; j < NBUF - 1; ++j) {
        load_kv(min(j, lt), rg[j], j <= lt);
        pin_issue_order();
      }
      int k = 0;
      for (; k + NBUF <= my_tiles; k += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          load_kv(min(k + u + NBUF - 1, lt), rg[(u + NBUF - 1) % NBUF], k + u + NBUF - 1 <= lt);
          pin_issue_order();
          compute(k + u, rg[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < NBUF - 1; ++u)
        if (k + u < my_tiles) compute(k + u, rg[u]);
    }
    sa = sb;
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

  // ---- merge the waves (ascending order = ascending positions) and write the partial
  for (int idx = threadIdx.x; idx < G * D; idx += kWaves * 64) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      M = fmaxf(M, sm_m[w][h]);
      nan |= sm_l[w][h] != sm_l[w][h];
    }
    const size_t frow = size_t(b) * p.Hq + size_t(g) * G + h;   // (b, q head)
    const size_t orow = frow * p.num_splits + s;
    // Empty split: no position seen.  A split whose every score was NaN also
    // leaves the running max at -inf (fmaxf drops NaN) but its sum is NaN, and
    // it must come out NaN, so it takes the general path (NaN * 0 stays NaN).
    if (M == -INFINITY && !nan) {
      if (p.out) {
        p.out[frow * D + d] = 0;
        if (d == 0 && p.lse_out) p.lse_out[frow] = -INFINITY;
      } else {
        p.o_partial[orow * D + d] = 0.f;
        if (d == 0) p.lse_partial[orow] = -INFINITY;
      }
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
    const float lse = (M + __builtin_amdgcn_logf(l)) * kLn2;
    if (p.out) {
      // the merge of one split: weight exp(lse - lse) = 1, so out is this
      // split's output rounded once, and a NaN lse gives the canonical NaN
      const bool bad = lse != lse;
      p.out[frow * D + d] = uint16_t(f32_to_bf16_rne(bad ? NAN : o / l));
      if (d == 0 && p.lse_out) p.lse_out[frow] = bad ? NAN : lse;
    } else {
      p.o_partial[orow * D + d] = o / l;
      if (d == 0) p.lse_partial[orow] = lse;
    }
  }
}

template <int D, int G, int kMode>
hipError_t launch_mfma(const DecodeParams &p, hipStream_t stream) {
  constexpr int kWaves = 4;
  const dim3 grid{unsigned(p.num_splits * p.Hkv * p.B)}, block{kWaves * 64};
  // tiles in the register ring: with 8 heads at D = 128 a ring of two keeps
  // the kernel within 256 registers, so two workgroups share a CU
  constexpr int NBUF = D == 128 ? (G == 8 ? 2 : 3) : 4;
  if (p.page_log2 >= 4)
    hipLaunchKernelGGL((paged_decode_mfma_kernel<D, G, true, NBUF, kWaves, kMode>), grid, block, 0,
                       stream, p);
  else
    hipLaunchKernelGGL((paged_decode_mfma_kernel<D, G, false, NBUF, kWaves, kMode>), grid, block, 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode(const DecodeParams &p, hipStream_t stream) {
  if (paged_decode_rows_applies(p)) return launch_paged_decode_rows(p, stream);
  return launch_paged_decode_mfma(p, stream);
}

hipError_t launch_paged_decode_mfma(const DecodeParams &p, hipStream_t stream) {
#define PKV_CASE(DD, GG)                                                        \
  if (p.D == DD && p.G == GG)                                                   \
    return p.q_pos ? launch_mfma<DD, GG, 1>(p, stream)                        \
                   : (p.k_new ? launch_mfma<DD, GG, 2>(p, stream) : launch_mfma<DD, GG, 0>(p, stream));
  PKV_CASE(64, 1) PKV_CASE(64, 2) PKV_CASE(64, 4) PKV_CASE(64, 8)
  PKV_CASE(128, 1) PKV_CASE(128, 2) PKV_CASE(128, 4) PKV_CASE(128, 8)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
