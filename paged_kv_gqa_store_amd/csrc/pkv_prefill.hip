// Paged prefill attention: packed multi-token queries over the paged pool.
//
// Follows AstrAI "CUDA Kernels": section "Q Scheduling and KV Addressing"
// (packed [total_q, q_heads, head_dim] queries cut into 64-row Q tiles with a
// tile -> (request, tile index) map; the paged KV source only translates
// logical positions; HB = min(G, waves) q heads of one kv-head group packed
// per workgroup so a K/V tile is read once for all of them; the grid is
// (num_q_tiles * HB) x (kv_heads * ceil(G / HB))) and section "Python
// Wrappers" (is_causal; scale 1/sqrt(head_dim)).  A request's query rows are
// its last q_len positions: with the causal mask, row j of a request with
// kv_len tokens sees positions <= kv_len - q_len + j.
//
// gfx950 design, per wave: 16 or 32 query rows (one or two 16-row blocks) of
// one q head.
//   S^T = K Q^T    v_mfma_f32_16x16x32_bf16 with A = a 16-token block of the
//                  K tile (LDS, row-major) and B = Q^T (registers, loaded once):
//                  the output puts one query row per lane (lane & 15) and 4
//                  tokens per register group, so the online softmax of a row
//                  reduces over 16 registers and the 4 lane groups.
//   O^T += V^T P^T the probabilities are already in the B-operand layout of
//                  P^T (8 tokens of the lane's row); A = V^T comes straight
//                  from the row-major V tile through the LDS transpose read
//                  (ds_read_b64_tr_b16).  P is rounded to bf16 for the matrix
//                  core; the accumulators and the softmax statistics stay fp32.
// K and V tiles of 64 tokens move from the pool into LDS with direct loads
// (global_load_lds_dwordx4: 16 bytes per lane, no registers, no staging
// code), double-buffered, so one barrier per tile separates the loads of tile
// t + 1 from the reads of tile t.  Each row's 16-byte chunks are permuted by
// an XOR with a function of the row (swz below) chosen so that both the K
// reads (16 rows, one chunk) and the transpose reads (4 rows, 2 chunks per
// 16-lane group) hit distinct banks.
#include <math.h>

#include "pkv.h"
#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_prefill_launch.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kQTile = PKV_PREFILL_TILE_ROWS;   // query rows per host tile
constexpr int kKT = 64;                         // tokens per K/V tile
constexpr int kThreads = 256;                   // 4 waves

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// two fp32 -> packed bf16 (round to nearest even) on the hardware converter
__device__ __forceinline__ unsigned cvt_pk_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// 16-byte chunk permutation of K/V row r (only r & 15 matters): an XOR with a
// bit shuffle of r such that chunk c of 16 consecutive rows lands on distinct
// chunks, and so do chunks {2i, 2i + 1} of rows 4a .. 4a + 3 (D = 128: 16
// chunks per 256-byte row; D = 64: 8 chunks per 128-byte row, where rows of
// one parity also share banks).
template <int D>
__device__ __forceinline__ int swz(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
  if constexpr (D == 128) return r2 | (r0 << 1) | (r1 << 2) | (r3 << 3);
  else return r2 | ((r0 ^ r3) << 1) | ((r1 ^ r2) << 2);
}

// 16-byte sources for direct loads of rows that are not in the pool: zeros
// past the sequence end (masked positions must not carry NaN into P V), NaN
// for a page id outside the pool
__device__ __attribute__((aligned(16))) u32x4 kFillRows[2] = {
    {0u, 0u, 0u, 0u}, {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u}};

#define PKV_LDS __attribute__((address_space(3)))

template <int D, int HB, int RB>
__global__ __launch_bounds__(kThreads) void paged_prefill_kernel(PrefillParams p) {
  constexpr int KS = D / 32;                 // MFMA k-steps over the head dimension
  constexpr int DB = D / 16;                 // 16-dim blocks of the output
  constexpr int PITCH = 2 * D;               // bytes per K/V row in LDS
  constexpr int LPR = D / 8;                 // lanes (16-byte chunks) per row
  constexpr int RPI = 64 / LPR;              // rows per direct load (64 lanes)
  constexpr int NI = kKT / (4 * RPI);        // direct loads per wave, tile and tensor
  constexpr int R = 16 * RB;                 // query rows per wave (RB blocks of 16)
  constexpr int WPH = 4 / HB;                // waves per q head
  constexpr int RW = WPH * R;                // query rows per workgroup and head
  constexpr int CH = kQTile / RW;            // workgroups along one host tile
  static_assert(CH * RW == kQTile, "row split");
  static_assert(16 % RPI == 0 || RPI == 16, "a wave loads whole 16-row groups");
  // two buffers per tensor, separate objects so that reads of one buffer
  // need not wait for the direct loads in flight into the other
  __shared__ __attribute__((aligned(16))) unsigned char sm_k0[kKT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char sm_v0[kKT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char sm_k1[kKT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char sm_v1[kKT * PITCH];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // 1-D grid, XCD-aware: consecutive workgroup ids go round-robin to the 8
  // XCDs, so id i is given logical slot (i % 8) * (n / 8) + i / 8 and each XCD
  // runs a contiguous slice of the logical order (kv-head group major, then
  // q chunks), whose workgroups read the same K/V rows through one L2.  The
  // q chunks run last-first: with the causal mask they are the longest.
  const int hgroups = (p.G + HB - 1) / HB;
  const int n_x = p.num_q_tiles * CH;                         // workgroups per group
  const unsigned nwg = gridDim.x, per_xcd = nwg / 8;
  const unsigned lin = blockIdx.x;
  const int logical = int(lin < 8 * per_xcd ? (lin % 8) * per_xcd + lin / 8 : lin);
  const int gy = logical / n_x, qx = n_x - 1 - logical % n_x;
  const int host_tile = qx / CH, chunk = qx % CH;
  const int g = gy / hgroups, hg = gy % hgroups;
  const int b = p.tile_to_batch[host_tile];
  if (unsigned(b) >= unsigned(p.B)) return;                   // whole workgroup
  // rows past total_q and positions past the page table are never touched
  const int q0 = min(max(p.qo_indptr[b], 0), p.total_q);
  const int q_len = min(p.qo_indptr[b + 1], p.total_q) - q0;
  const int kv_len = min(max(p.kv_lens[b], 0), p.max_pages << p.page_log2);
  // rows of this workgroup within the request, and of this wave
  const int wg_row0 = p.tile_to_index[host_tile] * kQTile + chunk * RW;
  const int wg_rows = min(RW, q_len - wg_row0);
  if (wg_row0 < 0 || wg_rows <= 0) return;                   // whole workgroup
  const int h_in_group = hg * HB + wave / WPH;
  const bool head_ok = h_in_group < p.G;
  const int h = g * p.G + (head_ok ? h_in_group : 0);
  const int row0 = wg_row0 + (wave % WPH) * R;               // first row of this wave
  const int pos_base = kv_len - q_len;                        // position of row 0
  int my_row[RB], my_pos[RB];
  bool row_ok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    my_row[rb] = row0 + 16 * rb + (lane & 15);                // this lane's query rows
    row_ok[rb] = head_ok && my_row[rb] < q_len;
    my_pos[rb] = pos_base + my_row[rb];
  }
  // positions the workgroup needs: [0, kv_end)
  const int kv_end = p.causal ? min(kv_len, pos_base + wg_row0 + wg_rows) : kv_len;
  const int log2P = p.page_log2, pmask = (1 << log2P) - 1;
  const int32_t *pt = p.page_table + size_t(b) * p.max_pages;
  const size_t row_stride = size_t(p.Hkv) * D;

  // Q^T as the B operand: lane = query row (lane & 15), dims 32j + 8(lane >> 4)
  bf16x8 qb[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row_ok[rb])
        w = *reinterpret_cast<const u32x4 *>(p.q + (size_t(q0 + my_row[rb]) * p.Hq + h) * D + 32 * j + 8 * (lane >> 4));
      qb[rb][j] = as_bf16x8(w);
    }

  float m[RB], l[RB];   // running max (log2 domain) and this lane's partial sum, per row block
  f32x4 o[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int i = 0; i < DB; ++i) o[rb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Direct loads: load n of this wave fills tile rows 16 * wave + n * RPI + lrow
  // (lrow = lane / LPR); the lane's 16 bytes land at physical chunk lane % LPR,
  // so it fetches the logical chunk that swz maps there.
  const int lrow = lane / LPR, pc = lane % LPR;
  // A wave loads 16 consecutive positions per tile; with pages of 16 or more
  // tokens they share one page, whose id is wave-uniform and prefetched a
  // tile ahead with a scalar load (its own counter, so waiting for it never
  // waits for the direct loads in flight).
  const bool big_pages = log2P >= 4;
  // (read-only here: the constant address space lets the uniform load be scalar)
  const __attribute__((address_space(4))) int32_t *pt_s =
      (const __attribute__((address_space(4))) int32_t *)(pt);
  int pid_next = 0;
  auto fetch_pid = [&](int t0) {
    const int t = t0 + 16 * wave;
    pid_next = (big_pages && t < kv_end) ? pt_s[t >> log2P] : 0;
  };
  const u32x4 *fill = kFillRows;
  // byte offset of this lane's chunk within a pool row, per load
  int colb[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) colb[n] = 2 * (g * D + 8 * (pc ^ swz<D>(n * RPI + lrow)));
  const unsigned row_bytes = unsigned(row_stride) * 2u;
  const unsigned char *kbytes = reinterpret_cast<const unsigned char *>(p.k_pool);
  const unsigned char *vbytes = reinterpret_cast<const unsigned char *>(p.v_pool);
  auto issue = [&](int t0, unsigned char *kb, unsigned char *vb) {
    const int pid = __builtin_amdgcn_readfirstlane(pid_next);
    if (big_pages && t0 + kKT <= kv_end && unsigned(pid) < unsigned(p.num_pages)) {
      // the wave's 16 positions are inside the sequence, in one pool page
      const unsigned row0 = (unsigned(pid) << log2P) | unsigned((t0 + 16 * wave) & pmask);
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const uint64_t a = uint64_t(row0 + unsigned(n * RPI + lrow)) * row_bytes + unsigned(colb[n]);
        const int dst = (16 * wave + n * RPI) * PITCH;
        __builtin_amdgcn_global_load_lds(const_cast<unsigned char *>(kbytes + a), (PKV_LDS void *)(kb + dst), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(const_cast<unsigned char *>(vbytes + a), (PKV_LDS void *)(vb + dst), 16, 0, 0);
      }
      return;
    }
    // general case: every lane looks its page up; positions past the end
    // read zeros, a page id outside the pool reads NaN
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int t = t0 + 16 * wave + n * RPI + lrow;
      const int c = pc ^ swz<D>(n * RPI + lrow);
      const int pg = t < kv_end ? pt[t >> log2P] : 0;
      const bool in_pool = t < kv_end && unsigned(pg) < unsigned(p.num_pages);
      const size_t off = ((size_t(in_pool ? pg : 0) << log2P) + (t & pmask)) * row_stride +
                         size_t(g) * D + 8 * c;
      const u32x4 *alt = fill + (t < kv_end ? 1 : 0);
      const u32x4 *ks = in_pool ? reinterpret_cast<const u32x4 *>(p.k_pool + off) : alt;
      const u32x4 *vs = in_pool ? reinterpret_cast<const u32x4 *>(p.v_pool + off) : alt;
      const int dst = (16 * wave + n * RPI) * PITCH;
      __builtin_amdgcn_global_load_lds(const_cast<u32x4 *>(ks), (PKV_LDS void *)(kb + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(const_cast<u32x4 *>(vs), (PKV_LDS void *)(vb + dst), 16, 0, 0);
    }
  };
  // The direct loads write LDS outside the compiler's memory model: each lane
  // waits for its own loads before the barrier that hands the tile to the
  // other waves.
  auto tile_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // LDS read offsets.  K (A operand of S^T): row lane & 15 of a 16-row block,
  // logical chunk 4j + (lane >> 4).  V (transpose read): lane 4k + q of
  // 16-lane group G points at tile row 4G + k (+16), dims 16i + 4q .. + 3.
  int koff[KS], voff[DB];
  {
    const int i = lane & 15, G = lane >> 4;
#pragma unroll
    for (int j = 0; j < KS; ++j) koff[j] = i * PITCH + 16 * ((4 * j + G) ^ swz<D>(i));
    const int k = i >> 2, q = i & 3, vr = 4 * G + k;
#pragma unroll
    for (int d = 0; d < DB; ++d) voff[d] = vr * PITCH + 16 * ((2 * d + (q >> 1)) ^ swz<D>(vr)) + 8 * (q & 1);
  }

  auto compute = [&](const unsigned char *kb, const unsigned char *vb, int t0) {
    // every position of the tile is seen by every row of the workgroup: no mask
    const bool full_tile = t0 + kKT <= kv_end && (!p.causal || t0 + kKT - 1 <= pos_base + wg_row0);

    // S^T for 4 blocks of 16 tokens: lane holds tokens 16mb + 4(lane >> 4) + r of
    // row (lane & 15) of each row block; one K read from LDS feeds RB products
    f32x4 s[RB][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const u32x4 ka = *reinterpret_cast<const u32x4 *>(kb + koff[j] + 16 * mb * PITCH);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), qb[rb][j], s[rb][mb], 0, 0, 0);
      }
    }
    // probabilities in the B layout of P^T: k-slot 8(lane >> 4) + i <-> token
    // 32kb + 4(lane >> 4) + i (i < 4) or 32kb + 16 + 4(lane >> 4) + i - 4.
    // The running max m (log2 domain) moves only when a row's tile max passes
    // it by more than kLazy: until then the probabilities are taken against
    // the old max (at most 2^kLazy, exact in fp32 and bf16 range) and the
    // accumulators need no rescale; o / l is the same quotient either way.
    constexpr float kLazy = 8.f;
    float ts[RB];
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // mask, then the tile max of this lane's row on the raw scores (scale > 0)
      float tmax = -INFINITY;
      if (full_tile) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, s[rb][mb][r]);
      } else {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int pos = t0 + 16 * mb + 4 * (lane >> 4) + r;
            const bool seen = pos < kv_end && (!p.causal || pos <= my_pos[rb]);
            s[rb][mb][r] = seen ? s[rb][mb][r] : -INFINITY;
            tmax = fmaxf(tmax, s[rb][mb][r]);
          }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      ts[rb] = tmax * p.scale_log2;
      grow |= ts[rb] > m[rb] + kLazy;
    }
    if (__any(grow)) {               // wave-uniform: rescale every row block
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float mn = fmaxf(m[rb], ts[rb]);
        const float alpha = (m[rb] == mn) ? 1.f : fast_exp2(m[rb] - mn);
        m[rb] = mn;
        l[rb] *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) o[rb][i] *= alpha;
      }
    }
    u32x4 pb[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float nm = m[rb] == -INFINITY ? 0.f : -m[rb];   // masked scores give exp2(-inf) = 0
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int r = 0; r < 4; r += 2) {
            const float p0 = fast_exp2(fmaf(s[rb][2 * kb2 + half][r], p.scale_log2, nm));
            const float p1 = fast_exp2(fmaf(s[rb][2 * kb2 + half][r + 1], p.scale_log2, nm));
            l[rb] += p0 + p1;
            pb[rb][kb2][2 * half + r / 2] = cvt_pk_bf16(p0, p1);
          }
    }
    // O^T += V^T P^T over the tile's two 32-token k-blocks; one V^T read feeds RB products
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        const unsigned char *vp = vb + voff[i] + 32 * kb2 * PITCH;
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PKV_LDS i16x4 *)(vp)));
        const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PKV_LDS i16x4 *)(vp + 16 * PITCH)));
        const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          o[rb][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb[rb][kb2]), o[rb][i], 0, 0, 0);
      }
    }
  };

  // two tiles per trip, one per buffer; the barrier at each tile start waits
  // for this tile's direct loads (all lanes) and for every wave to be done
  // with the buffer that the next loads overwrite
  const int ntiles = (kv_end + kKT - 1) / kKT;
  if (ntiles > 0) {
    fetch_pid(0);
    issue(0, sm_k0, sm_v0);
    fetch_pid(kKT);
  }
  for (int kt = 0; kt < ntiles; kt += 2) {
    tile_barrier();
    if (kt + 1 < ntiles) issue((kt + 1) * kKT, sm_k1, sm_v1);
    compute(sm_k0, sm_v0, kt * kKT);
    if (kt + 1 >= ntiles) break;
    fetch_pid((kt + 2) * kKT);       // its latency hides in the barrier's wait
    tile_barrier();
    if (kt + 2 < ntiles) issue((kt + 2) * kKT, sm_k0, sm_v0);
    compute(sm_k1, sm_v1, (kt + 1) * kKT);
    fetch_pid((kt + 3) * kKT);
  }

  // row sums over the 4 lane groups, then the output rows
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lsum = l[rb];
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (!row_ok[rb]) continue;
    const float inv = 1.f / lsum;
    uint16_t *orow = p.out + (size_t(q0 + my_row[rb]) * p.Hq + h) * D;
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      u32x2 w;
      w[0] = cvt_pk_bf16(o[rb][i][0] * inv, o[rb][i][1] * inv);
      w[1] = cvt_pk_bf16(o[rb][i][2] * inv, o[rb][i][3] * inv);
      *reinterpret_cast<u32x2 *>(orow + 16 * i + 4 * (lane >> 4)) = w;
    }
    if (p.lse && lane < 16)
      p.lse[size_t(q0 + my_row[rb]) * p.Hq + h] = (m[rb] + __builtin_amdgcn_logf(lsum)) * kLn2;
  }
}

template <int D, int HB, int RB>
hipError_t launch(const PrefillParams &p, hipStream_t stream) {
  constexpr int CH = kQTile / ((4 / HB) * 16 * RB);
  const int hgroups = (p.G + HB - 1) / HB;
  const dim3 grid{unsigned(p.num_q_tiles * CH * p.Hkv * hgroups)}, block{kThreads};
  hipLaunchKernelGGL((paged_prefill_kernel<D, HB, RB>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_prefill(const PrefillParams &p, hipStream_t stream) {
  // HB = min(G, 4) q heads per workgroup.  At D = 64 a wave takes two 16-row
  // blocks once a workgroup holds two or more heads (one K/V^T read from LDS
  // then feeds two products); at D = 128 the second block's registers would
  // leave one wave per SIMD, which measured slower, so a wave keeps one block.
  const int HB = p.G < 4 ? p.G : 4;
#define PKV_CASE(DD, HH, RR) \
  if (p.D == DD && HB == HH) return launch<DD, HH, RR>(p, stream);
  PKV_CASE(64, 1, 1) PKV_CASE(64, 2, 2) PKV_CASE(64, 4, 2)
  PKV_CASE(128, 1, 1) PKV_CASE(128, 2, 2) PKV_CASE(128, 4, 2)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
