// Paged prefill attention: packed multi-token queries over the paged pool.
//
// Follows AstrAI "CUDA Kernels": section "Q Scheduling and KV Addressing"
// (packed [total_q, q_heads, head_dim] queries cut into 64-row Q tiles with a
// tile -> (request, tile index) map; the paged KV source only translates
// logical positions; HB = min(G, waves) q heads of one kv-head group packed
// per workgroup so a K/V tile is read once for all of them) and section
// "Python Wrappers" (is_causal; scale 1/sqrt(head_dim)).  A request's query
// rows are its last q_len positions: with the causal mask, row j of a request
// with kv_len tokens sees positions <= kv_len - q_len + j.
//
// gfx950 design.  Both products run on the matrix cores with the softmax in
// between kept per query row in registers:
//   S^T = K Q^T    A = a block of tokens of the K tile (LDS, row-major),
//                  B = Q^T (registers, loaded once); the output holds one
//                  query row per lane and a run of tokens per register group.
//   O^T += V^T P^T the probabilities are already in the B-operand layout of
//                  P^T; A = V^T comes straight from the row-major V tile
//                  through the LDS transpose read (ds_read_b64_tr_b16).  P is
//                  rounded to bf16 for the matrix core; the accumulators and
//                  the softmax statistics stay fp32.
// With two or more q heads per kv head a wave owns 32 query rows of one head
// and both products use v_mfma_f32_32x32x16_bf16, which sustained about
// twice the rate of the 16x16x32 form in a microbenchmark on this chip
// (independent accumulation chains); with four or more q heads per kv head
// the workgroup has 8 waves (4 heads x 64 rows), so one K/V tile in LDS
// serves twice the rows.  With one q head per kv head and long requests a
// workgroup takes a pair of host tiles, 128 rows of one head on 4 waves of
// the 32x32 form; with short requests its 64 rows are spread over its 4
// waves, 16 each, on the 16x16x32 form.
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kQTile = PKV_PREFILL_TILE_ROWS;   // query rows per host tile
constexpr int kKT = 64;                         // tokens per K/V tile
constexpr int kThreads = 256;                   // 4 waves (the 16x16x32 kernel)
constexpr float kLazy = 8.f;                    // lazy rescale threshold (log2 units)

#define PKV_LDS __attribute__((address_space(3)))

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// two fp32 -> packed bf16 (round to nearest even) on the hardware converter
__device__ __forceinline__ unsigned cvt_pk_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// max / sum of x over lanes l and l ^ 32 on the VALU: v_permlane32_swap on two
// copies of x leaves {x[l % 32], x[l % 32 + 32]} in the pair, on every lane
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte chunk permutation of K/V row r (only r & 15 matters), a bit
// shuffle of r XORed into the chunk index.  The LDS serves 256 bytes a cycle
// over 64 four-byte banks: 16 lanes of a 16-byte read, 32 lanes of an 8-byte
// (transpose) read.  The shuffle makes each of them touch every bank once:
//   - K reads, 16 rows at one logical chunk: the rows land on 16 distinct
//     chunks (D = 128, 256-byte rows), or on distinct (row parity, chunk)
//     pairs (D = 64, two 128-byte rows per bank line);
//   - transpose reads of the 32-row kernel, 4 rows (4a .. 4a + 3) x a block of
//     4 chunks: bits 2-3 of the shuffle (D = 128), or bit 2 across rows of
//     one parity (D = 64), take distinct values on those rows, so the 4 rows
//     land on 4 different chunk blocks;
//   - transpose reads of the 16-row kernel, 8 rows x a pair of chunks: bits
//     1-3 (D = 128), or bits 1-2 across rows of one parity (D = 64), take
//     distinct values on each aligned group of 8 rows.
template <int D>
__device__ __forceinline__ int swz(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
  if constexpr (D == 128) return r3 | (r2 << 1) | (r0 << 2) | (r1 << 3);
  else return r3 | (r2 << 1) | (r1 << 2);
}

// 16-byte sources for direct loads of rows that are not in the pool: zeros
// past the sequence end (masked positions must not carry NaN into P V), NaN
// for a page id outside the pool
__device__ __attribute__((aligned(16))) u32x4 kFillRows[2] = {
    {0u, 0u, 0u, 0u}, {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u}};

// The workgroup's slice of the work: a q chunk of RW rows of one request for
// HB q heads of one kv head.
struct Slice {
  int b, g, hg;              // request, kv head, group of HB q heads
  int q0, q_len, kv_len;     // first packed row, rows and positions of the request
  int wg_row0, wg_rows;      // the chunk's rows within the request
  int pos_base;              // position of the request's row 0
  int kv_end;                // positions the workgroup needs: [0, kv_end)
};

// 1-D grid, XCD-aware: consecutive workgroup ids go round-robin to the 8 XCDs,
// so id i takes logical slot (i % 8) * (n / 8) + i / 8 and each XCD runs a
// contiguous slice of the logical order (kv-head group major, then q chunks),
// whose workgroups read the same K/V rows through one L2.  The q chunks run
// last-first: with the causal mask they are the longest.  The n % 8 slots
// past the slices keep their ids.
__device__ __forceinline__ int xcd_slot(unsigned lin, unsigned n) {
  const unsigned per_xcd = n / 8;
  return int(lin < 8 * per_xcd ? (lin % 8) * per_xcd + lin / 8 : lin);
}

// Two jobs per workgroup: workgroup i of XCD i % 8 takes slots j and
// per_xcd - 1 - j of that XCD's slice, j = i / 8: the j-th longest q chunk and
// the j-th shortest, so every workgroup of the XCD gets about the same work,
// and the second job's loads and products hide the first job's prologue and
// the drain of its output stores (a workgroup of 8 waves fills its CU, so
// no other workgroup can).  An odd slice's middle slot runs once; the n % 8
// slots past the slices get a workgroup each.  -1: no such job.
__device__ __forceinline__ int paired_slot(unsigned lin, unsigned n, int job) {
  const unsigned per_xcd = n / 8, half = (per_xcd + 1) / 2;
  if (lin >= 8 * half) return job == 0 ? int(8 * per_xcd + (lin - 8 * half)) : -1;
  const unsigned x = lin % 8, j = lin / 8;
  const unsigned s = job == 0 ? j : per_xcd - 1 - j;
  if (job == 1 && s == j) return -1;
  return int(x * per_xcd + s);
}
__host__ __device__ constexpr unsigned paired_grid(unsigned n) { return 8 * ((n / 8 + 1) / 2) + n % 8; }

// The job at logical slot `logical` (one of the orders above).
//
template <int HB, int RW>
__device__ __forceinline__ bool locate(const PrefillParams &p, Slice &w, int job, int logical) {
  constexpr int CH = RW < kQTile ? kQTile / RW : 1;   // workgroups along one host tile
  constexpr int TPW = RW > kQTile ? RW / kQTile : 1;  // host tiles per workgroup
  static_assert(TPW <= 2, "at most a pair of host tiles per workgroup");
  const int hgroups = (p.G + HB - 1) / HB;
  const int n_x = (p.num_q_tiles + TPW - 1) / TPW * CH;   // workgroups per group
  // With long requests, the GB = groups / 8 groups of one XCD interleave
  // their q chunks inside the XCD's slice, so that the XCD starts every
  // group's longest chunks first rather than one group's after another's.
  const int n_groups = p.Hkv * hgroups;
  const int GB = p.interleave && n_groups % 8 == 0 ? n_groups / 8 : 1;
  const int blk = logical / (n_x * GB), rem = logical % (n_x * GB);
  const int gy = blk * GB + rem % GB, qx = n_x - 1 - rem / GB;
  int host_tile = qx / CH * TPW, rows = RW;
  const int chunk = qx % CH;
  w.g = gy / hgroups;
  w.hg = gy % hgroups;
  w.b = p.tile_to_batch[host_tile];
  int tile_index = p.tile_to_index[host_tile];
  if constexpr (TPW == 2) {
    const int t1 = host_tile + 1;
    const bool has_t1 = t1 < p.num_q_tiles;
    const int b1 = has_t1 ? p.tile_to_batch[t1] : -1;
    const int i1 = has_t1 ? p.tile_to_index[t1] : -1;
    const bool merged = has_t1 && b1 == w.b && i1 == tile_index + 1;
    if (job == 1) {
      if (merged || !has_t1) return false;
      w.b = b1;
      tile_index = i1;
    }
    rows = merged ? RW : kQTile;
  }
  if (unsigned(w.b) >= unsigned(p.B)) return false;
  // rows past total_q and positions past the page table are never touched
  w.q0 = min(max(p.qo_indptr[w.b], 0), p.total_q);
  w.q_len = min(p.qo_indptr[w.b + 1], p.total_q) - w.q0;
  w.kv_len = min(max(p.kv_lens[w.b], 0), p.max_pages << p.page_log2);
  w.wg_row0 = tile_index * kQTile + chunk * RW;
  w.wg_rows = min(rows, w.q_len - w.wg_row0);
  if (w.wg_row0 < 0 || w.wg_rows <= 0) return false;
  w.pos_base = w.kv_len - w.q_len;
  w.kv_end = p.causal ? min(w.kv_len, w.pos_base + w.wg_row0 + w.wg_rows) : w.kv_len;
  return true;
}

// Direct loads of one 64-token K/V tile into a pair of LDS buffers by the W
// waves of a workgroup: load n of a wave fills tile rows RWV * wave + n * RPI
// + lrow (RWV = 64 / W, lrow = lane / LPR); the lane's 16 bytes land at
// physical chunk lane % LPR, so it fetches the logical chunk that swz maps
// there.
template <int D, int W = 4>
struct TileLoader {
  static constexpr int PITCH = 2 * D;        // bytes per K/V row in LDS
  static constexpr int LPR = D / 8;          // lanes (16-byte chunks) per row
  static constexpr int RPI = 64 / LPR;       // rows per direct load (64 lanes)
  static constexpr int RWV = kKT / W;        // tile rows loaded by each wave
  static constexpr int NI = RWV / RPI;       // direct loads per wave, tile and tensor
  // the fast path reads a wave's RWV rows from one page of >= 16 tokens
  static_assert(RWV <= 16, "a wave's rows of a tile must fit in one 16-token page");

  const PrefillParams &p;
  const int32_t *pt;                         // the request's page-table row
  const __attribute__((address_space(4))) int32_t *pt_s;
  int wave, lrow, pc, g, kv_end, log2P, pmask;
  bool big_pages;
  size_t row_stride;                         // elements per pool row (slot)
  unsigned row_bytes;
  int colb[NI];                              // byte offset of the lane's chunk in a pool row
  int pid_next = 0;                          // page id of the wave's rows in the next tile

  __device__ TileLoader(const PrefillParams &p_, const Slice &w, int wave_, int lane)
      : p(p_), wave(wave_), g(w.g), kv_end(w.kv_end) {
    log2P = p.page_log2;
    pmask = (1 << log2P) - 1;
    // A wave loads RWV <= 16 consecutive positions per tile; with pages of 16
    // or more tokens they share one page, whose id is wave-uniform and read a
    // tile ahead with a scalar load (its own counter, so waiting for it never
    // waits for the direct loads in flight; the page table is read-only here,
    // and the constant address space lets the uniform load be scalar).
    big_pages = log2P >= 4;
    pt = p.page_table + size_t(w.b) * p.max_pages;
    pt_s = (const __attribute__((address_space(4))) int32_t *)(pt);
    lrow = lane / LPR;
    pc = lane % LPR;
    row_stride = size_t(p.Hkv) * D;
    row_bytes = unsigned(row_stride) * 2u;
#pragma unroll
    for (int n = 0; n < NI; ++n) colb[n] = 2 * (g * D + 8 * (pc ^ swz<D>((RWV * wave + n * RPI + lrow) & 15)));
  }

  __device__ __forceinline__ void fetch_pid(int t0) {
    const int t = t0 + RWV * wave;
    pid_next = (big_pages && t < kv_end) ? pt_s[t >> log2P] : 0;
  }

  __device__ __forceinline__ void issue(int t0, unsigned char *kb, unsigned char *vb) {
    const int pid = __builtin_amdgcn_readfirstlane(pid_next);
    if (big_pages && t0 + kKT <= kv_end && unsigned(pid) < unsigned(p.num_pages)) {
      // the wave's RWV positions are inside the sequence, in one pool page
      const unsigned row0 = (unsigned(pid) << log2P) | unsigned((t0 + RWV * wave) & pmask);
      const unsigned char *kbytes = reinterpret_cast<const unsigned char *>(p.k_pool);
      const unsigned char *vbytes = reinterpret_cast<const unsigned char *>(p.v_pool);
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const uint64_t a = uint64_t(row0 + unsigned(n * RPI + lrow)) * row_bytes + unsigned(colb[n]);
        const int dst = (RWV * wave + n * RPI) * PITCH;
        __builtin_amdgcn_global_load_lds(const_cast<unsigned char *>(kbytes + a), (PKV_LDS void *)(kb + dst), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(const_cast<unsigned char *>(vbytes + a), (PKV_LDS void *)(vb + dst), 16, 0, 0);
      }
      return;
    }
    // general case: every lane looks its page up; positions past the end
    // read zeros, a page id outside the pool reads NaN
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int t = t0 + RWV * wave + n * RPI + lrow;
      const int c = pc ^ swz<D>((RWV * wave + n * RPI + lrow) & 15);
      const int pg = t < kv_end ? pt[t >> log2P] : 0;
      const bool in_pool = t < kv_end && unsigned(pg) < unsigned(p.num_pages);
      const size_t off = ((size_t(in_pool ? pg : 0) << log2P) + (t & pmask)) * row_stride +
                         size_t(g) * D + 8 * c;
      const u32x4 *alt = kFillRows + (t < kv_end ? 1 : 0);
      const u32x4 *ks = in_pool ? reinterpret_cast<const u32x4 *>(p.k_pool + off) : alt;
      const u32x4 *vs = in_pool ? reinterpret_cast<const u32x4 *>(p.v_pool + off) : alt;
      const int dst = (RWV * wave + n * RPI) * PITCH;
      __builtin_amdgcn_global_load_lds(const_cast<u32x4 *>(ks), (PKV_LDS void *)(kb + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(const_cast<u32x4 *>(vs), (PKV_LDS void *)(vb + dst), 16, 0, 0);
    }
  }
};

// The direct loads write LDS outside the compiler's memory model: each lane
// waits for its own loads before the barrier that hands the tile to the other
// waves.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Two tiles per trip, one per LDS buffer pair; the barrier at each tile start
// waits for this tile's direct loads (all lanes) and for every wave to be done
// with the buffer pair that the next loads overwrite.  The page id of the tile
// after next is fetched at the end of a tile, so its latency hides in the
// barrier's wait.
template <class Loader, class Compute>
__device__ __forceinline__ void tile_loop(Loader &ld, int kv_end, unsigned char *k0,
                                          unsigned char *v0, unsigned char *k1, unsigned char *v1,
                                          Compute &&compute) {
  const int ntiles = (kv_end + kKT - 1) / kKT;
  if (ntiles > 0) {
    ld.fetch_pid(0);
    ld.issue(0, k0, v0);
    ld.fetch_pid(kKT);
  }
  for (int kt = 0; kt < ntiles; kt += 2) {
    tile_barrier();
    if (kt + 1 < ntiles) ld.issue((kt + 1) * kKT, k1, v1);
    compute(k0, v0, kt * kKT);
    if (kt + 1 >= ntiles) break;
    ld.fetch_pid((kt + 2) * kKT);
    tile_barrier();
    if (kt + 2 < ntiles) ld.issue((kt + 2) * kKT, k0, v0);
    compute(k1, v1, (kt + 1) * kKT);
    ld.fetch_pid((kt + 3) * kKT);
  }
}

// One q head per kv head: 4 waves x 16 rows of a 64-row q chunk, each on the
// 16x16x32 form (lane & 15 = query row, 4 tokens per register group).
template <int D>
__global__ __launch_bounds__(kThreads) void paged_prefill16_kernel(PrefillParams p) {
  constexpr int KS = D / 32;                 // MFMA k-steps over the head dimension
  constexpr int DB = D / 16;                 // 16-dim blocks of the output
  constexpr int PITCH = TileLoader<D>::PITCH;
  __shared__ __attribute__((aligned(16))) unsigned char sm_k0[kKT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char sm_v0[kKT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char sm_k1[kKT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char sm_v1[kKT * PITCH];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Slice w;
  if (!locate<1, kQTile>(p, w, 0, xcd_slot(blockIdx.x, gridDim.x))) return;
  const int h = w.g * p.G + w.hg;            // G == 1: the kv head's only q head
  const int my_row = w.wg_row0 + 16 * wave + (lane & 15);
  const bool row_ok = my_row < w.q_len;
  const int my_pos = w.pos_base + my_row;
  const int kv_end = w.kv_end;

  // Q^T as the B operand: lane = query row (lane & 15), dims 32j + 8(lane >> 4)
  bf16x8 qb[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row_ok)
      v = *reinterpret_cast<const u32x4 *>(p.q + (size_t(w.q0 + my_row) * p.Hq + h) * D + 32 * j + 8 * (lane >> 4));
    qb[j] = as_bf16x8(v);
  }
  float m = -INFINITY, l = 0.f;              // running max (log2 domain), lane's partial sum
  f32x4 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

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
    const bool full_tile = t0 + kKT <= kv_end && (!p.causal || t0 + kKT - 1 <= w.pos_base + w.wg_row0);
    // S^T for 4 blocks of 16 tokens: lane holds tokens 16mb + 4(lane >> 4) + r
    f32x4 s[4];
    // the next block's K fragments are read before this block's products
    // (pinned by a scheduling barrier)
    u32x4 ka[2][KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) ka[0][j] = *reinterpret_cast<const u32x4 *>(kb + koff[j]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb + 1 < 4)
#pragma unroll
        for (int j = 0; j < KS; ++j)
          ka[(mb + 1) & 1][j] = *reinterpret_cast<const u32x4 *>(kb + koff[j] + 16 * (mb + 1) * PITCH);
      __builtin_amdgcn_sched_barrier(0);
      s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j)
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[mb & 1][j]), qb[j], s[mb], 0, 0, 0);
    }
    // mask, then the tile max of this lane's row on the raw scores (scale > 0)
    float tmax = -INFINITY;
    if (!full_tile) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pos = t0 + 16 * mb + 4 * (lane >> 4) + r;
          const bool seen = pos < kv_end && (!p.causal || pos <= my_pos);
          s[mb][r] = seen ? s[mb][r] : -INFINITY;
        }
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, s[mb][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // The running max moves only when a row's tile max passes it by more than
    // kLazy: until then the probabilities are taken against the old max (at
    // most 2^kLazy) and the accumulators need no rescale; o / l is the same
    // quotient either way.
    const float ts = tmax * p.scale_log2;
    if (__any(ts > m + kLazy)) {             // wave-uniform
      const float mn = fmaxf(m, ts);
      const float alpha = (m == mn) ? 1.f : fast_exp2(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) o[i] *= alpha;
    }
    // probabilities in the B layout of P^T: k-slot 8(lane >> 4) + i <-> token
    // 32kb + 4(lane >> 4) + i (i < 4) or 32kb + 16 + 4(lane >> 4) + i - 4
    const float nm = m == -INFINITY ? 0.f : -m;   // masked scores give exp2(-inf) = 0
    u32x4 pb[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const float p0 = fast_exp2(fmaf(s[2 * kb2 + half][r], p.scale_log2, nm));
          const float p1 = fast_exp2(fmaf(s[2 * kb2 + half][r + 1], p.scale_log2, nm));
          l += p0 + p1;
          pb[kb2][2 * half + r / 2] = cvt_pk_bf16(p0, p1);
        }
    // O^T += V^T P^T over the tile's two 32-token k-blocks
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        const unsigned char *vp = vb + voff[i] + 32 * kb2 * PITCH;
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_LDS i16x4 *)(vp)));
        const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_LDS i16x4 *)(vp + 16 * PITCH)));
        const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
        o[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb[kb2]), o[i], 0, 0, 0);
      }
  };
  TileLoader<D> ld(p, w, wave, lane);
  tile_loop(ld, kv_end, sm_k0, sm_v0, sm_k1, sm_v1, compute);

  // row sums over the 4 lane groups, then the output row
  float lsum = l;
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (!row_ok) return;
  const float inv = 1.f / lsum;
  uint16_t *orow = p.out + (size_t(w.q0 + my_row) * p.Hq + h) * D;
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    u32x2 v;
    v[0] = cvt_pk_bf16(o[i][0] * inv, o[i][1] * inv);
    v[1] = cvt_pk_bf16(o[i][2] * inv, o[i][3] * inv);
    *reinterpret_cast<u32x2 *>(orow + 16 * i + 4 * (lane >> 4)) = v;
  }
  if (p.lse && lane < 16)
    p.lse[size_t(w.q0 + my_row) * p.Hq + h] = (m + __builtin_amdgcn_logf(lsum)) * kLn2;
}

// A wave owns 32 query rows of one head, on the 32x32x16 form (lane & 31 =
// query row; register r of a 32-token block is token 8(r / 4) + 4(lane >> 5)
// + r % 4).  HB heads per workgroup, W / HB waves per head (W = 8 when HB = 4
// and D = 128, else 4), so RW = 32 W / HB rows per head: 32 or 64 rows of one
// host tile, or with HB = 1 the 128 rows of a pair of host tiles.  The job
// loop of the pair form would take the kernel past 256 registers (one wave
// per SIMD); two waves per SIMD are asked for explicitly.
template <int D, int HB, int W>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2))) void paged_prefill32_kernel(
    PrefillParams p) {
  constexpr int KS = D / 16;                 // k-steps of S^T over the head dimension
  constexpr int MB = D / 32;                 // 32-dim blocks of O^T
  constexpr int WPH = W / HB;                // waves per q head
  constexpr int RW = WPH * 32;               // query rows per workgroup and head
  static_assert(kQTile % RW == 0 || RW % kQTile == 0, "row split");
  constexpr int PITCH = TileLoader<D>::PITCH;
  __shared__ __attribute__((aligned(16))) unsigned char sm_k0[kKT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char sm_v0[kKT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char sm_k1[kKT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char sm_v1[kKT * PITCH];

  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // one job; or two for a pair of host tiles that does not continue one
  // request; or with 8 waves the two mirrored slots of paired_slot
  constexpr int TPW = RW > kQTile ? RW / kQTile : 1;
  constexpr bool kPaired = W == 8 && TPW == 1;
  constexpr int NJ = kPaired ? 2 : TPW;
  constexpr int CH = RW < kQTile ? kQTile / RW : 1;
  const unsigned n_slots = unsigned((p.num_q_tiles + TPW - 1) / TPW * CH * p.Hkv * ((p.G + HB - 1) / HB));
  for (int job = 0; job < NJ; ++job) {
    Slice w;
    const int slot = kPaired ? paired_slot(blockIdx.x, n_slots, job) : xcd_slot(blockIdx.x, gridDim.x);
    if (slot < 0 || !locate<HB, RW>(p, w, kPaired ? 0 : job, slot)) continue;
    if (job > 0) __syncthreads();            // every wave is done with the previous job's tiles
    const int h_in_group = w.hg * HB + wave / WPH;
    const bool head_ok = h_in_group < p.G;
    const int h = w.g * p.G + (head_ok ? h_in_group : 0);
    const int wave_row0 = w.wg_row0 + (wave % WPH) * 32;
    const int my_row = wave_row0 + (lane & 31);
    const int row_end = w.wg_row0 + w.wg_rows;  // the job's rows: [wg_row0, row_end)
    const bool row_ok = head_ok && my_row < row_end;
    const int my_pos = w.pos_base + my_row;
    const int kv_end = w.kv_end;
    // a wave with no rows of the job skips every tile's products, and with
    // the causal mask a wave skips the tiles past its last row's position
    // (all of their scores are masked: exp gives 0 and the max is unchanged)
    const int wave_last_pos = head_ok && wave_row0 < row_end
                                  ? (p.causal ? w.pos_base + min(wave_row0 + 31, row_end - 1) : kv_end - 1)
                                  : -1;

    // Q^T as the B operand: lane = query row (lane & 31), dims 16j + 8(lane >> 5)
    bf16x8 qb[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok)
        v = *reinterpret_cast<const u32x4 *>(p.q + (size_t(w.q0 + my_row) * p.Hq + h) * D + 16 * j + 8 * hl);
      qb[j] = as_bf16x8(v);
    }
    float m = -INFINITY, l = 0.f;              // running max (log2 domain), lane's partial sum
    f32x16 o[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] = 0.f;

    // LDS read offsets.  K (A operand of S^T): row lane & 31 of a 32-row block,
    // logical chunk 2j + (lane >> 5).  V (transpose read, A operand of O^T):
    // lane 4k + q of the 16-lane group (hl, u) points at tile row 4hl + k (lo)
    // or 8 + 4hl + k (hi) of a 16-row block, dims 32i + 16u + 4q .. + 3.
    int koff[KS], vlo[MB], vhi[MB];
    {
      const int r = lane & 31;
#pragma unroll
      for (int j = 0; j < KS; ++j) koff[j] = r * PITCH + 16 * ((2 * j + hl) ^ swz<D>(r & 15));
      const int u = (lane >> 4) & 1, i = lane & 15, k = i >> 2, q = i & 3;
      const int r_lo = 4 * hl + k, r_hi = 8 + 4 * hl + k;
#pragma unroll
      for (int d = 0; d < MB; ++d) {
        const int c = 4 * d + 2 * u + (q >> 1);
        vlo[d] = r_lo * PITCH + 16 * (c ^ swz<D>(r_lo)) + 8 * (q & 1);
        vhi[d] = r_hi * PITCH + 16 * (c ^ swz<D>(r_hi)) + 8 * (q & 1);
      }
    }

    auto compute = [&](const unsigned char *kb, const unsigned char *vb, int t0) {
      if (t0 > wave_last_pos) return;          // wave-uniform
      const bool full_tile = t0 + kKT <= kv_end && (!p.causal || t0 + kKT - 1 <= w.pos_base + wave_row0);
      // S^T for 2 blocks of 32 tokens
      // (the two blocks are independent chains, interleaved k-step by k-step)
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][r] = 0.f;
      // (the K fragments of k-step j + RA are read while step j's products run;
      // the scheduling barrier keeps the compiler from sinking those reads back
      // next to their use)
      constexpr int RA = 3;
      u32x4 ka[RA + 1][2];
#pragma unroll
      for (int j = 0; j < RA; ++j)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) ka[j][mb] = *reinterpret_cast<const u32x4 *>(kb + koff[j] + 32 * mb * PITCH);
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        if (j + RA < KS)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            ka[(j + RA) % (RA + 1)][mb] = *reinterpret_cast<const u32x4 *>(kb + koff[j + RA] + 32 * mb * PITCH);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[j % (RA + 1)][mb]), qb[j], s[mb], 0, 0, 0);
      }
      float tmax = -INFINITY;
      if (!full_tile) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int pos = t0 + 32 * mb + 8 * (r >> 2) + 4 * hl + (r & 3);
            const bool seen = pos < kv_end && (!p.causal || pos <= my_pos);
            s[mb][r] = seen ? s[mb][r] : -INFINITY;
          }
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[mb][r]);
      tmax = max_xor32(tmax);
      const float ts = tmax * p.scale_log2;
      if (__any(ts > m + kLazy)) {             // wave-uniform lazy rescale
        const float mn = fmaxf(m, ts);
        const float alpha = (m == mn) ? 1.f : fast_exp2(m - mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < MB; ++i) o[i] *= alpha;
      }
      // P^T as the B operand of 4 k-steps of 16 tokens: k-slot 8(lane >> 5) + e
      // of step st <-> token 16st + 4(lane >> 5) + e (e < 4) or 16st + 8 +
      // 4(lane >> 5) + e - 4, i.e. register groups 2(st % 2) and 2(st % 2) + 1
      // of block st / 2
      const float nm = m == -INFINITY ? 0.f : -m;
      u32x4 pb[4];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int r = 8 * (st & 1) + e;
          const float p0 = fast_exp2(fmaf(s[st >> 1][r], p.scale_log2, nm));
          const float p1 = fast_exp2(fmaf(s[st >> 1][r + 1], p.scale_log2, nm));
          l += p0 + p1;
          pb[st][e >> 1] = cvt_pk_bf16(p0, p1);
        }
      // O^T += V^T P^T
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (PKV_LDS i16x4 *)(vb + vlo[i] + 16 * st * PITCH)));
          const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (PKV_LDS i16x4 *)(vb + vhi[i] + 16 * st * PITCH)));
          const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
          o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb[st]), o[i], 0, 0, 0);
        }
    };
    TileLoader<D, W> ld(p, w, wave, lane);
    tile_loop(ld, kv_end, sm_k0, sm_v0, sm_k1, sm_v1, compute);

    const float lsum = sum_xor32(l);
    if (row_ok) {
      const float inv = 1.f / lsum;
      uint16_t *orow = p.out + (size_t(w.q0 + my_row) * p.Hq + h) * D;
      // register 4q + e of block i is dim 32i + 8q + 4(lane >> 5) + e
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x2 v;
          v[0] = cvt_pk_bf16(o[i][4 * q] * inv, o[i][4 * q + 1] * inv);
          v[1] = cvt_pk_bf16(o[i][4 * q + 2] * inv, o[i][4 * q + 3] * inv);
          *reinterpret_cast<u32x2 *>(orow + 32 * i + 8 * q + 4 * hl) = v;
        }
      if (p.lse && lane < 32)
        p.lse[size_t(w.q0 + my_row) * p.Hq + h] = (m + __builtin_amdgcn_logf(lsum)) * kLn2;
    }
  }
}

template <int D>
hipError_t launch16(const PrefillParams &p, hipStream_t stream) {
  const dim3 grid{unsigned(p.num_q_tiles * p.Hkv * p.G)}, block{kThreads};
  hipLaunchKernelGGL((paged_prefill16_kernel<D>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int D, int HB, int W = 8>
hipError_t launch32(const PrefillParams &p, hipStream_t stream) {
  constexpr int RW = (W / HB) * 32;
  constexpr int CH = RW < kQTile ? kQTile / RW : 1;
  constexpr int TPW = RW > kQTile ? RW / kQTile : 1;
  const int hgroups = (p.G + HB - 1) / HB;
  const unsigned n_slots = unsigned((p.num_q_tiles + TPW - 1) / TPW * CH * p.Hkv * hgroups);
  const dim3 grid{W == 8 && TPW == 1 ? paired_grid(n_slots) : n_slots}, block{W * 64};
  hipLaunchKernelGGL((paged_prefill32_kernel<D, HB, W>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_prefill(const PrefillParams &params, hipStream_t stream) {
  // The XCD interleave of the work order pays with at least 8 host tiles per
  // request on average: on 2 x 2048-token causal prompts at D = 128 it took
  // one q head per kv head from 122-124 to 97-99 us and two from 107-110 to
  // 99-101 us, but 16 requests of 300 rows ran 4-5% slower with it, and 64
  // requests of 64 rows at D = 64 11% slower.
  PrefillParams p = params;
  p.interleave = p.num_q_tiles >= 8 * int64_t(p.B) ? 1 : 0;
  // HB = min(G, 4) q heads per workgroup share each K/V tile.  With four
  // heads at D = 128 the workgroup has 8 waves (64 rows per head, one per
  // CU); at D = 64 a tile carries half the products per barrier and
  // 4-wave workgroups, two per CU, measured 23% faster.
  const int HB = p.G < 4 ? p.G : 4;
  // One q head per kv head: 128-row workgroups (pairs of host tiles) on the
  // 32x32 form when the requests average at least 2 host tiles (D = 128) or 8
  // (D = 64), so that most pairs continue one request.  A pair split by a
  // request boundary runs as two jobs on half the waves, so batches of short
  // requests stay on the 16-row kernel: on 64 requests of 64 rows over 2048
  // cached tokens it is 4% (D = 128) and 16% (D = 64) faster, and on 2 x 2048
  // causal prompts it is 17% (D = 128) and 6% (D = 64) slower.
  if (HB == 1 && p.num_q_tiles < (p.D == 128 ? 2 : 8) * int64_t(p.B)) {
    if (p.D == 64) return launch16<64>(p, stream);
    if (p.D == 128) return launch16<128>(p, stream);
    return hipErrorInvalidValue;
  }
#define PKV_CASE(DD, HH) \
  if (p.D == DD && HB == HH) return launch32<DD, HH, (HH == 4 && DD == 128) ? 8 : 4>(p, stream);
  PKV_CASE(64, 1) PKV_CASE(64, 2) PKV_CASE(64, 4) PKV_CASE(128, 1) PKV_CASE(128, 2) PKV_CASE(128, 4)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
