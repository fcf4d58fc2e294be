/*
 * pkv_bench.h -- C ABI of libpkv_bench.so: two plain 16-byte copy kernels
 * that bound what the store can reach on the same GPU.  They are measurement
 * instruments of bench.py, not steps of the decode path.
 *
 * Follows: mini-sglang handbook, "Custom CUDA kernels", section "Moving whole
 * rows by index" (a row move is pure memory traffic, so its ceiling is a copy
 * of the same bytes) and section "Exercises" (bytes moved per store).
 *
 * Conventions as include/pkv.h: device pointers, the caller's stream (a
 * hipStream_t, NULL = default), nothing allocated, freed or synchronised;
 * status 0 on success, PKV_ERR_* (-1 null, -2 shape, -4 alignment, -5 HIP)
 * otherwise, with nothing launched on an argument error.
 */
#ifndef PKV_BENCH_H
#define PKV_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pkvb_copy_linear -- dst[0 .. bytes) <- src[0 .. bytes): one 16-byte unit per
 * lane and iteration, a grid of up to 65536 workgroups striding over the
 * buffer, non-temporal loads and stores.  The contiguous-destination ceiling
 * of a read + write move.  bytes a multiple of 16; both pointers 16-byte
 * aligned; the buffers must not overlap.
 */
int32_t pkvb_copy_linear(void *dst, const void *src, int64_t bytes, void *stream);

/*
 * pkvb_copy_page_runs -- for every run r: rows run_src_row[r] .. + run_rows[r]
 * of k_src / v_src go to pool rows run_dst_slot[r] .. + run_rows[r] of k_dst /
 * v_dst.  One workgroup per run, 16-byte units, non-temporal.  With the runs
 * of a bulk fill (one run per page a sequence fills), this moves exactly the
 * bytes of pkv_kv_store, to exactly its destinations, without a per-row index:
 * the ceiling of the store's own access pattern.
 *   rows of row_bytes (a multiple of 16) at a stride of row_bytes on both
 *   sides; run arrays device int32 [n_runs]; src_rows / dst_rows bound every
 *   run (checked on the device: a run outside them is skipped).
 */
int32_t pkvb_copy_page_runs(void *k_dst, void *v_dst, int64_t dst_rows, const void *k_src,
                            const void *v_src, int64_t src_rows, const int32_t *run_src_row,
                            const int32_t *run_dst_slot, const int32_t *run_rows, int64_t n_runs,
                            int64_t row_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BENCH_H */
