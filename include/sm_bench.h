/*
 * sm_bench.h -- measurement-only kernels shipped in the same library.
 *
 * These are not part of the softmax operation. They exist so that a bench can
 * (1) empty the GPU's caches before each timed call, the cold lane that the
 * pages make their headline (Warpline README, the paragraph on the cold lane,
 * which touches a large buffer before every timed call; "Triton: Writing GPU
 * Kernels in Python, Measured", section "How it was timed", which zeroes a
 * buffer larger than L2), and (2) measure a plain 16-byte copy of known size,
 * the bandwidth ceiling against which the softmax is read (Warpline README,
 * the measured device-memory bandwidth ceiling) and the calibration for the
 * profiler's FETCH_SIZE / WRITE_SIZE counters.
 */
#ifndef SM_BENCH_H
#define SM_BENCH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` from src to dst with 16-byte vector loads and stores.
 *   src, dst : device pointers, 16-byte aligned, non-overlapping
 *   bytes    : a multiple of 16
 *   grid     : workgroups of 256 threads (0 = 8 per CU); each thread moves
 *              16 bytes per step of a grid-stride loop
 *   store_scope : 0 = plain stores (written back from L2 when the dispatch
 *              ends); 1 = device-scope stores, which write through each XCD's
 *              L2 (the policy of the library's row kernels)
 *   start_event, stop_event : optional (NULL) events attached to the kernel
 *              dispatch, as in sm_softmax_opts
 * Returns SM_OK (0) or a negative sm_status (SM_ERR_INVALID for bad
 * alignment, size or store_scope, SM_ERR_HIP for a failed launch).
 */
int sm_bench_copy(const void *src, void *dst, size_t bytes, int grid, int store_scope,
                  hipStream_t stream, hipEvent_t start_event, hipEvent_t stop_event);

/*
 * Read every 16-byte word of `buf` and write nothing, so that afterwards the L2
 * caches and the MALL hold this buffer's clean lines instead of any earlier
 * data (dirty lines of earlier work are written back during the sweep, not
 * during the next timed call). Use a buffer of at least 1 GiB on MI355X
 * (256 MiB MALL, 8 x 4 MiB L2). Same argument rules as sm_bench_copy.
 */
int sm_bench_flush(const void *buf, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SM_BENCH_H */
