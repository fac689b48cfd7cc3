/*
 * glu_ref.h -- data-movement reference kernels for measuring the
 * gated-activation kernels against what the memory system attains.
 *
 * Not part of the method: these kernels move exactly the bytes the streaming
 * forward and backward move, in the same access pattern and launch shape
 * (16-byte non-temporal loads and stores, one vector per stream per thread,
 * the same workgroup size and resident-workgroup cap), with the arithmetic
 * replaced by a bitwise XOR that keeps every load live.  Their rate is the
 * ceiling a kernel of that traffic mix reaches on the same device in the
 * same process ("Write a Triton SiLU-Mul (SwiGLU) Kernel", Performance
 * requirements: report achieved bandwidth against a stated ceiling).
 *
 * Conventions:
 *  - Pointers are DEVICE pointers owned by the caller, 16-byte aligned;
 *    `bytes` is the size of ONE stream, a multiple of 16.  Each call
 *    enqueues one or more kernel launches on `stream` and returns.
 *  - Output streams may coincide exactly with input streams (the in-place
 *    backward's pattern); the values written are meaningless.
 *  - Returns 0 on success, -1 for a NULL or unaligned pointer or a size that
 *    is not a multiple of 16 (checked on the host, nothing enqueued), or the
 *    hipError_t of a failed launch.
 */
#ifndef GLU_REF_H
#define GLU_REF_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef GLU_REF_API
#define GLU_REF_API __attribute__((visibility("default")))
#endif

/* The forward's mix: read a and b, write y (2:1).  Launch shape of the
 * 16-bit forward. */
GLU_REF_API int glu_ref_fwd_mix(const void *a, const void *b, void *y, uint64_t bytes, hipStream_t stream);

/* The backward's mix: read a, b and dy, write da and db (3:2).  Launch shape
 * of the 16-bit backward. */
GLU_REF_API int glu_ref_bwd_mix(const void *a, const void *b, const void *dy, void *da, void *db,
                                uint64_t bytes, hipStream_t stream);

/* The fused add + RMSNorm forward's traffic: read x and residual, write h
 * and y (2:2), as a flat stream: 64-thread workgroups, one vector per stream
 * per thread and a 6400-byte LDS reservation, the fastest shape a sweep of
 * 64 / 128 / 256 threads and reservations found for this mix at 4096 rows of
 * 2048 to 8192 bf16 values. */
GLU_REF_API int glu_ref_rms_mix(const void *x, const void *r, void *h, void *y, uint64_t bytes,
                                hipStream_t stream);

/* The strided kernels' LDS-tiled access pattern, bf16 only: 64 x 64 tiles,
 * 256 threads, the tiled kernel's launch order, the transposed operand
 * turned around through LDS, and 48 KiB of LDS per workgroup (three per CU,
 * the fastest cap for these mixes).  a, b, da, db are row-major (rows, cols)
 * with row stride cols; dyT and yT are stored transposed, (cols, rows)
 * row-major.  rows and cols must be positive multiples of 64 (else -1).
 * The backward's mix reads a, b and dyT and writes da, db (which may be a,
 * b); the forward's reads a, b and writes yT. */
GLU_REF_API int glu_ref_tile_bwd_mix(const void *a, const void *b, const void *dyT, void *da, void *db,
                                     int64_t rows, int64_t cols, hipStream_t stream);
GLU_REF_API int glu_ref_tile_fwd_mix(const void *a, const void *b, void *yT, int64_t rows, int64_t cols,
                                     hipStream_t stream);

/* A plain copy (1:1), 256-thread workgroups: the kernel of known traffic the
 * HBM counters are calibrated on. */
GLU_REF_API int glu_ref_copy(const void *src, void *dst, uint64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GLU_REF_H */
