/*
 * rownorm_bench.h - benchmark helpers exported by librownorm.so beside the
 * normalization entry points of rownorm.h.  They are not part of the
 * normalization path: bench.py and the tests use them to measure a
 * streaming-copy ceiling, to evict caches, to calibrate hardware byte
 * counters, and to run the unfused add-then-RMSNorm comparison.  Status
 * codes are those of rownorm.h; arguments are checked before anything is
 * enqueued, on `stream`, without synchronizing.
 */
#ifndef ROWNORM_BENCH_H
#define ROWNORM_BENCH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "rownorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copies `bytes` bytes between two device buffers with one 16-byte load and
 * store per thread (1024-thread workgroups over the whole buffer, the
 * fastest plain streaming form measured on MI355X), byte by byte for an
 * unaligned tail.  Buffers must not overlap (RN_EOVERLAP); NULL with
 * bytes > 0 is RN_EINVAL. */
int rn_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

/* out = a + b over n elements of the activation type of `dtype` (float32
 * add, rounded to the storage type): the first launch of the unfused
 * add-then-RMSNorm comparison ("Write Triton Fused Add Rmsnorm Kernel",
 * Performance requirements: the traffic saved by fusing).  out may be
 * exactly a or b; any other overlap is RN_EOVERLAP. */
int rn_add(const void *a, const void *b, void *out, int64_t n, int dtype,
           hipStream_t stream);

/* How the backward at (N, H) on the current device reduces dgamma/dbeta on
 * the 16-byte vector path (vectorizable != 0) or the element-wise path:
 * *rows receives the number of float32 partial rows kernel 1 writes per
 * parameter (the persistent grid P, which does not grow with N), or 0 when
 * it writes none (the column sums of the rows, or a single workgroup that
 * writes dgamma/dbeta itself).  For reports: bench.py prints it beside each
 * backward's time.  Status codes as for the backward entry points. */
int rn_bwd_partial_rows(int64_t N, int64_t H, int dtype, int is_layernorm,
                        int vectorizable, int *rows);

#ifdef __cplusplus
}
#endif

#endif /* ROWNORM_BENCH_H */
