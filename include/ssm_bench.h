/*
 * ssm_bench.h -- C ABI of libssmbench.so, the measurement helpers the
 *                benchmark uses to state the roofline of this GPU.  Nothing
 *                here is part of the scan library (libssmscan.so).
 *
 * Both calls take DEVICE pointers, enqueue one kernel on `stream` (a
 * hipStream_t; NULL = the null stream) and return without waiting.  They
 * validate their arguments first and enqueue nothing on an error.
 */
#ifndef SSM_BENCH_H
#define SSM_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SSM_MB_OK = 0, SSM_MB_ERR_ARG = -1, SSM_MB_ERR_HIP = -6 };

/* Copy `bytes` (a multiple of 16) from src to dst, both 16-byte aligned and
 * not overlapping, with 16-byte non-temporal loads and stores: the streaming
 * bandwidth a kernel of this library can expect from HBM. */
int ssm_mb_copy(const void *src, void *dst, size_t bytes, void *stream);

/* fp32 VALU issue-rate probe: `blocks` workgroups of 256 lanes, each lane
 * running 8 independent chains of `iters` steps of one operation
 * (op 0: fma, 1: exp2, 2: log2, 3: reciprocal); out receives one float per
 * lane (blocks * 256 floats) so the work is not removed. */
int ssm_mb_valu(int op, float *out, int64_t blocks, int64_t iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_BENCH_H */
