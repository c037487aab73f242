/*
 * ssm_scan_testing.h -- entry points of libssmscan.so that exist only so
 * tests can drive its error paths.  Not for production callers.
 */
#ifndef SSM_SCAN_TESTING_H
#define SSM_SCAN_TESTING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ssm_testing_scan_fwd_no_handoff -- ssm_scan_fwd (same arguments, same
 * validation, same workspace) with the segment hand-off withheld: no segment
 * publishes its final state, and a segment's wait for its predecessor gives
 * up after `spin_limit` polls (1 .. 65536, else SSM_ERR_SHAPE).  Every job
 * past a tile's first segment therefore gives up, and every kernel still ends
 * normally.  Shapes with one segment per tile (short sequences, or few
 * channel tiles below d_state 16) run exactly as ssm_scan_fwd.  Afterwards
 * ssm_scan_status on the workspace reports SSM_ERR_WAIT and the outputs of
 * the given-up segments (their y rows and last_state) are NaN.
 */
int ssm_testing_scan_fwd_no_handoff(const void *x, const void *delta, const float *delta_bias,
                                    int delta_softplus, const float *A, const void *B, const void *C,
                                    const float *D, const void *z, const float *h0, void *y,
                                    float *last_state, int64_t batch, int64_t seqlen, int64_t d_inner,
                                    int64_t d_state, int io_dtype, void *workspace,
                                    size_t workspace_bytes, uint32_t spin_limit, void *stream);

/*
 * ssm_testing_bwd_segments -- how ssm_scan_bwd / ssm_scan_bwd_ckpt cut each
 * (channel tile, batch row) sequence in time for the given shape: the number
 * of segments (*segments, >= 1) and the 16-step blocks per segment
 * (*blocks_per_segment; the last segment may be shorter).  A pure function of
 * the shape and io dtype.  Same argument rules as
 * ssm_scan_bwd_workspace_bytes; SSM_ERR_NULL for a null output pointer.
 */
int ssm_testing_bwd_segments(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                             int io_dtype, int *segments, int *blocks_per_segment);

/*
 * ssm_testing_ssd_segments -- how ssd_scan_fwd cuts each (batch, head,
 * 64-channel) sequence in time for the given shape: the number of segments
 * (*segments, >= 1) and the 64-step chunks per segment (*chunks_per_segment;
 * the last segment may be shorter).  A pure function of the shape and io
 * dtype.  Same argument rules as ssd_scan_workspace_bytes; SSM_ERR_NULL for a
 * null output pointer.
 */
int ssm_testing_ssd_segments(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                             int64_t dstate, int io_dtype, int *segments, int *chunks_per_segment);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_TESTING_H */
