/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective-scan library
 *               (libssmscan.so).
 *
 * What the library computes (the Mamba-1 selective scan; definitions from
 * "Mamba State Space Models complete guide", youngju.dev, sections 2 and 5,
 * and the "Windows SM1 (Scalar Mamba1)" page for the d_state = 1 case):
 *
 *   for every batch b, channel d (independently) and step t = 0 .. T-1:
 *     v        = delta[b,t,d] + delta_bias[d]            (bias optional)
 *     Delta    = softplus(v) if delta_softplus else v    (section 5, selection)
 *     h[n]     = exp(Delta * A[d,n]) * h[n]              (section 2, ZOH Abar)
 *              + Delta * B[b,t,n] * x[b,t,d]             (section 5, Delta*B*x)
 *     out      = sum_n C[b,t,n] * h[n] + D[d] * x[b,t,d] (section 2 readout, D skip)
 *     y[b,t,d] = out * SiLU(z[b,t,d])                    (section 5 block gate; optional)
 *   with h starting at h0[b,d,:] (or 0) and last_state[b,d,:] = h after step T-1
 *   (h0 when T = 0).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, row-major, contiguous:
 *       x, delta, z, y : (batch, seqlen, d_inner)      -- io dtype
 *       B, C           : (batch, seqlen, d_state)      -- io dtype, shared by all d
 *       A              : (d_inner, d_state)            -- fp32
 *       D, delta_bias  : (d_inner)                     -- fp32
 *       h0, last_state, state : (batch, d_inner, d_state) -- fp32
 *     io dtype is SSM_F32 (float) or SSM_BF16 (bfloat16, stored as 16-bit
 *     words).  Internal arithmetic is fp32; y is rounded to the io dtype with
 *     round-to-nearest-even.
 *   - Ownership: every buffer is owned by the caller; the library never
 *     allocates or frees device memory, and keeps no pointer after a call
 *     returns.  The optional workspace is caller-provided scratch of at least
 *     the size the matching *_workspace_bytes() reports (NULL is allowed when
 *     that size is 0); its contents need not be initialised and are garbage
 *     after the call.
 *   - Aliasing: no output may overlap any input (y, last_state vs x, delta,
 *     z, B, C, h0 ...), except `state` of ssm_state_update, which is updated
 *     in place by design.
 *   - Streams: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns without waiting.  The caller synchronises.
 *   - Errors: arguments are validated before anything is enqueued; on a
 *     negative status nothing was launched and no output was touched.
 *     SSM_ERR_HIP means a HIP launch error was reported (nothing more is
 *     enqueued by that call).  A fault inside a kernel surfaces at the
 *     caller's next synchronisation, as for any HIP kernel.
 *   - Edge cases: batch == 0 or d_inner == 0 is a no-op returning SSM_OK.
 *     seqlen == 0 writes last_state := h0 (or zeros) and leaves y untouched.
 *   - Alignment: every pointer must be aligned to its element size (4 bytes
 *     for fp32 tensors, 2 bytes for bf16 tensors), else SSM_ERR_ALIGN.
 *   - Thread safety: the entry points may be called concurrently on different
 *     streams -- except ssm_scan_fwd_noalloc, whose calls share one scratch
 *     array per GPU (see there).  Their only global state is created once
 *     and guarded by locks: that scratch array's address, and the side stream
 *     of ssm_scan_bwd (see there).
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 3
#define SSM_MAX_D_STATE 16
#define SSM_MAX_CONV_WIDTH 4

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype_t;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_NULL = -1,      /* a required pointer is NULL                      */
    SSM_ERR_SHAPE = -2,     /* negative size, d_state outside [1, 16], overflow */
    SSM_ERR_DTYPE = -3,     /* io_dtype is not SSM_F32 / SSM_BF16              */
    SSM_ERR_ALIGN = -4,     /* a pointer is not aligned to its element size    */
    SSM_ERR_WORKSPACE = -5, /* workspace NULL or smaller than required         */
    SSM_ERR_HIP = -6,       /* the HIP runtime reported a launch error          */
    SSM_ERR_ALIAS = -7,     /* an output overlaps an input                      */
    SSM_ERR_WAIT = -8,      /* a segment's bounded wait gave up (ssm_scan_status) */
    SSM_ERR_SCRATCH = -9    /* the shape needs more than SSM_SCRATCH_BYTES (noalloc) */
} ssm_status_t;

/*
 * ssm_scan_fwd -- the forward selective scan over a whole sequence.
 * Passage: youngju.dev guide, section 5 ("complete Mamba implementation",
 * selective_scan; MambaBlock.forward for the gate), section 2 (ZOH and the
 * discrete recurrence).
 *   x, delta, B, C, A, y  required.
 *   delta_bias, D, z, h0  optional (NULL: no bias / no skip / no gate / h0 = 0).
 *   last_state            optional output (NULL: not written).
 *   d_state in [1, 16].
 */
int ssm_scan_fwd(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                 const float *A, const void *B, const void *C, const float *D, const void *z,
                 const float *h0, void *y, float *last_state, int64_t batch, int64_t seqlen,
                 int64_t d_inner, int64_t d_state, int io_dtype, void *workspace,
                 size_t workspace_bytes, void *stream);

/* Workspace bytes ssm_scan_fwd needs for this shape (0 = none). Returns
 * (size_t)-1 for invalid arguments. */
size_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                int io_dtype);

/*
 * ssm_scan_fwd_noalloc -- ssm_scan_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments as ssm_scan_fwd without the
 * workspace, same outputs (the same kernels run).  The scratch the scan needs
 * (ssm_scan_workspace_bytes for the shape) is taken from a static device array
 * of SSM_SCRATCH_BYTES that the library holds on each GPU it runs on until the
 * process ends; nothing is allocated or freed by the call.
 *   A shape whose scratch exceeds SSM_SCRATCH_BYTES: SSM_ERR_SCRATCH, nothing
 *   enqueued.  The scratch grows with batch x ceil(d_inner / 64) x d_state
 *   (512 bytes per state of a 64-channel tile): 16 MiB covers up to 2046 tiles
 *   at d_state 16, e.g. batch 16 at d_inner 8192.
 *   Every call on one GPU uses that GPU's array and leaves its contents
 *   behind; each call clears what must start at zero itself.  Calls that
 *   overlap on one GPU (different streams, or different host threads without
 *   ordering) race on the array and must not be issued.  ssm_scan_status does
 *   not apply (there is no caller workspace); a segment wait that gives up
 *   still poisons the affected outputs with NaN.  The first call on a device
 *   resolves the array's address there (once, under a lock).
 */
#define SSM_SCRATCH_BYTES (16u << 20)
int ssm_scan_fwd_noalloc(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                         const float *A, const void *B, const void *C, const float *D, const void *z,
                         const float *h0, void *y, float *last_state, int64_t batch, int64_t seqlen,
                         int64_t d_inner, int64_t d_state, int io_dtype, void *stream);

/*
 * ssm_conv_scan_fwd -- the Mamba block's prologue and the scan in one call
 * (youngju.dev guide, section 5, "complete Mamba implementation": the x
 * branch runs the causal depthwise conv1d, then SiLU, then the selective
 * scan).  The scan of ssm_scan_fwd runs on
 *     xc[b,t,d] = SiLU(conv_bias[d] + sum_{k<W} conv_weight[d,k] * x[b, t-(W-1)+k, d])
 * (W = conv_width; the inputs before step 0 come from conv_state_in, oldest
 * first, or are zeros): xc replaces x in Delta*B*x and in the D skip.  xc is
 * computed in fp32 and never rounded or stored; the result equals
 * ssm_causal_conv1d_fwd (apply_silu = 1) followed by ssm_scan_fwd up to that
 * intermediate rounding.
 *   x              : (batch, seqlen, d_inner) io dtype, the conv's input
 *   conv_weight    : (d_inner, conv_width) fp32, required; conv_width in [1, 4]
 *   conv_bias      : (d_inner) fp32, optional
 *   conv_state_in  : (batch, d_inner, conv_width - 1) io dtype, optional
 *   conv_state_out : same shape, optional output -- the last conv_width - 1
 *                    inputs of (conv_state_in, x), where a following call or
 *                    ssm_causal_conv1d_update continues
 *   every other argument as ssm_scan_fwd.  Workspace:
 *   ssm_conv_scan_workspace_bytes (at d_state 16 the scan's own: the filter
 *   runs inside the scan kernel; at other widths it adds room for xc in fp32,
 *   which the conv kernel writes there first and the scan then reads, so xc
 *   is not rounded to the io dtype on that path either).
 *   Errors as ssm_scan_fwd, plus conv_width outside [1, 4] (SSM_ERR_SHAPE),
 *   at d_state below 16 seqlen * d_inner * 4 bytes of 2 GiB or more
 *   (SSM_ERR_SHAPE),
 *   conv_weight NULL (SSM_ERR_NULL) and conv_state_out overlapping any input
 *   or output (SSM_ERR_ALIAS).  seqlen == 0 writes last_state = h0 and
 *   conv_state_out = conv_state_in (or zeros).
 */
int ssm_conv_scan_fwd(const void *x, const float *conv_weight, const float *conv_bias,
                      const void *conv_state_in, void *conv_state_out, int64_t conv_width,
                      const void *delta, const float *delta_bias, int delta_softplus, const float *A,
                      const void *B, const void *C, const float *D, const void *z, const float *h0,
                      void *y, float *last_state, int64_t batch, int64_t seqlen, int64_t d_inner,
                      int64_t d_state, int io_dtype, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Workspace bytes ssm_conv_scan_fwd needs (0 = none); (size_t)-1 for invalid
 * arguments. */
size_t ssm_conv_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                     int io_dtype);

/*
 * sm1_scan_fwd -- the d_state = 1 scan ("Windows SM1 (Scalar Mamba1)" page,
 * detailed sections: the scalar-state recurrence whose closed form is a
 * cumulative product and a cumulative sum).  Same definition as ssm_scan_fwd
 * with d_state = 1; the shapes drop the state axis:
 *   A: (d_inner)   B, C: (batch, seqlen)   h0, last_state: (batch, d_inner).
 * The kernel splits time into sub-chunks scanned in parallel inside one
 * workgroup and combines them with the associative (decay, offset) operator.
 * It needs no workspace (sm1_scan_workspace_bytes returns 0) except for
 * shapes it hands to the general kernel: seqlen == 0, or 256 rows of d_inner
 * spanning 2 GiB or more.
 */
int sm1_scan_fwd(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                 const float *A, const void *B, const void *C, const float *D, const void *z,
                 const float *h0, void *y, float *last_state, int64_t batch, int64_t seqlen,
                 int64_t d_inner, int io_dtype, void *workspace, size_t workspace_bytes,
                 void *stream);

size_t sm1_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int io_dtype);

/*
 * ssm_state_update -- one recurrent decode step (the recurrence with T = 1;
 * the constant-size state replaces any cache: "Windows SM1" page, detailed
 * sections, and the youngju.dev guide, section 2 duality note).
 *   state : (batch, d_inner, d_state) fp32, read and overwritten in place.
 *   x, delta, z, y : (batch, d_inner)   B, C : (batch, d_state).
 *   delta_bias, D, z optional.  d_state in [1, 16].
 */
int ssm_state_update(float *state, const void *x, const void *delta, const float *delta_bias,
                     int delta_softplus, const float *A, const void *B, const void *C,
                     const float *D, const void *z, void *y, int64_t batch, int64_t d_inner,
                     int64_t d_state, int io_dtype, void *stream);

/*
 * ssm_scan_bwd -- the gradient of ssm_scan_fwd (any d_state in [1, 16]; the
 * SM1 shapes are the d_state = 1 case with B, C of shape (batch, seqlen, 1)).
 * The pages train through the scan (youngju.dev guide, practical section: the
 * training loop's loss.backward(); "Windows SM1" page: the scalar-state model
 * is trained through autograd) without printing a backward: this is the exact
 * reverse-mode derivative of the definition above.
 *   Inputs: the forward's inputs (same layouts and conventions), plus
 *     dout  : (batch, seqlen, d_inner) io dtype  -- dL/dy
 *     dlast : (batch, d_inner, d_state) fp32     -- dL/dlast_state, optional
 *   Outputs (overwritten, never accumulated into):
 *     dx, ddelta     : (batch, seqlen, d_inner) io dtype, required
 *     dz             : same, required when z is given (not touched otherwise)
 *     dB, dC         : (batch, seqlen, d_state) io dtype, required
 *     dA             : (d_inner, d_state) fp32, required
 *     dD, ddelta_bias: (d_inner) fp32, optional (written only when D / delta_bias
 *                      are given and the pointer is not NULL)
 *     dh0            : (batch, d_inner, d_state) fp32, optional (written even
 *                      when h0 is NULL: it is dL/d(initial state))
 *   The gradient of delta is taken through softplus when delta_softplus is set.
 *   Workspace: ssm_scan_bwd_workspace_bytes() (state checkpoints every 16
 *   steps, per-tile partial sums and the carries of the time segments the
 *   reverse sweep is cut into; 256-byte aligned).  Sums over channels, over
 *   the batch and over segments are added in a fixed order, and the segments
 *   depend on the shape alone: results are deterministic.
 *   Limits: seqlen * d_inner and seqlen * d_state elements of one batch row,
 *   and d_inner * d_state fp32 checkpoints of one 16-step block, must span
 *   less than 2 GiB, else SSM_ERR_SHAPE.
 *   Streams: part of the work (the segment carries, which do not depend on the
 *   checkpoints) runs beside the checkpoint pass on a stream the library
 *   creates once per device (default priority, never destroyed), forked from
 *   `stream` and joined back into it by events; every kernel of the call is
 *   ordered after the work enqueued on `stream` before it, and the work
 *   enqueued on `stream` after it waits for all of them, also under graph
 *   capture of `stream`.  ssm_scan_bwd_ckpt runs on `stream` alone.
 *   Edge cases: seqlen == 0 gives dh0 = dlast (or 0) and zero dA, dD,
 *   ddelta_bias; batch == 0 gives zero dA, dD, ddelta_bias; d_inner == 0
 *   gives zero dB, dC.
 */
int ssm_scan_bwd(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                 const float *A, const void *B, const void *C, const float *D, const void *z,
                 const float *h0, const void *dout, const float *dlast, void *dx, void *ddelta,
                 float *ddelta_bias, float *dA, void *dB, void *dC, float *dD, void *dz,
                 float *dh0, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                 int io_dtype, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes ssm_scan_bwd needs for this shape.  Returns (size_t)-1 for
 * invalid arguments. */
size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                    int64_t d_state, int io_dtype);

/*
 * Saved checkpoints for training.  The backward recomputes the states of each
 * 16-step block from the state entering it (the "saved chunk carries" of a
 * checkpointed reverse sweep).  ssm_scan_bwd computes these checkpoints with
 * a forward pass of its own; a training step that runs the forward anyway
 * can record them there and hand them to ssm_scan_bwd_ckpt, which then skips
 * that pass.
 *
 * ssm_scan_ckpt_bytes -- bytes of the checkpoints for this shape:
 *   batch x ceil(seqlen / 16) x d_inner x d_state fp32, (size_t)-1 for
 *   invalid arguments.
 *
 * ssm_scan_fwd_ckpt -- ssm_scan_fwd (same arguments, same y and last_state,
 *   same workspace) that also writes `ckpt`: ckpt[b, j, d, n] is the state
 *   h[n] of chain (b, d) entering step 16 j (h0 for j = 0).  ckpt must be
 *   16-byte aligned (SSM_ERR_ALIGN), non-NULL when seqlen > 0 (SSM_ERR_NULL)
 *   and overlap no other argument (SSM_ERR_ALIAS).  At d_state 16 it is one
 *   pass; at other widths the forward and a checkpoint pass.
 *
 * ssm_scan_bwd_ckpt -- ssm_scan_bwd with `ckpt` as written by
 *   ssm_scan_fwd_ckpt on the same inputs (read only; same errors as above);
 *   the gradients are those ssm_scan_bwd returns.  Same workspace size.
 */
size_t ssm_scan_ckpt_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state);
int ssm_scan_fwd_ckpt(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                      const float *A, const void *B, const void *C, const float *D, const void *z,
                      const float *h0, void *y, float *last_state, float *ckpt, int64_t batch,
                      int64_t seqlen, int64_t d_inner, int64_t d_state, int io_dtype, void *workspace,
                      size_t workspace_bytes, void *stream);
int ssm_scan_bwd_ckpt(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                      const float *A, const void *B, const void *C, const float *D, const void *z,
                      const float *h0, const void *dout, const float *dlast, const float *ckpt, void *dx,
                      void *ddelta, float *ddelta_bias, float *dA, void *dB, void *dC, float *dD, void *dz,
                      float *dh0, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                      int io_dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssm_scan_fwd_2d -- one direction of the 2-D scan of the youngju.dev guide's
 * VMamba section (section 9, image processing): the sequence axis holds
 * height x width patches in row-major order, and the scan visits them in
 *   direction 0: row-major (left to right, top to bottom)
 *   direction 1: the reverse of 0 (right to left, bottom to top)
 *   direction 2: column-major (top to bottom, left to right: the grid transposed)
 *   direction 3: the reverse of 2
 * y is written at each patch's own (row-major) position, so the four
 * directions' outputs align for the block's sum; last_state is the state
 * after the last visited patch.  Same tensors and conventions as
 * ssm_scan_fwd with seqlen = height * width (height = 1 gives the plain
 * reversed 1-D scan with direction 1).  Direction 0 is the forward scan as
 * stored.  At d_state 16 the scan visits directions 1-3 in place (below 2^23
 * steps with a batch row under 2 GiB for directions 2 and 3); every other
 * case gathers the inputs into scan order and scatters y back.  The workspace
 * size (ssm_scan_2d_workspace_bytes, for the same direction) is the forward
 * scan's own workspace for the orders visited in place, and adds the gathered
 * copies of x, delta, z, B, C and y for the others.
 *   direction outside [0, 3] or negative height / width: SSM_ERR_SHAPE.
 */
int ssm_scan_fwd_2d(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                    const float *A, const void *B, const void *C, const float *D, const void *z,
                    const float *h0, void *y, float *last_state, int64_t batch, int64_t height,
                    int64_t width, int64_t d_inner, int64_t d_state, int direction, int io_dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of ssm_scan_fwd_2d in `direction` (has_z: whether z is
 * given); (size_t)-1 for invalid arguments (direction outside [0, 3]
 * included). */
size_t ssm_scan_2d_workspace_bytes(int64_t batch, int64_t height, int64_t width, int64_t d_inner,
                                   int64_t d_state, int direction, int has_z, int io_dtype);

/*
 * ssm_causal_conv1d_fwd -- the causal depthwise convolution (+ SiLU) that
 * produces the scan's input x in a Mamba block (youngju.dev guide, section 5,
 * "complete Mamba implementation": nn.Conv1d with groups = d_inner, kernel
 * size d_conv, padding d_conv - 1 and the output cut to seqlen, then SiLU):
 *     out[b,t,d] = bias[d] + sum_{k<width} weight[d,k] * x[b, t - (width-1) + k, d]
 *     (then SiLU when apply_silu)
 *   x, out        : (batch, seqlen, d_inner) io dtype
 *   weight        : (d_inner, width) fp32;  bias: (d_inner) fp32, optional
 *   conv_state_in : (batch, d_inner, width - 1) io dtype, optional -- the
 *                   inputs before step 0, oldest first (NULL: zeros)
 *   conv_state_out: same shape, optional -- the last width - 1 inputs of
 *                   (conv_state_in, x): the window a following call or
 *                   ssm_causal_conv1d_update continues from
 *   width in [1, SSM_MAX_CONV_WIDTH]; seqlen * d_inner of one batch row must
 *   span less than 2 GiB.  Outputs may not overlap inputs.
 */
int ssm_causal_conv1d_fwd(const void *x, const float *weight, const float *bias,
                          const void *conv_state_in, void *out, void *conv_state_out,
                          int apply_silu, int64_t batch, int64_t seqlen, int64_t d_inner,
                          int64_t width, int io_dtype, void *stream);

/*
 * ssm_causal_conv1d_update -- one decode token of the same convolution: the
 * window conv_state (batch, d_inner, width - 1) io dtype is read, out (batch,
 * d_inner) is computed over (window, x), and the window is shifted by one
 * with x appended, in place (the constant-size state of O(1) decoding,
 * "Windows SM1" page, detailed sections).
 */
int ssm_causal_conv1d_update(void *conv_state, const void *x, const float *weight,
                             const float *bias, void *out, int apply_silu, int64_t batch,
                             int64_t d_inner, int64_t width, int io_dtype, void *stream);

/*
 * ssm_dt_proj -- the projection that produces the scan's delta input in a
 * Mamba block (youngju.dev guide, section 5, "complete Mamba implementation":
 * dt_proj, a linear layer from dt_rank = d_model / 16 inputs to d_inner
 * outputs, applied to the first dt_rank columns of each x_proj output row,
 * then softplus; its bias is the scan's delta_bias, which ssm_scan_fwd adds
 * inside the softplus, so only the product is formed here):
 *     delta[m, d] = sum_{k < rank} xdt[m * ldx + k] * W[d * rank + k]
 *   xdt  : rows x ldx, io dtype (rows = batch * seqlen); only the first `rank`
 *          columns of each row are read (an x_proj row holds dt, then B, C)
 *   W    : (d_inner, rank), io dtype: the layer's weight, row-major
 *   delta: (rows, d_inner), io dtype, written; fp32 accumulation on the
 *          matrix cores, rounded once to the io dtype
 *   ldx >= rank; rank and ldx multiples of 8 (bf16) or 4 (fp32); d_inner a
 *   multiple of 4: else SSM_ERR_SHAPE.  xdt, W and delta 16-byte aligned:
 *   else SSM_ERR_ALIGN.  delta may not overlap xdt or W (SSM_ERR_ALIAS).
 *   rows == 0 or d_inner == 0: nothing is enqueued.
 */
int ssm_dt_proj(const void *xdt, int64_t ldx, const void *W, void *delta, int64_t rows,
                int64_t rank, int64_t d_inner, int io_dtype, void *stream);

/*
 * ssd_scan_fwd -- the Mamba-2 multi-head scan ("Mamba State Space Models
 * complete guide", youngju.dev, section 6 "Mamba 2": a multi-head SSM whose
 * decay is one scalar per head; the block's input projection yields x and z
 * per head, one B and one C per step shared by the heads, and one dt per
 * head).  For every batch row b, head h and channel p < headdim:
 *     Delta = softplus(dt[b,t,h] + dt_bias[h])        (softplus only if dt_softplus)
 *     s[n] <- exp(Delta * A[h]) s[n] + Delta * B[b,t,n] * x[b,t,h,p]
 *     y[b,t,h,p] = (sum_n C[b,t,n] s[n] + D[h] x[b,t,h,p]) * SiLU(z[b,t,h,p])
 * starting from h0[b,h,p,:] (zeros if NULL); last_state receives s after the
 * last step.  Evaluated in chunks of 64 steps with matrix products inside a
 * chunk and the recurrence between chunks (the section's SSD evaluation).
 *
 *   x, z, y       : (batch, seqlen, nheads, headdim) io dtype, row-major
 *   dt            : (batch, seqlen, nheads) io dtype
 *   B, C          : (batch, seqlen, dstate) io dtype
 *   A             : (nheads) fp32, required (negative for a decaying state)
 *   D, dt_bias    : (nheads) fp32, optional
 *   h0, last_state: (batch, nheads, headdim, dstate) fp32, optional
 * Supported: headdim a multiple of 16; dstate 32 or 64, and 128 for bf16 io,
 * else SSM_ERR_SHAPE.  x, z, y, B, C, h0, last_state must be 16-byte aligned
 * (SSM_ERR_ALIGN); one batch row of x (plus 128 steps) must span less than
 * 2 GiB (SSM_ERR_SHAPE).  Outputs may not overlap inputs (SSM_ERR_ALIAS).
 * All pointers are device memory, owned by the caller; nothing is allocated.
 *   workspace: ssd_scan_workspace_bytes() bytes, 256-byte aligned (may be
 *   NULL when that is 0): at few (batch, head, 64-channel) units the sequence
 *   is cut into time segments (bf16, headdim a multiple of 64, dstate <= 64),
 *   and the workspace holds each segment's final state from zero and its
 *   decay.  The segments depend on the shape alone: results are deterministic.
 *   Too small or NULL when needed: SSM_ERR_WORKSPACE.  It may not overlap any
 *   input or output (SSM_ERR_ALIAS).
 */
int ssd_scan_fwd(const void *x, const void *dt, const float *dt_bias, int dt_softplus,
                 const float *A, const void *B, const void *C, const float *D, const void *z,
                 const float *h0, void *y, float *last_state, int64_t batch, int64_t seqlen,
                 int64_t nheads, int64_t headdim, int64_t dstate, int io_dtype, void *workspace,
                 size_t workspace_bytes, void *stream);

/* Workspace bytes ssd_scan_fwd needs for a shape (0: none); SIZE_MAX for
 * arguments it would reject as SSM_ERR_SHAPE or SSM_ERR_DTYPE. */
size_t ssd_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                int64_t dstate, int io_dtype);

/*
 * ssm_scan_status -- whether the last forward scan that used `workspace`
 * completed its segment hand-offs.  No page covers this; it is the error
 * path of this library's own time split.
 *
 * The d_state-16 scan (and the general scan on many channel tiles) cuts long
 * sequences into segments; each segment waits for the state its predecessor
 * hands on through the workspace.  That wait is bounded: if it ever gives up,
 * the kernel sets an error word in the workspace and poisons the carried
 * state with NaN, so every output that depends on it (y from that segment on,
 * last_state) is NaN rather than a plausible wrong value.  This call
 * synchronises `stream` (waits for the work enqueued on it), reads that word
 * and returns
 *   SSM_OK        the waits of the last call on this workspace all completed
 *                 (also when that call needed no workspace wait at all);
 *   SSM_ERR_WAIT  a wait gave up: that call's y and last_state are invalid;
 *   SSM_ERR_NULL / SSM_ERR_WORKSPACE  workspace NULL or under 256 bytes;
 *   SSM_ERR_HIP   the synchronisation or the copy failed (for example a
 *                 fault of an earlier kernel on the stream).
 * `workspace` is the workspace of the last ssm_scan_fwd, ssm_scan_fwd_ckpt,
 * ssm_conv_scan_fwd or ssm_scan_fwd_2d call on `stream` (or of an sm1_scan_fwd call whose
 * sm1_scan_workspace_bytes was nonzero), not yet reused.  The error word is
 * cleared at the start of every such call.  Not capturable in a HIP graph
 * (it synchronises); call it outside a capture.
 */
int ssm_scan_status(const void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static string, never NULL). */
const char *ssm_status_string(int status);

/* SSM_ABI_VERSION of the built library. */
int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
