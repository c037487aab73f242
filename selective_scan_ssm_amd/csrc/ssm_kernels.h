// Internal interface between the C ABI (ssm_abi.cpp) and the kernel
// launchers (*.hip).  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

struct ScanArgs {
    const void *x, *delta, *z, *B, *C;   // io dtype
    const float *delta_bias, *A, *D, *h0;
    void *y;
    float *last_state;
    int64_t batch, seqlen, dim, dstate;
    int softplus;
    int bf16;                            // io dtype: 1 = bf16, 0 = fp32
    void *workspace;
    size_t workspace_bytes;
    // optional (read by the d_state-16 kernel; launch_scan_fwd_ckpt covers the
    // other widths): the state entering every 16-step block,
    // (batch, ceil(seqlen / 16), dim, dstate) fp32, for the backward's sweep
    float *ckpt = nullptr;
    // 1: visit the sequence from its last step to its first (d_state 16 only;
    // not with ckpt): y[t] is the readout after the steps t .. seqlen - 1 in
    // that order, and last_state the state after step 0
    int reverse = 0;
    // 1: the rows are patches of a grid_h x grid_w grid (seqlen = grid_h *
    // grid_w) visited column by column, step q at row (q mod grid_h) grid_w +
    // q div grid_h (q counted from the end with reverse); d_state 16 only, not
    // with ckpt, seqlen < 2^23 and seqlen * dim * io bytes < 2^31
    int column_major = 0;
    int64_t grid_h = 0, grid_w = 0;
    // error-path tests only: nonzero makes segments withhold their hand-off
    // and bounds the successor's wait at this many polls, so every job past
    // a tile's first segment gives up (and says so in the error word)
    uint32_t test_spin_limit = 0;
    // the block's prologue fused into the d_state-16 scan (launch_conv_scan_fwd):
    // x is the conv input; conv_w (dim, conv_k) fp32, conv_b (dim) optional,
    // conv_state (batch, dim, conv_k - 1) io dtype optional
    const float *conv_w = nullptr, *conv_b = nullptr;
    const void *conv_state = nullptr;
    int64_t conv_k = 0;
    // 1: x is fp32 while the other io tensors are bf16 (an internal fp32
    // intermediate, d_state below 16 only)
    int x_f32 = 0;
};

// The first 256 bytes of a forward scan's workspace: word 0 is the job
// ticket, word 1 the error word (nonzero once a segment's wait gave up),
// cleared by every call that uses the workspace.
constexpr size_t kErrorWordOffset = 4;

struct StepArgs {
    float *state;
    const void *x, *delta, *z, *B, *C;
    const float *delta_bias, *A, *D;
    void *y;
    int64_t batch, dim, dstate;
    int softplus;
    int bf16;
};

// General forward scan, 1 <= dstate <= 16.
size_t scan_fwd_workspace(const ScanArgs &a);
hipError_t launch_scan_fwd(const ScanArgs &a, hipStream_t s);

// The device address of this device's static scratch array (SSM_SCRATCH_BYTES,
// 256-byte aligned), resolved once per device: ssm_scan_fwd_noalloc's workspace.
hipError_t noalloc_scratch(void **out);

// d_state = 1 time-chunked scan.
size_t sm1_workspace(int64_t batch, int64_t seqlen, int64_t dim, int bf16);
hipError_t launch_sm1_scan(const ScanArgs &a, hipStream_t s);

// One decode step.
hipError_t launch_state_update(const StepArgs &a, hipStream_t s);

struct BwdArgs {
    const void *x, *delta, *z, *B, *C, *dout;     // io dtype
    const float *delta_bias, *A, *D, *h0, *dlast;
    void *dx, *ddelta, *dz, *dB, *dC;             // io dtype
    float *dA, *dD, *ddelta_bias, *dh0;
    int64_t batch, seqlen, dim, dstate;
    int softplus;
    int bf16;
    void *workspace;
    size_t workspace_bytes;
    // optional: the checkpoints a forward recorded (scan_ckpt_bytes); given,
    // the backward skips its own checkpoint pass
    const float *ckpt_in = nullptr;
};

// Backward of the forward scan, 1 <= dstate <= 16.
size_t scan_bwd_workspace(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int bf16);
// the time segments of the backward's sweep for a shape (segments, blocks each)
void scan_bwd_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int bf16, int *segments,
                   int *blocks_per_segment);
hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t s);
// The forward that also records the state entering every 16-step block in
// a.ckpt, (batch, ceil(seqlen / 16), dim, dstate) fp32, the layout the
// backward reads: one launch at d_state 16, the forward and a checkpoint pass
// otherwise.
hipError_t launch_scan_fwd_ckpt(const ScanArgs &a, hipStream_t s);

// The 2-D scan orders: gather into scan order, the forward scan, scatter y.
// The forward's own workspace comes first, so its error word sits where
// ssm_scan_status reads it; the gathered copies follow only for the orders
// that are not visited in place.
size_t scan_2d_workspace(const ScanArgs &a, bool has_z, int direction, int64_t height, int64_t width);
hipError_t launch_scan_2d(const ScanArgs &a, int64_t height, int64_t width, int direction, hipStream_t s);

struct ConvArgs {
    const void *x;                        // io dtype (batch, seqlen, dim)
    const float *weight, *bias;           // (dim, width), (dim)
    const void *state_in;                 // io dtype (batch, dim, width - 1) or null
    void *out, *state_out;
    int64_t batch, seqlen, dim;
    int width, silu, bf16;
    int out_f32 = 0;                      // 1: out is written in fp32 whatever the io dtype
};
struct ConvUpdateArgs {
    void *state;                          // io dtype (batch, dim, width - 1), in place
    const void *x;                        // (batch, dim)
    const float *weight, *bias;
    void *out;
    int64_t batch, dim;
    int width, silu, bf16;
};

struct SsdArgs {
    const void *x, *dt, *z, *B, *C;       // io dtype
    const float *dt_bias, *A, *D, *h0;    // (H), (H), (H), (batch, H, P, N)
    void *y;
    float *last_state;
    int64_t batch, seqlen, nheads, headdim, dstate;
    int softplus, bf16;
    void *workspace = nullptr;            // ssd_workspace() bytes, 256-byte aligned
    size_t workspace_bytes = 0;
};

// Mamba-2 multi-head scan (chunked, MFMA).
bool ssd_supported(int64_t headdim, int64_t dstate, int bf16);
// workspace of the time segments of the whole-line kernel (0: none needed)
size_t ssd_workspace(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int bf16);
// the time segments of a shape: (segments, 64-step chunks per segment)
void ssd_plan(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int bf16,
              int *segments, int *chunks_per_segment);
hipError_t launch_ssd_scan(const SsdArgs &a, hipStream_t s);

// dt_proj: delta (rows, dim) = xdt[:, :rank] (row stride ldx) x W^T, W (dim, rank);
// all three in the io dtype, fp32 accumulation on the matrix cores.
struct DtProjArgs {
    const void *xdt, *W;
    void *out;
    int64_t rows, rank, dim, ldx;
    int bf16;
};
hipError_t launch_dt_proj(const DtProjArgs &a, hipStream_t s);

// Causal depthwise conv1d (+ SiLU), whole sequence and one decode token.
hipError_t launch_conv1d(const ConvArgs &a, hipStream_t s);
// The window after a sequence alone: state_out = the last width - 1 inputs
// of (state_in, x) (a.out is not used).
hipError_t launch_conv_state_out(const ConvArgs &a, hipStream_t s);

// conv1d + SiLU feeding the forward scan: at d_state 16 one fused launch
// (the convolved x stays in registers); at other widths the filtered x goes
// to the workspace (after the scan's own) and the scan reads it.  The window
// after the sequence goes to conv_state_out when given.
size_t conv_scan_workspace(const ScanArgs &a);
hipError_t launch_conv_scan_fwd(const ScanArgs &a, void *conv_state_out, hipStream_t s);
hipError_t launch_conv1d_update(const ConvUpdateArgs &a, hipStream_t s);

}  // namespace ssm
