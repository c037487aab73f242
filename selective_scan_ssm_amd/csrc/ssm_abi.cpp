// C ABI of libssmscan.so (declared in include/ssm_scan.h): argument
// validation, then one launch on the caller's stream.  Validation never
// touches the HIP runtime, so every error path returns before anything is
// enqueued.
#include "ssm_scan.h"
#include "ssm_scan_testing.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <limits>

#include "ssm_kernels.h"

namespace {

constexpr int64_t kMaxGridY = 65535;   // batch rides on gridDim.y in the scan kernels

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// byte range [p, p + bytes) of one tensor, for overlap checks
struct Range {
    uintptr_t lo, hi;
};
Range range(const void *p, int64_t elems, size_t esize) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + static_cast<uintptr_t>(elems) * esize};
}
bool overlap(Range a, Range b) {
    if (a.lo == 0 || b.lo == 0 || a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// a*b*c without int64 overflow; -1 on overflow
int64_t mul3(int64_t a, int64_t b, int64_t c) {
    const int64_t big = std::numeric_limits<int64_t>::max() / 16;
    if (a < 0 || b < 0 || c < 0) return -1;
    if (a && b > big / a) return -1;
    const int64_t ab = a * b;
    if (ab && c > big / ab) return -1;
    return ab * c;
}

int check_dtype(int io) { return (io == SSM_F32 || io == SSM_BF16) ? SSM_OK : SSM_ERR_DTYPE; }
size_t io_size(int io) { return io == SSM_BF16 ? 2 : 4; }

// Validation shared by the two whole-sequence scans.
int validate_scan(const void *x, const void *delta, const float *delta_bias, const float *A,
                  const void *B, const void *C, const float *D, const void *z, const float *h0,
                  const void *y, const float *last_state, int64_t batch, int64_t seqlen,
                  int64_t dim, int64_t dstate, int io) {
    if (int r = check_dtype(io)) return r;
    if (batch < 0 || seqlen < 0 || dim < 0) return SSM_ERR_SHAPE;
    if (dstate < 1 || dstate > SSM_MAX_D_STATE) return SSM_ERR_SHAPE;
    if (batch > kMaxGridY) return SSM_ERR_SHAPE;
    const int64_t n_btd = mul3(batch, seqlen, dim);
    const int64_t n_btn = mul3(batch, seqlen, dstate);
    const int64_t n_bdn = mul3(batch, dim, dstate);
    if (n_btd < 0 || n_btn < 0 || n_bdn < 0 || mul3(dim, dstate, 1) < 0) return SSM_ERR_SHAPE;
    // workgroups are numbered by a 32-bit ticket: (batch x 64-channel tiles) x up to 8 time segments
    if (mul3(batch, (dim + 63) / 64, 8) > (int64_t(1) << 31)) return SSM_ERR_SHAPE;
    if (batch == 0 || dim == 0) return SSM_OK;   // nothing to read or write
    if (!A) return SSM_ERR_NULL;
    if (seqlen > 0 && (!x || !delta || !B || !C || !y)) return SSM_ERR_NULL;
    const size_t es = io_size(io);
    const void *io_ptrs[] = {x, delta, B, C, z, y};
    for (const void *p : io_ptrs)
        if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
    const void *f_ptrs[] = {delta_bias, A, D, h0, last_state};
    for (const void *p : f_ptrs)
        if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
    const Range outs[] = {range(y, seqlen > 0 ? n_btd : 0, es), range(last_state, n_bdn, 4)};
    const Range ins[] = {range(x, n_btd, es),        range(delta, n_btd, es),
                         range(z, n_btd, es),        range(B, n_btn, es),
                         range(C, n_btn, es),        range(A, dim * dstate, 4),
                         range(D, dim, 4),           range(delta_bias, dim, 4),
                         range(h0, n_bdn, 4)};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlap(o, i)) return SSM_ERR_ALIAS;
    if (overlap(outs[0], outs[1])) return SSM_ERR_ALIAS;
    return SSM_OK;
}

ssm::ScanArgs make_args(const void *x, const void *delta, const float *delta_bias, int softplus,
                        const float *A, const void *B, const void *C, const float *D,
                        const void *z, const float *h0, void *y, float *last_state,
                        int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io,
                        void *ws, size_t ws_bytes) {
    ssm::ScanArgs a;
    a.x = x; a.delta = delta; a.z = z; a.B = B; a.C = C;
    a.delta_bias = delta_bias; a.A = A; a.D = D; a.h0 = h0;
    a.y = y; a.last_state = last_state;
    a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.dstate = dstate;
    a.softplus = softplus ? 1 : 0;
    a.bf16 = io == SSM_BF16 ? 1 : 0;
    a.workspace = ws; a.workspace_bytes = ws_bytes;
    return a;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_ERR_HIP; }

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char *ssm_status_string(int status) {
    switch (status) {
    case SSM_OK: return "SSM_OK: success";
    case SSM_ERR_NULL: return "SSM_ERR_NULL: a required pointer is NULL";
    case SSM_ERR_SHAPE: return "SSM_ERR_SHAPE: invalid sizes (negative, d_state outside [1,16], batch > 65535 or overflow)";
    case SSM_ERR_DTYPE: return "SSM_ERR_DTYPE: io dtype must be SSM_F32 or SSM_BF16";
    case SSM_ERR_ALIGN: return "SSM_ERR_ALIGN: a pointer is not aligned to its element size";
    case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE: workspace missing or too small";
    case SSM_ERR_HIP: return "SSM_ERR_HIP: the HIP runtime reported a launch error";
    case SSM_ERR_ALIAS: return "SSM_ERR_ALIAS: an output overlaps an input";
    case SSM_ERR_WAIT: return "SSM_ERR_WAIT: a segment's bounded wait gave up; that call's outputs are invalid";
    case SSM_ERR_SCRATCH: return "SSM_ERR_SCRATCH: the shape needs more scratch than SSM_SCRATCH_BYTES (ssm_scan_fwd_noalloc)";
    default: return "unknown ssm status";
    }
}

size_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                int io_dtype) {
    if (check_dtype(io_dtype) || batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 1 ||
        d_state > SSM_MAX_D_STATE)
        return static_cast<size_t>(-1);
    ssm::ScanArgs a = make_args(nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr, nullptr, batch, seqlen, d_inner,
                                d_state, io_dtype, nullptr, 0);
    return ssm::scan_fwd_workspace(a);
}

int ssm_scan_fwd(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                 const float *A, const void *B, const void *C, const float *D, const void *z,
                 const float *h0, void *y, float *last_state, int64_t batch, int64_t seqlen,
                 int64_t d_inner, int64_t d_state, int io_dtype, void *workspace,
                 size_t workspace_bytes, void *stream) {
    int r = validate_scan(x, delta, delta_bias, A, B, C, D, z, h0, y, last_state, batch, seqlen,
                          d_inner, d_state, io_dtype);
    if (r) return r;
    if (batch == 0 || d_inner == 0) return SSM_OK;
    ssm::ScanArgs a = make_args(x, delta, delta_bias, delta_softplus, A, B, C, D, z, h0, y,
                                last_state, batch, seqlen, d_inner, d_state, io_dtype, workspace,
                                workspace_bytes);
    const size_t need = ssm::scan_fwd_workspace(a);
    if (need && (!workspace || workspace_bytes < need)) return SSM_ERR_WORKSPACE;
    if (need && !aligned(workspace, 256)) return SSM_ERR_ALIGN;
    return hip_status(ssm::launch_scan_fwd(a, static_cast<hipStream_t>(stream)));
}

int ssm_scan_fwd_noalloc(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                         const float *A, const void *B, const void *C, const float *D, const void *z,
                         const float *h0, void *y, float *last_state, int64_t batch, int64_t seqlen,
                         int64_t d_inner, int64_t d_state, int io_dtype, void *stream) {
    int r = validate_scan(x, delta, delta_bias, A, B, C, D, z, h0, y, last_state, batch, seqlen,
                          d_inner, d_state, io_dtype);
    if (r) return r;
    if (batch == 0 || d_inner == 0) return SSM_OK;
    ssm::ScanArgs a = make_args(x, delta, delta_bias, delta_softplus, A, B, C, D, z, h0, y,
                                last_state, batch, seqlen, d_inner, d_state, io_dtype, nullptr, 0);
    const size_t need = ssm::scan_fwd_workspace(a);
    if (need > SSM_SCRATCH_BYTES) return SSM_ERR_SCRATCH;
    if (need) {
        void *ptr = nullptr;             // this device's static scratch array
        if (ssm::noalloc_scratch(&ptr) != hipSuccess) return SSM_ERR_HIP;
        a.workspace = ptr;
        a.workspace_bytes = SSM_SCRATCH_BYTES;
    }
    return hip_status(ssm::launch_scan_fwd(a, static_cast<hipStream_t>(stream)));
}

size_t ssm_conv_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                     int io_dtype) {
    if (check_dtype(io_dtype) || batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 1 ||
        d_state > SSM_MAX_D_STATE || mul3(batch, seqlen, d_inner) < 0)
        return static_cast<size_t>(-1);
    ssm::ScanArgs a = make_args(nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr, nullptr, batch, seqlen, d_inner,
                                d_state, io_dtype, nullptr, 0);
    return ssm::conv_scan_workspace(a);
}

int ssm_conv_scan_fwd(const void *x, const float *conv_weight, const float *conv_bias,
                      const void *conv_state_in, void *conv_state_out, int64_t conv_width,
                      const void *delta, const float *delta_bias, int delta_softplus, const float *A,
                      const void *B, const void *C, const float *D, const void *z, const float *h0,
                      void *y, float *last_state, int64_t batch, int64_t seqlen, int64_t d_inner,
                      int64_t d_state, int io_dtype, void *workspace, size_t workspace_bytes,
                      void *stream) {
    int r = validate_scan(x, delta, delta_bias, A, B, C, D, z, h0, y, last_state, batch, seqlen,
                          d_inner, d_state, io_dtype);
    if (r) return r;
    if (conv_width < 1 || conv_width > SSM_MAX_CONV_WIDTH) return SSM_ERR_SHAPE;
    const int64_t n_win = mul3(batch, d_inner, conv_width - 1);
    if (n_win < 0) return SSM_ERR_SHAPE;
    // below d_state 16 the filtered x of one batch row (fp32) is addressed
    // with 32-bit byte offsets
    if (d_state != 16 && mul3(seqlen, d_inner, 4) > (int64_t(1) << 31) - 1) return SSM_ERR_SHAPE;
    if (batch == 0 || d_inner == 0) return SSM_OK;
    if (!conv_weight) return SSM_ERR_NULL;
    const size_t es = io_size(io_dtype);
    if (!aligned(conv_weight, 4) || (conv_bias && !aligned(conv_bias, 4))) return SSM_ERR_ALIGN;
    if ((conv_state_in && !aligned(conv_state_in, es)) || (conv_state_out && !aligned(conv_state_out, es)))
        return SSM_ERR_ALIGN;
    const int64_t n_btd = mul3(batch, seqlen, d_inner), n_btn = mul3(batch, seqlen, d_state);
    const int64_t n_bdn = mul3(batch, d_inner, d_state);
    const Range win_out = range(conv_state_out, n_win, es);
    const Range ins[] = {range(x, n_btd, es),         range(delta, n_btd, es),
                         range(z, n_btd, es),         range(B, n_btn, es),
                         range(C, n_btn, es),         range(A, d_inner * d_state, 4),
                         range(D, d_inner, 4),        range(delta_bias, d_inner, 4),
                         range(h0, n_bdn, 4),         range(conv_weight, d_inner * conv_width, 4),
                         range(conv_bias, d_inner, 4), range(conv_state_in, n_win, es)};
    const Range outs[] = {range(y, seqlen > 0 ? n_btd : 0, es), range(last_state, n_bdn, 4), win_out};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlap(o, i)) return SSM_ERR_ALIAS;
    if (overlap(outs[0], win_out) || overlap(outs[1], win_out)) return SSM_ERR_ALIAS;
    ssm::ScanArgs a = make_args(x, delta, delta_bias, delta_softplus, A, B, C, D, z, h0, y,
                                last_state, batch, seqlen, d_inner, d_state, io_dtype, workspace,
                                workspace_bytes);
    a.conv_w = conv_weight; a.conv_b = conv_bias; a.conv_state = conv_state_in; a.conv_k = conv_width;
    const size_t need = ssm::conv_scan_workspace(a);
    if (need && (!workspace || workspace_bytes < need)) return SSM_ERR_WORKSPACE;
    if (need && !aligned(workspace, 256)) return SSM_ERR_ALIGN;
    return hip_status(ssm::launch_conv_scan_fwd(a, conv_state_out, static_cast<hipStream_t>(stream)));
}

size_t sm1_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int io_dtype) {
    if (check_dtype(io_dtype) || batch < 0 || seqlen < 0 || d_inner < 0)
        return static_cast<size_t>(-1);
    return ssm::sm1_workspace(batch, seqlen, d_inner, io_dtype == SSM_BF16);
}

int sm1_scan_fwd(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                 const float *A, const void *B, const void *C, const float *D, const void *z,
                 const float *h0, void *y, float *last_state, int64_t batch, int64_t seqlen,
                 int64_t d_inner, int io_dtype, void *workspace, size_t workspace_bytes,
                 void *stream) {
    int r = validate_scan(x, delta, delta_bias, A, B, C, D, z, h0, y, last_state, batch, seqlen,
                          d_inner, 1, io_dtype);
    if (r) return r;
    if (batch == 0 || d_inner == 0) return SSM_OK;
    const size_t need = ssm::sm1_workspace(batch, seqlen, d_inner, io_dtype == SSM_BF16);
    if (need && (!workspace || workspace_bytes < need)) return SSM_ERR_WORKSPACE;
    if (need && !aligned(workspace, 256)) return SSM_ERR_ALIGN;
    ssm::ScanArgs a = make_args(x, delta, delta_bias, delta_softplus, A, B, C, D, z, h0, y,
                                last_state, batch, seqlen, d_inner, 1, io_dtype, workspace,
                                workspace_bytes);
    return hip_status(ssm::launch_sm1_scan(a, static_cast<hipStream_t>(stream)));
}

int ssm_state_update(float *state, const void *x, const void *delta, const float *delta_bias,
                     int delta_softplus, const float *A, const void *B, const void *C,
                     const float *D, const void *z, void *y, int64_t batch, int64_t d_inner,
                     int64_t d_state, int io_dtype, void *stream) {
    if (int r = check_dtype(io_dtype)) return r;
    if (batch < 0 || d_inner < 0 || d_state < 1 || d_state > SSM_MAX_D_STATE) return SSM_ERR_SHAPE;
    const int64_t n_bd = mul3(batch, d_inner, 1), n_bdn = mul3(batch, d_inner, d_state);
    // one quad of lanes per chain, 64 chains per workgroup: the grid's lane
    // count (batch x d_inner rounded up to 64, x 4) must stay below 2^32
    const int64_t lanes = mul3(batch, (d_inner + 63) / 64 * 64, 4);
    if (n_bd < 0 || n_bdn < 0 || lanes < 0 || lanes >= (int64_t(1) << 32)) return SSM_ERR_SHAPE;
    if (batch == 0 || d_inner == 0) return SSM_OK;
    if (!state || !x || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;
    const size_t es = io_size(io_dtype);
    const void *io_ptrs[] = {x, delta, B, C, z, y};
    for (const void *p : io_ptrs)
        if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
    const void *f_ptrs[] = {state, delta_bias, A, D};
    for (const void *p : f_ptrs)
        if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
    const int64_t n_bn = batch * d_state;
    const Range outs[] = {range(y, n_bd, es), range(state, n_bdn, 4)};
    const Range ins[] = {range(x, n_bd, es),       range(delta, n_bd, es), range(z, n_bd, es),
                         range(B, n_bn, es),       range(C, n_bn, es),     range(A, d_inner * d_state, 4),
                         range(D, d_inner, 4),     range(delta_bias, d_inner, 4)};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlap(o, i)) return SSM_ERR_ALIAS;
    if (overlap(outs[0], outs[1])) return SSM_ERR_ALIAS;
    ssm::StepArgs a;
    a.state = state; a.x = x; a.delta = delta; a.z = z; a.B = B; a.C = C;
    a.delta_bias = delta_bias; a.A = A; a.D = D; a.y = y;
    a.batch = batch; a.dim = d_inner; a.dstate = d_state;
    a.softplus = delta_softplus ? 1 : 0;
    a.bf16 = io_dtype == SSM_BF16 ? 1 : 0;
    return hip_status(ssm::launch_state_update(a, static_cast<hipStream_t>(stream)));
}

size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                    int64_t d_state, int io_dtype) {
    if (check_dtype(io_dtype) || batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 1 ||
        d_state > SSM_MAX_D_STATE)
        return static_cast<size_t>(-1);
    return ssm::scan_bwd_workspace(batch, seqlen, d_inner, d_state, io_dtype == SSM_BF16);
}

}  // extern "C"

namespace {
// ssm_scan_bwd and ssm_scan_bwd_ckpt: ckpt == nullptr computes the checkpoints
int scan_bwd_impl(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                  const float *A, const void *B, const void *C, const float *D, const void *z,
                  const float *h0, const void *dout, const float *dlast, void *dx, void *ddelta,
                  float *ddelta_bias, float *dA, void *dB, void *dC, float *dD, void *dz,
                  float *dh0, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                  int io_dtype, void *workspace, size_t workspace_bytes, void *stream,
                  const float *ckpt, bool ckpt_given) {
    if (int r = check_dtype(io_dtype)) return r;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 1 || d_state > SSM_MAX_D_STATE)
        return SSM_ERR_SHAPE;
    if (batch > kMaxGridY) return SSM_ERR_SHAPE;
    const size_t es = io_size(io_dtype);
    const int64_t n_btd = mul3(batch, seqlen, d_inner), n_btn = mul3(batch, seqlen, d_state);
    const int64_t n_bdn = mul3(batch, d_inner, d_state), n_dn = mul3(d_inner, d_state, 1);
    if (n_btd < 0 || n_btn < 0 || n_bdn < 0 || n_dn < 0) return SSM_ERR_SHAPE;
    // one batch row of x (seqlen x d_inner) and of B (seqlen x d_state) is
    // addressed with 32-bit byte offsets
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (mul3(seqlen, d_inner, static_cast<int64_t>(es)) > lim ||
        mul3(seqlen, d_state, static_cast<int64_t>(es)) > lim)
        return SSM_ERR_SHAPE;
    // and the checkpoints of one block (d_inner x d_state fp32)
    if (mul3(d_inner, d_state, 4) > lim) return SSM_ERR_SHAPE;
    // required pointers, for whatever this shape reads or writes
    if (n_dn > 0 && (!A || !dA)) return SSM_ERR_NULL;
    if (n_btd > 0 && (!x || !delta || !dout || !dx || !ddelta)) return SSM_ERR_NULL;
    if (n_btd > 0 && z && !dz) return SSM_ERR_NULL;
    if (n_btn > 0 && (!B || !C || !dB || !dC)) return SSM_ERR_NULL;
    const int64_t n_ck = mul3(mul3(batch, (seqlen + 15) / 16, d_inner), d_state, 1);
    if (n_ck < 0) return SSM_ERR_SHAPE;
    if (ckpt_given && n_btd > 0 && !ckpt) return SSM_ERR_NULL;
    if (ckpt && !aligned(ckpt, 16)) return SSM_ERR_ALIGN;
    const void *io_ptrs[] = {x, delta, B, C, z, dout, dx, ddelta, dB, dC, dz};
    for (const void *p : io_ptrs)
        if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
    const void *f_ptrs[] = {delta_bias, A, D, h0, dlast, ddelta_bias, dA, dD, dh0};
    for (const void *p : f_ptrs)
        if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
    const Range ins[] = {range(x, n_btd, es),         range(delta, n_btd, es),
                         range(z, n_btd, es),         range(dout, n_btd, es),
                         range(B, n_btn, es),         range(C, n_btn, es),
                         range(A, n_dn, 4),           range(D, d_inner, 4),
                         range(delta_bias, d_inner, 4), range(h0, n_bdn, 4),
                         range(dlast, n_bdn, 4),      range(ckpt, n_ck, 4)};
    const Range outs[] = {range(dx, n_btd, es),        range(ddelta, n_btd, es),
                          range(z ? dz : nullptr, n_btd, es), range(dB, n_btn, es),
                          range(dC, n_btn, es),        range(dA, n_dn, 4),
                          range(D ? dD : nullptr, d_inner, 4),
                          range(delta_bias ? ddelta_bias : nullptr, d_inner, 4),
                          range(dh0, n_bdn, 4)};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlap(o, i)) return SSM_ERR_ALIAS;
    constexpr int n_out = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < n_out; ++i)
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(outs[i], outs[j])) return SSM_ERR_ALIAS;
    if (batch == 0 && d_inner == 0) return SSM_OK;
    const size_t need = ssm::scan_bwd_workspace(batch, seqlen, d_inner, d_state, io_dtype == SSM_BF16);
    if (need && (!workspace || workspace_bytes < need)) return SSM_ERR_WORKSPACE;
    if (need && !aligned(workspace, 256)) return SSM_ERR_ALIGN;
    ssm::BwdArgs a;
    a.x = x; a.delta = delta; a.z = z; a.B = B; a.C = C; a.dout = dout;
    a.delta_bias = delta_bias; a.A = A; a.D = D; a.h0 = h0; a.dlast = dlast;
    a.dx = dx; a.ddelta = ddelta; a.dz = z ? dz : nullptr; a.dB = dB; a.dC = dC;
    a.dA = dA; a.dD = D ? dD : nullptr; a.ddelta_bias = delta_bias ? ddelta_bias : nullptr;
    a.dh0 = dh0;
    a.batch = batch; a.seqlen = seqlen; a.dim = d_inner; a.dstate = d_state;
    a.softplus = delta_softplus ? 1 : 0;
    a.bf16 = io_dtype == SSM_BF16 ? 1 : 0;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.ckpt_in = ckpt;
    return hip_status(ssm::launch_scan_bwd(a, static_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" {

int ssm_scan_bwd(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                 const float *A, const void *B, const void *C, const float *D, const void *z,
                 const float *h0, const void *dout, const float *dlast, void *dx, void *ddelta,
                 float *ddelta_bias, float *dA, void *dB, void *dC, float *dD, void *dz,
                 float *dh0, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                 int io_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return scan_bwd_impl(x, delta, delta_bias, delta_softplus, A, B, C, D, z, h0, dout, dlast, dx, ddelta,
                         ddelta_bias, dA, dB, dC, dD, dz, dh0, batch, seqlen, d_inner, d_state, io_dtype,
                         workspace, workspace_bytes, stream, nullptr, false);
}

int ssm_scan_bwd_ckpt(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                      const float *A, const void *B, const void *C, const float *D, const void *z,
                      const float *h0, const void *dout, const float *dlast, const float *ckpt, void *dx,
                      void *ddelta, float *ddelta_bias, float *dA, void *dB, void *dC, float *dD, void *dz,
                      float *dh0, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                      int io_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return scan_bwd_impl(x, delta, delta_bias, delta_softplus, A, B, C, D, z, h0, dout, dlast, dx, ddelta,
                         ddelta_bias, dA, dB, dC, dD, dz, dh0, batch, seqlen, d_inner, d_state, io_dtype,
                         workspace, workspace_bytes, stream, ckpt, true);
}

size_t ssm_scan_ckpt_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 1 || d_state > SSM_MAX_D_STATE)
        return static_cast<size_t>(-1);
    const int64_t n = mul3(mul3(batch, (seqlen + 15) / 16, d_inner), d_state, 4);
    return n < 0 ? static_cast<size_t>(-1) : static_cast<size_t>(n);
}

int ssm_scan_fwd_ckpt(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                      const float *A, const void *B, const void *C, const float *D, const void *z,
                      const float *h0, void *y, float *last_state, float *ckpt, int64_t batch,
                      int64_t seqlen, int64_t d_inner, int64_t d_state, int io_dtype, void *workspace,
                      size_t workspace_bytes, void *stream) {
    int r = validate_scan(x, delta, delta_bias, A, B, C, D, z, h0, y, last_state, batch, seqlen,
                          d_inner, d_state, io_dtype);
    if (r) return r;
    if (batch == 0 || d_inner == 0) return SSM_OK;
    const int64_t n_ck = mul3(mul3(batch, (seqlen + 15) / 16, d_inner), d_state, 1);
    if (n_ck < 0) return SSM_ERR_SHAPE;
    if (n_ck > 0 && !ckpt) return SSM_ERR_NULL;
    if (ckpt && !aligned(ckpt, 16)) return SSM_ERR_ALIGN;
    const size_t es = io_size(io_dtype);
    const int64_t n_btd = mul3(batch, seqlen, d_inner), n_btn = mul3(batch, seqlen, d_state);
    const int64_t n_bdn = mul3(batch, d_inner, d_state);
    const Range ck = range(ckpt, n_ck, 4);
    const Range others[] = {range(x, n_btd, es),  range(delta, n_btd, es), range(z, n_btd, es),
                            range(B, n_btn, es),  range(C, n_btn, es),     range(A, d_inner * d_state, 4),
                            range(D, d_inner, 4), range(delta_bias, d_inner, 4), range(h0, n_bdn, 4),
                            range(y, seqlen > 0 ? n_btd : 0, es), range(last_state, n_bdn, 4)};
    for (const Range &o : others)
        if (overlap(ck, o)) return SSM_ERR_ALIAS;
    ssm::ScanArgs a = make_args(x, delta, delta_bias, delta_softplus, A, B, C, D, z, h0, y,
                                last_state, batch, seqlen, d_inner, d_state, io_dtype, workspace,
                                workspace_bytes);
    a.ckpt = ckpt;
    const size_t need = ssm::scan_fwd_workspace(a);
    if (need && (!workspace || workspace_bytes < need)) return SSM_ERR_WORKSPACE;
    if (need && !aligned(workspace, 256)) return SSM_ERR_ALIGN;
    return hip_status(ssm::launch_scan_fwd_ckpt(a, static_cast<hipStream_t>(stream)));
}

size_t ssm_scan_2d_workspace_bytes(int64_t batch, int64_t height, int64_t width, int64_t d_inner,
                                   int64_t d_state, int direction, int has_z, int io_dtype) {
    if (check_dtype(io_dtype) || batch < 0 || height < 0 || width < 0 || d_inner < 0 || d_state < 1 ||
        d_state > SSM_MAX_D_STATE || direction < 0 || direction > 3)
        return static_cast<size_t>(-1);
    const int64_t L = mul3(height, width, 1);
    if (L < 0) return static_cast<size_t>(-1);
    ssm::ScanArgs a = make_args(nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr, nullptr, batch, L, d_inner, d_state,
                                io_dtype, nullptr, 0);
    return ssm::scan_2d_workspace(a, has_z != 0, direction, height, width);
}

int ssm_scan_fwd_2d(const void *x, const void *delta, const float *delta_bias, int delta_softplus,
                    const float *A, const void *B, const void *C, const float *D, const void *z,
                    const float *h0, void *y, float *last_state, int64_t batch, int64_t height,
                    int64_t width, int64_t d_inner, int64_t d_state, int direction, int io_dtype,
                    void *workspace, size_t workspace_bytes, void *stream) {
    if (direction < 0 || direction > 3) return SSM_ERR_SHAPE;
    if (height < 0 || width < 0) return SSM_ERR_SHAPE;
    const int64_t L = mul3(height, width, 1);
    if (L < 0) return SSM_ERR_SHAPE;
    int r = validate_scan(x, delta, delta_bias, A, B, C, D, z, h0, y, last_state, batch, L, d_inner,
                          d_state, io_dtype);
    if (r) return r;
    if (batch == 0 || d_inner == 0) return SSM_OK;
    ssm::ScanArgs a = make_args(x, delta, delta_bias, delta_softplus, A, B, C, D, z, h0, y,
                                last_state, batch, L, d_inner, d_state, io_dtype, workspace,
                                workspace_bytes);
    const size_t need = ssm::scan_2d_workspace(a, z != nullptr, direction, height, width);
    if (need && (!workspace || workspace_bytes < need)) return SSM_ERR_WORKSPACE;
    if (need && !aligned(workspace, 256)) return SSM_ERR_ALIGN;
    return hip_status(ssm::launch_scan_2d(a, height, width, direction, static_cast<hipStream_t>(stream)));
}

int ssm_causal_conv1d_fwd(const void *x, const float *weight, const float *bias,
                          const void *conv_state_in, void *out, void *conv_state_out,
                          int apply_silu, int64_t batch, int64_t seqlen, int64_t d_inner,
                          int64_t width, int io_dtype, void *stream) {
    if (int r = check_dtype(io_dtype)) return r;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || width < 1 || width > SSM_MAX_CONV_WIDTH)
        return SSM_ERR_SHAPE;
    if (batch > kMaxGridY) return SSM_ERR_SHAPE;
    const size_t es = io_size(io_dtype);
    const int64_t n_btd = mul3(batch, seqlen, d_inner), n_bdh = mul3(batch, d_inner, width - 1);
    if (n_btd < 0 || n_bdh < 0) return SSM_ERR_SHAPE;
    if (mul3(seqlen, d_inner, static_cast<int64_t>(es)) > (int64_t(1) << 31) - 1) return SSM_ERR_SHAPE;
    if (batch == 0 || d_inner == 0) return SSM_OK;
    if (!weight) return SSM_ERR_NULL;
    if (n_btd > 0 && (!x || !out)) return SSM_ERR_NULL;
    const void *io_ptrs[] = {x, out, conv_state_in, conv_state_out};
    for (const void *p : io_ptrs)
        if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
    if (!aligned(weight, 4) || (bias && !aligned(bias, 4))) return SSM_ERR_ALIGN;
    const Range ins[] = {range(x, n_btd, es), range(weight, d_inner * width, 4), range(bias, d_inner, 4),
                         range(conv_state_in, n_bdh, es)};
    const Range outs[] = {range(out, n_btd, es), range(conv_state_out, n_bdh, es)};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlap(o, i)) return SSM_ERR_ALIAS;
    if (overlap(outs[0], outs[1])) return SSM_ERR_ALIAS;
    ssm::ConvArgs a;
    a.x = x; a.weight = weight; a.bias = bias; a.state_in = conv_state_in;
    a.out = out; a.state_out = conv_state_out;
    a.batch = batch; a.seqlen = seqlen; a.dim = d_inner;
    a.width = static_cast<int>(width); a.silu = apply_silu ? 1 : 0;
    a.bf16 = io_dtype == SSM_BF16 ? 1 : 0;
    return hip_status(ssm::launch_conv1d(a, static_cast<hipStream_t>(stream)));
}

int ssm_dt_proj(const void *xdt, int64_t ldx, const void *W, void *delta, int64_t rows,
                int64_t rank, int64_t d_inner, int io_dtype, void *stream) {
    if (int r = check_dtype(io_dtype)) return r;
    const int64_t pe = io_dtype == SSM_BF16 ? 8 : 4;   // elements per 16-byte piece
    if (rows < 0 || d_inner < 0 || rank < 1 || ldx < rank) return SSM_ERR_SHAPE;
    if (rank % pe || ldx % pe || d_inner % 4) return SSM_ERR_SHAPE;
    const int64_t n_x = mul3(rows, ldx, 1), n_w = mul3(d_inner, rank, 1), n_o = mul3(rows, d_inner, 1);
    if (n_x < 0 || n_w < 0 || n_o < 0) return SSM_ERR_SHAPE;
    // one workgroup per 128 x 128 tile of delta, numbered in 32 bits
    if (mul3((rows + 127) / 128, (d_inner + 127) / 128, 1) > (int64_t(1) << 31) - 1) return SSM_ERR_SHAPE;
    if (rows == 0 || d_inner == 0) return SSM_OK;
    if (!xdt || !W || !delta) return SSM_ERR_NULL;
    if (!aligned(xdt, 16) || !aligned(W, 16) || !aligned(delta, 16)) return SSM_ERR_ALIGN;
    const size_t es = io_size(io_dtype);
    const Range o = range(delta, n_o, es);
    if (overlap(o, range(xdt, n_x, es)) || overlap(o, range(W, n_w, es))) return SSM_ERR_ALIAS;
    ssm::DtProjArgs a;
    a.xdt = xdt; a.W = W; a.out = delta;
    a.rows = rows; a.rank = rank; a.dim = d_inner; a.ldx = ldx;
    a.bf16 = io_dtype == SSM_BF16 ? 1 : 0;
    return hip_status(ssm::launch_dt_proj(a, static_cast<hipStream_t>(stream)));
}

int ssm_causal_conv1d_update(void *conv_state, const void *x, const float *weight,
                             const float *bias, void *out, int apply_silu, int64_t batch,
                             int64_t d_inner, int64_t width, int io_dtype, void *stream) {
    if (int r = check_dtype(io_dtype)) return r;
    if (batch < 0 || d_inner < 0 || width < 1 || width > SSM_MAX_CONV_WIDTH) return SSM_ERR_SHAPE;
    const size_t es = io_size(io_dtype);
    const int64_t n_bd = mul3(batch, d_inner, 1), n_bdh = mul3(batch, d_inner, width - 1);
    if (n_bd < 0 || n_bdh < 0 || n_bd >= (int64_t(1) << 31)) return SSM_ERR_SHAPE;
    if (batch == 0 || d_inner == 0) return SSM_OK;
    if (!x || !weight || !out || (width > 1 && !conv_state)) return SSM_ERR_NULL;
    const void *io_ptrs[] = {x, out, conv_state};
    for (const void *p : io_ptrs)
        if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
    if (!aligned(weight, 4) || (bias && !aligned(bias, 4))) return SSM_ERR_ALIGN;
    const Range ins[] = {range(x, n_bd, es), range(weight, d_inner * width, 4), range(bias, d_inner, 4)};
    const Range outs[] = {range(out, n_bd, es), range(conv_state, n_bdh, es)};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlap(o, i)) return SSM_ERR_ALIAS;
    if (overlap(outs[0], outs[1])) return SSM_ERR_ALIAS;
    ssm::ConvUpdateArgs a;
    a.state = conv_state; a.x = x; a.weight = weight; a.bias = bias; a.out = out;
    a.batch = batch; a.dim = d_inner;
    a.width = static_cast<int>(width); a.silu = apply_silu ? 1 : 0;
    a.bf16 = io_dtype == SSM_BF16 ? 1 : 0;
    return hip_status(ssm::launch_conv1d_update(a, static_cast<hipStream_t>(stream)));
}

namespace {
// the shape checks of ssd_scan_fwd (and its workspace and plan queries)
int check_ssd_shape(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                    int io_dtype) {
    if (int r = check_dtype(io_dtype)) return r;
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 0) return SSM_ERR_SHAPE;
    if (!ssm::ssd_supported(headdim, dstate, io_dtype == SSM_BF16)) return SSM_ERR_SHAPE;
    const size_t es = io_size(io_dtype);
    const int64_t hp = mul3(nheads, headdim, 1);
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (hp < 0 || mul3(batch, seqlen, hp) < 0 || mul3(batch, hp, dstate) < 0) return SSM_ERR_SHAPE;
    if (mul3(seqlen + 128, hp, es) > lim || mul3(seqlen + 128, dstate, es) > lim ||
        mul3(seqlen + 128, nheads, es) > lim)
        return SSM_ERR_SHAPE;
    if (mul3(batch, hp / 16, 1) > lim) return SSM_ERR_SHAPE;
    return SSM_OK;
}
}  // namespace

size_t ssd_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                int64_t dstate, int io_dtype) {
    if (check_ssd_shape(batch, seqlen, nheads, headdim, dstate, io_dtype)) return static_cast<size_t>(-1);
    return ssm::ssd_workspace(batch, seqlen, nheads, headdim, dstate, io_dtype == SSM_BF16);
}

int ssd_scan_fwd(const void *x, const void *dt, const float *dt_bias, int dt_softplus,
                 const float *A, const void *B, const void *C, const float *D, const void *z,
                 const float *h0, void *y, float *last_state, int64_t batch, int64_t seqlen,
                 int64_t nheads, int64_t headdim, int64_t dstate, int io_dtype, void *workspace,
                 size_t workspace_bytes, void *stream) {
    if (int r = check_dtype(io_dtype)) return r;
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 0) return SSM_ERR_SHAPE;
    if (!ssm::ssd_supported(headdim, dstate, io_dtype == SSM_BF16)) return SSM_ERR_SHAPE;
    const size_t es = io_size(io_dtype);
    const int64_t hp = mul3(nheads, headdim, 1);
    const int64_t n_bthp = mul3(batch, seqlen, hp < 0 ? -1 : hp);
    const int64_t n_bth = mul3(batch, seqlen, nheads);
    const int64_t n_btn = mul3(batch, seqlen, dstate);
    const int64_t n_bhpn = mul3(batch, hp < 0 ? -1 : hp, dstate);
    if (hp < 0 || n_bthp < 0 || n_bth < 0 || n_btn < 0 || n_bhpn < 0) return SSM_ERR_SHAPE;
    // 32-bit byte offsets within one batch row, including the chunk fetched past the end
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (mul3(seqlen + 128, hp, es) > lim || mul3(seqlen + 128, dstate, es) > lim ||
        mul3(seqlen + 128, nheads, es) > lim)
        return SSM_ERR_SHAPE;
    if (mul3(batch, hp / 16, 1) > lim) return SSM_ERR_SHAPE;      // workgroups (1-D grid)
    if (batch == 0 || nheads == 0) return SSM_OK;
    if (!A) return SSM_ERR_NULL;
    if (seqlen > 0 && (!x || !dt || !B || !C || !y)) return SSM_ERR_NULL;
    const void *v16[] = {x, z, y, B, C, h0, last_state};
    for (const void *p : v16)
        if (p && !aligned(p, 16)) return SSM_ERR_ALIGN;
    if (dt && !aligned(dt, es)) return SSM_ERR_ALIGN;
    const void *f_ptrs[] = {dt_bias, A, D};
    for (const void *p : f_ptrs)
        if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
    const Range outs[] = {range(y, seqlen > 0 ? n_bthp : 0, es), range(last_state, n_bhpn, 4)};
    const Range ins[] = {range(x, n_bthp, es), range(dt, n_bth, es),    range(z, n_bthp, es),
                         range(B, n_btn, es),  range(C, n_btn, es),     range(A, nheads, 4),
                         range(D, nheads, 4),  range(dt_bias, nheads, 4), range(h0, n_bhpn, 4)};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlap(o, i)) return SSM_ERR_ALIAS;
    if (overlap(outs[0], outs[1])) return SSM_ERR_ALIAS;
    const size_t need = ssm::ssd_workspace(batch, seqlen, nheads, headdim, dstate, io_dtype == SSM_BF16);
    if (need && (!workspace || workspace_bytes < need)) return SSM_ERR_WORKSPACE;
    if (need && !aligned(workspace, 256)) return SSM_ERR_ALIGN;
    if (need) {
        const Range wsr = range(workspace, static_cast<int64_t>(need), 1);
        for (const Range &o : outs)
            if (overlap(o, wsr)) return SSM_ERR_ALIAS;
        for (const Range &i : ins)
            if (overlap(i, wsr)) return SSM_ERR_ALIAS;
    }
    ssm::SsdArgs a;
    a.x = x; a.dt = dt; a.z = z; a.B = B; a.C = C;
    a.dt_bias = dt_bias; a.A = A; a.D = D; a.h0 = h0;
    a.y = y; a.last_state = last_state;
    a.batch = batch; a.seqlen = seqlen; a.nheads = nheads; a.headdim = headdim; a.dstate = dstate;
    a.softplus = dt_softplus ? 1 : 0;
    a.bf16 = io_dtype == SSM_BF16 ? 1 : 0;
    a.workspace = need ? workspace : nullptr;
    a.workspace_bytes = need ? workspace_bytes : 0;
    return hip_status(ssm::launch_ssd_scan(a, static_cast<hipStream_t>(stream)));
}

int ssm_scan_status(const void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace) return SSM_ERR_NULL;
    if (workspace_bytes < 256) return SSM_ERR_WORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t word = 0;
    if (hipStreamSynchronize(s) != hipSuccess) return SSM_ERR_HIP;
    if (hipMemcpy(&word, static_cast<const char *>(workspace) + ssm::kErrorWordOffset, sizeof(word),
                  hipMemcpyDeviceToHost) != hipSuccess)
        return SSM_ERR_HIP;
    return word ? SSM_ERR_WAIT : SSM_OK;
}

int ssm_testing_scan_fwd_no_handoff(const void *x, const void *delta, const float *delta_bias,
                                    int delta_softplus, const float *A, const void *B, const void *C,
                                    const float *D, const void *z, const float *h0, void *y,
                                    float *last_state, int64_t batch, int64_t seqlen, int64_t d_inner,
                                    int64_t d_state, int io_dtype, void *workspace, size_t workspace_bytes,
                                    uint32_t spin_limit, void *stream) {
    if (spin_limit == 0 || spin_limit > (1u << 16)) return SSM_ERR_SHAPE;
    int r = validate_scan(x, delta, delta_bias, A, B, C, D, z, h0, y, last_state, batch, seqlen,
                          d_inner, d_state, io_dtype);
    if (r) return r;
    if (batch == 0 || d_inner == 0) return SSM_OK;
    ssm::ScanArgs a = make_args(x, delta, delta_bias, delta_softplus, A, B, C, D, z, h0, y,
                                last_state, batch, seqlen, d_inner, d_state, io_dtype, workspace,
                                workspace_bytes);
    a.test_spin_limit = spin_limit;
    const size_t need = ssm::scan_fwd_workspace(a);
    if (need && (!workspace || workspace_bytes < need)) return SSM_ERR_WORKSPACE;
    if (need && !aligned(workspace, 256)) return SSM_ERR_ALIGN;
    return hip_status(ssm::launch_scan_fwd(a, static_cast<hipStream_t>(stream)));
}

int ssm_testing_ssd_segments(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                             int64_t dstate, int io_dtype, int *segments, int *chunks_per_segment) {
    if (!segments || !chunks_per_segment) return SSM_ERR_NULL;
    if (int r = check_ssd_shape(batch, seqlen, nheads, headdim, dstate, io_dtype)) return r;
    ssm::ssd_plan(batch, seqlen, nheads, headdim, dstate, io_dtype == SSM_BF16, segments, chunks_per_segment);
    return SSM_OK;
}

int ssm_testing_bwd_segments(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                             int io_dtype, int *segments, int *blocks_per_segment) {
    if (!segments || !blocks_per_segment) return SSM_ERR_NULL;
    if (check_dtype(io_dtype)) return SSM_ERR_DTYPE;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 1 || d_state > SSM_MAX_D_STATE)
        return SSM_ERR_SHAPE;
    ssm::scan_bwd_plan(batch, seqlen, d_inner, d_state, io_dtype == SSM_BF16, segments, blocks_per_segment);
    return SSM_OK;
}

}  // extern "C"
