// Entry points of the forward scan (ssm_kernels.h): workspace sizes, the
// dispatch to the kernel shares of scan_rows_*.hip / scan_general_*.hip, and
// the fused prologue's launch sequence.
#include "scan_fwd_kernels.h"

namespace ssm {

size_t scan_fwd_workspace(const ScanArgs &a) {
    if (a.batch == 0 || a.dim == 0 || a.seqlen == 0) return 0;
    return make_layout(a.batch, a.seqlen, a.dim, a.dstate, (a.bf16 && !a.x_f32) ? 2 : 4).total;
}

size_t conv_scan_workspace(const ScanArgs &a) {
    if (a.batch == 0 || a.dim == 0 || a.seqlen == 0) return 0;
    if (rows_path(a.dstate)) return scan_fwd_workspace(a);
    // other widths: the filtered x, in fp32 (never rounded to the io dtype),
    // after the scan's own workspace
    ScanArgs f = a;
    f.x_f32 = 1;
    const size_t fwd = scan_fwd_workspace(f);
    return ((fwd + 255) & ~size_t(255)) + size_t(a.batch) * a.seqlen * a.dim * sizeof(float);
}

hipError_t launch_conv_scan_fwd(const ScanArgs &a, void *conv_state_out, hipStream_t s) {
    if (a.batch == 0 || a.dim == 0) return hipSuccess;
    ConvArgs c{};
    c.x = a.x; c.weight = a.conv_w; c.bias = a.conv_b; c.state_in = a.conv_state;
    c.state_out = conv_state_out;
    c.batch = a.batch; c.seqlen = a.seqlen; c.dim = a.dim;
    c.width = static_cast<int>(a.conv_k); c.silu = 1; c.bf16 = a.bf16;
    hipError_t e = hipSuccess;
    if (a.seqlen > 0) {
        if (rows_path(a.dstate)) {
            e = launch_scan_fwd(a, s);                  // one pass: the conv runs inside the scan
        } else {
            ScanArgs f = a;
            f.x_f32 = 1;
            f.conv_w = nullptr; f.conv_b = nullptr; f.conv_state = nullptr; f.conv_k = 0;
            const size_t fwd = scan_fwd_workspace(f);
            void *xc = static_cast<char *>(a.workspace) + ((fwd + 255) & ~size_t(255));
            c.out = xc;
            c.out_f32 = 1;                              // the filtered x stays fp32
            e = launch_conv1d(c, s);
            if (e != hipSuccess) return e;
            f.x = xc;
            e = launch_scan_fwd(f, s);
        }
    } else {
        e = launch_scan_fwd(a, s);                      // last_state = h0
    }
    if (e != hipSuccess) return e;
    return launch_conv_state_out(c, s);
}

hipError_t launch_scan_fwd(const ScanArgs &a, hipStream_t s) {
    if (a.batch == 0 || a.dim == 0) return hipSuccess;
    if (a.seqlen == 0) {
        if (!a.last_state) return hipSuccess;
        const int64_t n = a.batch * a.dim * a.dstate;
        hipLaunchKernelGGL(copy_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                           a.h0, a.last_state, n);
        return hipGetLastError();
    }
    if (a.workspace == nullptr || a.workspace_bytes < scan_fwd_workspace(a)) return hipErrorInvalidValue;
    if (rows_path(a.dstate)) {
        const bool in_order = !a.reverse && !a.column_major;
        if (a.bf16) return in_order ? scan_rows_main_bf16(a, s) : scan_rows_2d_bf16(a, s);
        return in_order ? scan_rows_main_f32(a, s) : scan_rows_2d_f32(a, s);
    }
    if (a.bf16) return a.x_f32 ? scan_general_bf16_xf32(a, s) : scan_general_bf16(a, s);
    return scan_general_f32(a, s);
}

}  // namespace ssm
