// The 2-D scan of the youngju.dev guide's VMamba section (section 9, image
// processing): a batch of height x width patches (row-major along the
// sequence axis) is scanned in one of four orders -- row-major, its reverse,
// column-major (the patch grid transposed), its reverse -- and y comes back
// at each patch's own position.
//
// Row-major order is the forward scan as stored.  At d_state 16 the row
// kernel visits the other three in place: the reversed order read backwards,
// the column-major orders with each step's patch row computed in the kernel
// (sequences below 2^23 steps whose batch row spans under 2 GiB).  The
// remaining cases (other d_state, larger grids) permute the sequence axis:
//   gather x, delta, z, B, C into scan order (permute_rows_kernel),
//   the forward scan of this library on the gathered tensors,
//   scatter y back to the patches' positions (the same kernel, inverse map).
// The permutation kernels move whole rows (d_inner or d_state elements of one
// step) with 16-byte accesses where the row allows; they are HBM-bound copies.
#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

// Row-major patch index of scan step s (0 <= s < H W).
__device__ __forceinline__ int64_t patch_of_step(int64_t s, int64_t H, int64_t W, int dir) {
    const int64_t L = H * W;
    const int64_t q = (dir & 1) ? L - 1 - s : s;      // the reversed orders walk backwards
    if (dir < 2) return q;                            // row-major
    const int64_t wi = q / H, hi = q - wi * H;        // column-major: q = w H + h
    return hi * W + wi;
}

// dst row s = src row patch_of_step(s) (gather), or dst row patch_of_step(s)
// = src row s (scatter); rows of row_bytes bytes, copied in 16-, 4- or 2-byte
// units (the largest dividing the row and the pointers).
template <typename U>
__global__ __launch_bounds__(256) void permute_rows_kernel(const void *src, void *dst, int64_t batch, int64_t H,
                                                           int64_t W, int dir, int64_t row_units, int scatter) {
    const int64_t L = H * W;
    const int64_t total = batch * L * row_units;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total; i += stride) {
        const int64_t u = i % row_units, r = i / row_units;
        const int64_t s = r % L, b = r / L;
        const int64_t p = patch_of_step(s, H, W, dir);
        const int64_t from = scatter ? r : b * L + p;
        const int64_t to = scatter ? b * L + p : r;
        static_cast<U *>(dst)[to * row_units + u] = static_cast<const U *>(src)[from * row_units + u];
    }
}

hipError_t permute(const void *src, void *dst, int64_t batch, int64_t H, int64_t W, int dir, int64_t row_bytes,
                   bool scatter, hipStream_t s) {
    const int64_t total_bytes = batch * H * W * row_bytes;
    if (total_bytes == 0) return hipSuccess;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
    int64_t unit = 2;
    if (row_bytes % 16 == 0 && a % 16 == 0) unit = 16;
    else if (row_bytes % 4 == 0 && a % 4 == 0) unit = 4;
    const int64_t n = total_bytes / unit;
    const int64_t blocks = (n + 255) / 256;
    const dim3 grid(static_cast<unsigned>(blocks < 65536 ? blocks : 65536));
    const int64_t ru = row_bytes / unit;
    const int sc = scatter ? 1 : 0;
    if (unit == 16)
        hipLaunchKernelGGL(permute_rows_kernel<uint4>, grid, dim3(256), 0, s, src, dst, batch, H, W, dir, ru, sc);
    else if (unit == 4)
        hipLaunchKernelGGL(permute_rows_kernel<uint32_t>, grid, dim3(256), 0, s, src, dst, batch, H, W, dir, ru, sc);
    else
        hipLaunchKernelGGL(permute_rows_kernel<uint16_t>, grid, dim3(256), 0, s, src, dst, batch, H, W, dir, ru, sc);
    return hipGetLastError();
}

// a grid of one row or one column is visited column-major in row-major order
int effective_direction(int direction, int64_t height, int64_t width) {
    return (direction >= 2 && (height == 1 || width == 1)) ? direction - 2 : direction;
}
// orders the scan kernels visit without a gathered copy
bool visits_in_place(const ScanArgs &a, int direction) {
    const size_t esz = a.bf16 ? 2 : 4;
    return direction == 0 ||
           (a.dstate == 16 && (direction == 1 || (a.seqlen < (int64_t(1) << 23) &&
                                                  size_t(a.seqlen) * a.dim * esz < (size_t(1) << 31))));
}

struct Scan2dLayout {
    size_t fwd_bytes, x_off, d_off, z_off, b_off, c_off, y_off, total;
};
size_t up256(size_t v) { return (v + 255) & ~size_t(255); }
Scan2dLayout scan2d_layout(const ScanArgs &a, bool has_z, bool in_place) {
    const size_t es = a.bf16 ? 2 : 4;
    const size_t btd = size_t(a.batch) * a.seqlen * a.dim * es, btn = size_t(a.batch) * a.seqlen * a.dstate * es;
    Scan2dLayout l;
    l.fwd_bytes = scan_fwd_workspace(a);
    size_t o = up256(l.fwd_bytes);
    if (in_place) {
        l.x_off = l.d_off = l.z_off = l.b_off = l.c_off = l.y_off = 0;
        l.total = l.fwd_bytes;
        return l;
    }
    l.x_off = o; o = up256(o + btd);
    l.d_off = o; o = up256(o + btd);
    l.z_off = o; o = up256(o + (has_z ? btd : 0));
    l.b_off = o; o = up256(o + btn);
    l.c_off = o; o = up256(o + btn);
    l.y_off = o; o = up256(o + btd);
    l.total = o;
    return l;
}

}  // namespace

size_t scan_2d_workspace(const ScanArgs &a, bool has_z, int direction, int64_t height, int64_t width) {
    return scan2d_layout(a, has_z, visits_in_place(a, effective_direction(direction, height, width))).total;
}

hipError_t launch_scan_2d(const ScanArgs &a, int64_t height, int64_t width, int direction, hipStream_t s) {
    if (a.batch == 0 || a.dim == 0) return hipSuccess;
    direction = effective_direction(direction, height, width);
    const bool in_place = visits_in_place(a, direction);
    const Scan2dLayout l = scan2d_layout(a, a.z != nullptr, in_place);
    char *ws = static_cast<char *>(a.workspace);
    if (in_place) {
        // row-major: the sequence as stored, or read backwards; column-major at
        // d_state 16: the kernel computes each step's patch row itself
        ScanArgs f = a;
        f.reverse = direction & 1;
        f.column_major = direction >= 2;
        f.grid_h = height; f.grid_w = width;
        f.workspace = ws; f.workspace_bytes = l.fwd_bytes;
        return launch_scan_fwd(f, s);
    }
    const size_t es = a.bf16 ? 2 : 4;
    const int64_t rd = a.dim * es, rn = a.dstate * es;
    ScanArgs f = a;
    f.x = ws + l.x_off; f.delta = ws + l.d_off; f.z = a.z ? ws + l.z_off : nullptr;
    f.B = ws + l.b_off; f.C = ws + l.c_off; f.y = ws + l.y_off;
    f.workspace = ws; f.workspace_bytes = l.fwd_bytes;
    hipError_t e;
    if ((e = permute(a.x, const_cast<void *>(f.x), a.batch, height, width, direction, rd, false, s))) return e;
    if ((e = permute(a.delta, const_cast<void *>(f.delta), a.batch, height, width, direction, rd, false, s))) return e;
    if (a.z && (e = permute(a.z, const_cast<void *>(f.z), a.batch, height, width, direction, rd, false, s))) return e;
    if ((e = permute(a.B, const_cast<void *>(f.B), a.batch, height, width, direction, rn, false, s))) return e;
    if ((e = permute(a.C, const_cast<void *>(f.C), a.batch, height, width, direction, rn, false, s))) return e;
    if ((e = launch_scan_fwd(f, s))) return e;
    return permute(f.y, a.y, a.batch, height, width, direction, rd, true, s);
}

}  // namespace ssm
