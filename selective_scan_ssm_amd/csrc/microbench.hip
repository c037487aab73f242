// libssmbench.so (include/ssm_bench.h): measurement helpers behind the
// benchmark's roofline figures -- the copy bandwidth a 16-byte streaming
// kernel reaches on this HBM, and the issue rate of the fp32 VALU operations
// the scans are built from (fma, and the v_exp_f32 behind every decay
// factor).  They are not part of any scan and live in a library of their own,
// apart from the scan library's C ABI.
#include "ssm_bench.h"

#include <cstdint>

#include "ssm_device.h"

namespace ssm {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// grid-stride copy of n16 16-byte words, non-temporal loads and stores
__global__ __launch_bounds__(256) void mb_copy_kernel(const void *src, void *dst, uint64_t n16) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * 256;
    const u32x4_t *s = static_cast<const u32x4_t *>(src);
    u32x4_t *d = static_cast<u32x4_t *>(dst);
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

// 8 independent chains of one op per lane, `iters` steps each; the chains
// stay bounded (fma: x <- 0.999 x + 0.001; exp2: x <- 2^-x, fixed point
// ~0.64; log2: x <- log2(x + 2) in [1, 2]; rcp: x <- 1 / (x + 1) in [0.5, 1])
template <int OP>
__global__ __launch_bounds__(256) void mb_valu_kernel(float *out, int64_t iters) {
    float x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = 0.1f * static_cast<float>(c + 1) + 1e-6f * static_cast<float>(threadIdx.x);
#pragma unroll 8
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if constexpr (OP == 0) x[c] = fmaf(x[c], 0.999f, 0.001f);
            else if constexpr (OP == 1) x[c] = fast_exp2(-x[c]);
            else if constexpr (OP == 2) x[c] = fast_log2(x[c] + 2.0f);
            else x[c] = fast_rcp(x[c] + 1.0f);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) s += x[c];
    out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}

hipError_t launch_mb_copy(const void *src, void *dst, uint64_t bytes, hipStream_t s) {
    const uint64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    const uint64_t blocks = (n16 + 255) / 256;
    const unsigned grid = static_cast<unsigned>(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(mb_copy_kernel, dim3(grid), dim3(256), 0, s, src, dst, n16);
    return hipGetLastError();
}

hipError_t launch_mb_valu(int op, float *out, int64_t blocks, int64_t iters, hipStream_t s) {
    if (blocks == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks));
    switch (op) {
    case 0: hipLaunchKernelGGL(mb_valu_kernel<0>, grid, dim3(256), 0, s, out, iters); break;
    case 1: hipLaunchKernelGGL(mb_valu_kernel<1>, grid, dim3(256), 0, s, out, iters); break;
    case 2: hipLaunchKernelGGL(mb_valu_kernel<2>, grid, dim3(256), 0, s, out, iters); break;
    default: hipLaunchKernelGGL(mb_valu_kernel<3>, grid, dim3(256), 0, s, out, iters); break;
    }
    return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; }

}  // namespace
}  // namespace ssm

extern "C" {

int ssm_mb_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (bytes == 0) return SSM_MB_OK;
    if (!src || !dst) return SSM_MB_ERR_ARG;
    if (bytes % 16 != 0 || !ssm::aligned16(src) || !ssm::aligned16(dst)) return SSM_MB_ERR_ARG;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + bytes && b < a + bytes) return SSM_MB_ERR_ARG;
    return ssm::launch_mb_copy(src, dst, bytes, static_cast<hipStream_t>(stream)) == hipSuccess ? SSM_MB_OK
                                                                                               : SSM_MB_ERR_HIP;
}

int ssm_mb_valu(int op, float *out, int64_t blocks, int64_t iters, void *stream) {
    if (op < 0 || op > 3 || blocks < 0 || iters < 0 || blocks > (int64_t(1) << 31) - 1) return SSM_MB_ERR_ARG;
    if (blocks == 0) return SSM_MB_OK;
    if (!out || (reinterpret_cast<uintptr_t>(out) % 4) != 0) return SSM_MB_ERR_ARG;
    return ssm::launch_mb_valu(op, out, blocks, iters, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SSM_MB_OK
               : SSM_MB_ERR_HIP;
}

}  // extern "C"
