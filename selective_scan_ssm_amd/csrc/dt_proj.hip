// dt_proj on gfx950: the projection that produces the selective scan's delta
// input ("Mamba State Space Models complete guide" (youngju.dev), section 5,
// the MambaBlock of the complete implementation: a linear layer from
// dt_rank = d_model / 16 inputs to d_inner outputs, applied to the first
// dt_rank columns of each x_proj output row; its bias is the scan's
// delta_bias, added inside the softplus, so only the product is formed here):
//     delta[m, d] = sum_{k < rank} xdt[m * ldx + k] * W[d * rank + k]
//
// A dense contraction, so it runs on the matrix cores: v_mfma_f32_16x16x32_bf16
// for bf16 io, v_mfma_f32_16x16x4_f32 for fp32 io, fp32 accumulation, the
// result rounded once to the io dtype.  At the Mamba shapes the rank is small
// (48, 160) and the output (rows x d_inner) dominates the traffic, so the
// kernel is bound by writing delta to HBM; the operands are re-read from L2
// (W is 1.6 MB at the 2.8b layer, a 128-row slab of xdt 40 KB).
//
//   * A workgroup of 4 waves owns a 128 (rows) x 128 (channels) tile of
//     delta.  Blocks are renumbered so that the channel tiles of one row slab
//     run on one XCD: its xdt rows are then fetched into that XCD's L2 once,
//     and W is shared by all slabs.
//   * K is staged through LDS in chunks of 128 bytes per row (64 bf16 / 32
//     fp32): each thread copies 16-byte pieces of 4 W rows and 4 xdt rows;
//     pieces past the rank, the rows or the channels are zeros.  Rows are
//     padded by 16 bytes, so the 8 lanes of a 128-bit LDS read hit 8
//     distinct groups of 4 banks.
//   * Wave w computes a 64 x 64 sub-tile as 4 x 4 MFMA tiles.  W supplies the
//     A operand (rows = channels) and xdt the B operand (columns = rows of
//     delta), so each lane's four accumulator values are four consecutive
//     channels of one row of delta.
//   * The finished tile goes back through LDS (the K staging space, reused)
//     and leaves in whole rows: 16-byte pieces, eight lanes per 128-byte line,
//     so a store instruction covers full lines instead of 32-byte pieces of 16
//     rows (which HBM serves at a fraction of the rate).
#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTM = 128;    // rows of delta per workgroup
constexpr int kTD = 128;    // channels of delta per workgroup

template <typename T> struct DtOps;
template <> struct DtOps<bf16_t> {
    using E = uint16_t;                       // LDS element
    static constexpr int KB = 32, KPL = 8;    // K per MFMA, K per lane
    using frag = bf16x8_t;
    static __device__ __forceinline__ frag load(const E *p) {
        return __builtin_bit_cast(frag, *reinterpret_cast<const u16x8_t *>(p));
    }
    static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // four consecutive results, rounded to bf16, as one 8-byte store
    static __device__ __forceinline__ void store4(void *dst, f32x4_t v) {
        const u32x2_t q = {static_cast<uint32_t>(from_f32<bf16_t>(v[0]).bits) |
                               (static_cast<uint32_t>(from_f32<bf16_t>(v[1]).bits) << 16),
                           static_cast<uint32_t>(from_f32<bf16_t>(v[2]).bits) |
                               (static_cast<uint32_t>(from_f32<bf16_t>(v[3]).bits) << 16)};
        *reinterpret_cast<u32x2_t *>(dst) = q;
    }
};
template <> struct DtOps<float> {
    using E = float;
    static constexpr int KB = 4, KPL = 1;
    using frag = float;
    static __device__ __forceinline__ frag load(const E *p) { return *p; }
    static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ void store4(void *dst, f32x4_t v) { *reinterpret_cast<f32x4_t *>(dst) = v; }
};

template <typename T>
__global__ __launch_bounds__(256) void dt_proj_kernel(DtProjArgs a) {
    using O = DtOps<T>;
    using E = typename O::E;
    constexpr int es = sizeof(E);
    constexpr int PE = 16 / es;               // elements per 16-byte piece
    constexpr int KC = 128 / es;              // K elements per LDS chunk (128 bytes per row)
    constexpr int RS = KC + PE;               // LDS row stride: 16 bytes of padding
    // K staging (sW, sX), reused for the output tile once the products are done
    constexpr int OS = kTD + 32 / es;         // output row stride: 32 bytes of padding
    constexpr int kStageBytes = (kTD + kTM) * RS * es, kOutBytes = kTM * OS * es;
    __shared__ __attribute__((aligned(16))) char smem[kStageBytes > kOutBytes ? kStageBytes : kOutBytes];
    E *sW = reinterpret_cast<E *>(smem);
    E *sX = sW + kTD * RS;
    E *sO = reinterpret_cast<E *>(smem);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, kq = lane >> 4;
    const int wd = w & 1, wm = w >> 1;        // this wave's 64-channel / 64-row half
    const int64_t M = a.rows, R = a.rank, D = a.dim, ldx = a.ldx;
    // block -> tile: the hardware deals consecutive blocks out to the 8 XCDs
    // in turn, each XCD with its own L2; renumbering keeps the channel tiles
    // of one row slab (which share its xdt rows) on one XCD
    const int64_t ntd = (D + kTD - 1) / kTD;
    const int64_t total = static_cast<int64_t>(gridDim.x);
    int64_t lin = blockIdx.x;
    if (total % 8 == 0) lin = (lin % 8) * (total / 8) + lin / 8;
    const int64_t m0 = lin / ntd * kTM;
    const int64_t d0 = lin % ntd * kTD;
    const E *xdt = static_cast<const E *>(a.xdt);
    const E *W = static_cast<const E *>(a.W);

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // K chunk [k0, k0 + KC) of 128 W rows and 128 xdt rows: piece
    // q = tid + 256 i is row q / 8, 16-byte piece q % 8 (8 threads per row).
    u32x4_t vw[4], vx[4];
    auto fetch = [&](int64_t k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i;
            const int row = q >> 3, kp = (q & 7) * PE;
            const int64_t k = k0 + kp;
            vw[i] = u32x4_t{0u, 0u, 0u, 0u};
            vx[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (d0 + row < D && k < R) vw[i] = *reinterpret_cast<const u32x4_t *>(W + (d0 + row) * R + k);
            if (m0 + row < M && k < R) vx[i] = *reinterpret_cast<const u32x4_t *>(xdt + (m0 + row) * ldx + k);
        }
    };
    for (int64_t k0 = 0; k0 < R; k0 += KC) {
        fetch(k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i;
            const int row = q >> 3, kp = (q & 7) * PE;
            *reinterpret_cast<u32x4_t *>(&sW[row * RS + kp]) = vw[i];
            *reinterpret_cast<u32x4_t *>(&sX[row * RS + kp]) = vx[i];
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < KC / O::KB; ++ks) {
            typename O::frag fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[i] = O::load(&sW[(wd * 64 + i * 16 + l16) * RS + ks * O::KB + kq * O::KPL]);
                fb[i] = O::load(&sX[(wm * 64 + i * 16 + l16) * RS + ks * O::KB + kq * O::KPL]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = O::mma(fa[i], fb[j], acc[i][j]);
        }
        __syncthreads();
    }

    // lane: channels d .. d + 3 of row m of each 16 x 16 tile, into the tile
    // in LDS (the loop's last barrier freed the staging space)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int dl = wd * 64 + i * 16 + kq * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) O::store4(&sO[(wm * 64 + j * 16 + l16) * OS + dl], acc[i][j]);
    }
    __syncthreads();
    // whole rows out: piece q (16 bytes) is row q / PR, PE channels at (q % PR) PE
    constexpr int PR = kTD / PE;              // pieces per tile row
    char *out = static_cast<char *>(a.out);
    // rows start 16-byte aligned when d_inner is a multiple of a piece; else
    // (bf16, d_inner % 8 == 4) 8-byte aligned, and pieces go out in halves
    const bool whole = D % PE == 0;
#pragma unroll
    for (int q = tid; q < kTM * PR; q += 256) {
        const int row = q / PR, c = (q % PR) * PE;
        const int64_t m = m0 + row, d = d0 + c;
        if (m >= M || d >= D) continue;
        char *dst = out + (m * D + d) * static_cast<int64_t>(es);
        if (whole) {
            *reinterpret_cast<u32x4_t *>(dst) = *reinterpret_cast<const u32x4_t *>(&sO[row * OS + c]);
        } else {
            // 8-byte halves; d_inner % 4 == 0, so a half is whole or past the end
            for (int hh = 0; hh < PE && d + hh < D; hh += 8 / es)
                *reinterpret_cast<u32x2_t *>(dst + hh * es) = *reinterpret_cast<const u32x2_t *>(&sO[row * OS + c + hh]);
        }
    }
}

}  // namespace

hipError_t launch_dt_proj(const DtProjArgs &a, hipStream_t s) {
    if (a.rows == 0 || a.dim == 0) return hipSuccess;
    const int64_t blocks = ((a.rows + kTM - 1) / kTM) * ((a.dim + kTD - 1) / kTD);
    if (a.bf16)
        hipLaunchKernelGGL(dt_proj_kernel<bf16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(dt_proj_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ssm
