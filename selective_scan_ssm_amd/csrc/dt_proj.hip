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
//
// bf16 io with rank <= 160 (both Mamba shapes) runs dt_proj_rows_kernel
// instead, which keeps the store stream going:
//   * Persistent workgroups: workgroup i keeps the 128-channel slice
//     i mod (channel tiles) of W in LDS for its whole life (43 KB at rank 160)
//     and walks every nrep-th 128-row slab of delta.
//   * The xdt operand never passes through LDS: each lane loads its MFMA
//     fragment (8 consecutive k of one row) straight from global memory as one
//     16-byte load, and the fragments of the next slab are loaded as soon as
//     the current slab's k step has consumed the registers, so they arrive
//     during the rest of the slab's products and its stores.
//   * Two workgroups per CU (80 KB of LDS each): while one finishes a slab's
//     products, the other's whole-row stores of the previous slab drain.
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


// ---------------------------------------------------------------------------
// bf16, rank <= 32 NK: persistent, W resident, xdt fragments from global
constexpr int kDtPerCU = 2;                  // workgroups per CU (LDS <= 80 KB each)
constexpr int kDtCUs = 256;

// WHOLE: d_inner is a multiple of 8, so output rows are 16-byte aligned and
// leave in 16-byte pieces; else (d_inner % 8 == 4) in 8-byte halves.
//
// No memory operation sits behind a branch: the counter the waits use counts
// loads and stores in issue order, and a branch around either makes the
// compiler wait for everything in flight where the paths join.  The prefetch
// past the last slab reads through an empty descriptor, and stores out of the
// tile go to offsets outside their descriptor (both dropped).
template <int NK, bool WHOLE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kDtPerCU, kDtPerCU)))
void dt_proj_rows_kernel(DtProjArgs a) {
    using O = DtOps<bf16_t>;
    using E = uint16_t;
    constexpr int es = 2;
    constexpr int PE = 8;                     // elements per 16-byte piece
    constexpr int WS = 32 * NK + PE;          // LDS row stride of W (16 bytes of padding)
    constexpr int OS = kTD + 16;              // output row stride (32 bytes of padding)
    constexpr int PR = kTD / PE;              // output pieces per tile row
    constexpr int NQ = kTM * PR / 256;        // output pieces per thread and slab
    extern __shared__ __attribute__((aligned(16))) char dsmem[];
    E *sW = reinterpret_cast<E *>(dsmem);     // [kTD][WS]
    E *sO = sW + kTD * WS;                    // [kTM][OS]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // rows 32 w .. 32 w + 31 of the slab
    const int l16 = lane & 15, kq = lane >> 4;
    const int64_t M = a.rows, R = a.rank, D = a.dim, ldx = a.ldx;
    const int64_t ntd = (D + kTD - 1) / kTD, nslab = (M + kTM - 1) / kTM;
    const int64_t total = static_cast<int64_t>(gridDim.x);
    const int64_t nrep = total / ntd;         // slabs are dealt out nrep apart
    // consecutive workgroups (one row class, every channel tile) on one XCD:
    // a slab's xdt rows are then fetched into one L2
    int64_t lin = blockIdx.x;
    if (total % 8 == 0) lin = (lin % 8) * (total / 8) + lin / 8;
    const int64_t d0 = lin % ntd * kTD;
    const int64_t first = lin / ntd;
    const E *W = static_cast<const E *>(a.W);

    // W[d0 .. d0 + 128)[0 .. 32 NK) into LDS once; past the rank or d_inner: 0
    for (int q = tid; q < kTD * 4 * NK; q += 256) {
        const int row = q / (4 * NK), kp = (q % (4 * NK)) * PE;
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if (d0 + row < D && kp < R) v = *reinterpret_cast<const u32x4_t *>(W + (d0 + row) * R + kp);
        *reinterpret_cast<u32x4_t *>(&sW[row * WS + kp]) = v;
    }

    // the lane's xdt fragments of a slab: row 32 w + 16 j + l16, k = 32 ks + 8 kq
    // .. + 7, through a descriptor over the slab's rows (rows past the end,
    // pieces past the rank and slabs past the last read 0: the columns after
    // the rank hold B and C).  Two sets: the next slab's arrive during this
    // slab's products.
    O::frag bfr[2][NK][2];
    uint32_t boff[NK][2];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int k = 32 * ks + 8 * kq;
            boff[ks][j] = k < R ? static_cast<uint32_t>(((w * 32 + 16 * j + l16) * ldx + k) * es) : kOffNone;
        }
    auto slab_rsrc = [&](int64_t slab) __attribute__((always_inline)) {
        const int64_t m0 = slab * kTM;
        const int64_t nr = slab < nslab ? (M - m0 < kTM ? M - m0 : kTM) : 0;
        return make_rsrc(static_cast<const char *>(a.xdt) + (slab < nslab ? m0 * ldx * es : 0),
                         static_cast<uint32_t>(nr * ldx * es));
    };
    auto load_b = [&](const rsrc_t &rx, O::frag (&dst)[NK][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < NK; ++ks)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                dst[ks][j] = __builtin_bit_cast(O::frag, __builtin_amdgcn_raw_buffer_load_b128(rx, boff[ks][j], 0, 0));
    };
    // the thread's output pieces of a tile: piece q = tid + 256 i is row q / PR,
    // channels (q % PR) PE .. (the same column for every i: PR divides 256)
    static_assert(256 % PR == 0, "one column per thread");
    const int ocol = (tid % PR) * PE;
    const bool ovalid = d0 + ocol < D;
    char *out = static_cast<char *>(a.out);
    auto store_tile = [&](const rsrc_t &ro) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int row = (tid + 256 * i) / PR;
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(&sO[row * OS + ocol]);
            const uint32_t off = ovalid ? static_cast<uint32_t>((row * D + d0 + ocol) * es) : kOffNone;
            if constexpr (WHOLE) {
                __builtin_amdgcn_raw_buffer_store_b128(v, ro, off, 0, kStream);
            } else {
                // d_inner % 4 == 0: the upper half of the last piece of a row
                // is past d_inner exactly when d0 + ocol + 4 == d_inner
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v[0], v[1]}, ro, off, 0, kStream);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v[2], v[3]}, ro,
                                                      d0 + ocol + 4 < D ? off + 8 : kOffNone, 0, kStream);
            }
        }
    };
    auto out_rsrc = [&](int64_t slab) __attribute__((always_inline)) {
        const int64_t m0 = slab * kTM;
        const int64_t nr = M - m0 < kTM ? M - m0 : kTM;
        return make_rsrc(out + m0 * D * es, static_cast<uint32_t>(nr * D * es));
    };

    load_b(slab_rsrc(first), bfr[0]);
    // the stores a slab issues after its loads, dropped here: every way into
    // the loop has the same memory history
    store_tile(make_rsrc(out, 0u));
    __syncthreads();                          // W is in LDS

    // one slab from fragment set B: the next slab's fragments into set 1 - B
    // first, then the products, the tile through LDS and its stores
    auto slab_step = [&](int64_t slab, O::frag (&cur)[NK][2], O::frag (&nxt)[NK][2]) __attribute__((always_inline)) {
        load_b(slab_rsrc(slab + nrep), nxt);
        f32x4_t acc[8][2];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
            for (int ih = 0; ih < 2; ++ih) {      // the 128 channels in two halves of 4 tiles
                O::frag fa[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    fa[i] = O::load(&sW[(64 * ih + 16 * i + l16) * WS + 32 * ks + 8 * kq]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[4 * ih + i][j] = O::mma(fa[i], cur[ks][j], acc[4 * ih + i][j]);
            }
        }
        __syncthreads();                      // every wave is done reading the previous tile
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) O::store4(&sO[(32 * w + 16 * j + l16) * OS + 16 * i + 4 * kq], acc[i][j]);
        __syncthreads();
        store_tile(out_rsrc(slab));
    };
    for (int64_t slab = first; slab < nslab; slab += 2 * nrep) {
        slab_step(slab, bfr[0], bfr[1]);
        if (slab + nrep < nslab) slab_step(slab + nrep, bfr[1], bfr[0]);
    }
}

template <int NK> hipError_t launch_rows(const DtProjArgs &a, hipStream_t s) {
    constexpr int WS = 32 * NK + 8, OS = kTD + 16;
    constexpr size_t lds = (static_cast<size_t>(kTD) * WS + static_cast<size_t>(kTM) * OS) * 2;
    static_assert(lds <= 160 * 1024 / kDtPerCU, "two workgroups per CU");
    const int64_t ntd = (a.dim + kTD - 1) / kTD, nslab = (a.rows + kTM - 1) / kTM;
    // slabs per workgroup as even as the resident slots allow
    int64_t nrep = static_cast<int64_t>(kDtCUs) * kDtPerCU / ntd;
    nrep = nrep < 1 ? 1 : (nrep > nslab ? nslab : nrep);
    const int64_t per = (nslab + nrep - 1) / nrep;
    nrep = (nslab + per - 1) / per;
    const dim3 grid(static_cast<unsigned>(ntd * nrep));
    if (a.dim % 8 == 0) hipLaunchKernelGGL((dt_proj_rows_kernel<NK, true>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((dt_proj_rows_kernel<NK, false>), grid, dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dt_proj(const DtProjArgs &a, hipStream_t s) {
    if (a.rows == 0 || a.dim == 0) return hipSuccess;
    if (a.bf16 && a.rank <= 160) {
        switch ((a.rank + 31) / 32) {
        case 1: return launch_rows<1>(a, s);
        case 2: return launch_rows<2>(a, s);
        case 3: return launch_rows<3>(a, s);
        case 4: return launch_rows<4>(a, s);
        default: return launch_rows<5>(a, s);
        }
    }
    const int64_t blocks = ((a.rows + kTM - 1) / kTM) * ((a.dim + kTD - 1) / kTD);
    if (a.bf16)
        hipLaunchKernelGGL(dt_proj_kernel<bf16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(dt_proj_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ssm
