// Forward selective scan for 1 <= d_state <= 16 on gfx950: the kernels and
// their launch templates.  The translation units scan_rows_*.hip and
// scan_general_*.hip each instantiate a share of them (so the library builds
// in parallel); scan_fwd.hip holds the entry points that dispatch to them.
//
// Recurrence per (b, d) chain (youngju.dev guide, section 2 ZOH + discrete
// recurrence; section 5 selective_scan with Delta*B*x input, D skip, SiLU(z)
// gate of the block):
//     h[n] <- exp(Delta_t A[d,n]) h[n] + Delta_t B[b,t,n] x[b,t,d]
//     y     = (sum_n C[b,t,n] h[n] + D[d] x) * SiLU(z)
//
// At d_state 16 the scan is bound by VALU issue, not by HBM: every (t, d, n)
// item needs one v_exp_f32 (half rate on gfx950) and four full-rate ops, while
// it moves only half a byte of HBM traffic.  Two kernels live here.
//
// scan_rows_kernel (d_state 16, the Mamba layer) is described above its
// definition: a wave owns 16 channels and all their states, rows of lanes
// exchange through lane-swap instructions, waves never synchronise, and
// persistent workgroups take (segment, tile) jobs from a queue.
//
// scan_fwd_kernel (every other d_state):
//   * A workgroup owns a tile of 64 consecutive channels of one batch row
//     (lane = channel, so every global access of a wave is one contiguous
//     128-byte (bf16) / 256-byte (fp32) row).  Its NW waves split the d_state
//     axis: wave w keeps states [w*NPW, (w+1)*NPW) of all 64 chains in VGPRs.
//   * Per block of TB steps the per-element work (softplus of delta + bias,
//     Delta*x) is done once per (t, d), split over the waves, and shared
//     through LDS; B and C of the block are widened to fp32 once into LDS and
//     read back as wave-uniform broadcasts.  Each wave's partial readout
//     sum_{n in its slice} C h goes to LDS, and the epilogue (sum of the NW
//     partials, D skip, SiLU gate, rounding, store) is split over the waves
//     again.  The three phases form a software pipeline over blocks (produce
//     block j, finish block j-2, scan block j-1) with double-buffered LDS and
//     one barrier per block; global loads are issued two blocks ahead of
//     their use, which hides the HBM latency behind two scan phases.
//   * Long sequences are cut into segments.  Each (tile, segment) is one
//     workgroup; segments are taken in order from an atomic ticket and hand
//     the 64 x d_state state to the next segment of the same tile through
//     global memory (release / acquire at agent scope).  A workgroup only
//     waits on a segment that started before it, and the dispatcher places
//     each next segment wherever a CU frees up, which evens out the load when
//     the tile count is not a multiple of the CU count.
#pragma once

#include <type_traits>
#include <utility>

#include "ssm_device.h"
#include "ssm_kernels.h"

#ifndef SSM_SCAN_TB
#define SSM_SCAN_TB 16            // steps per pipeline block
#endif
#ifndef SSM_SCAN_MAX_SEGS
#define SSM_SCAN_MAX_SEGS 8       // most segments per tile
#endif
#ifndef SSM_SCAN_MIN_SEG_STEPS
#define SSM_SCAN_MIN_SEG_STEPS 512
#endif
#ifndef SSM_ROWS_MAX_SEGS
#define SSM_ROWS_MAX_SEGS 4       // most segments per tile in the row kernel
#endif
#ifndef SSM_SCAN_SMALL_TILES
// Below this many channel tiles (the CU count of an MI355X) every tile of
// scan_fwd_kernel has a CU to itself: sequences are then not cut into
// segments (nothing to balance).
#define SSM_SCAN_SMALL_TILES 256
#endif

namespace ssm {
namespace {

constexpr int kTB = SSM_SCAN_TB;
constexpr int kTile = 64;                    // channels per workgroup (one per lane)
constexpr uint32_t kSpinLimit = 1u << 22;    // bounded wait on the previous segment (polls)

template <int N> constexpr int waves_for() {
    return N % 4 == 0 ? 4 : (N % 2 == 0 ? 2 : 1);
}

struct Params {
    const void *x, *delta, *z, *B, *C;
    const float *A, *D, *bias, *h0;
    void *y;
    float *last;
    uint32_t *words;     // [0] ticket, [1] error flag, [64 ..) per-tile progress
    uint32_t spin_limit; // polls before a wait on the previous segment gives up
    int publish;         // 0: segments never hand their state on (error-path tests only)
    float *hbuf;         // per tile: d_state x 64 carried states
    float *ckpt;         // row kernel, optional: state entering each 16-step block
    int64_t seqlen, dim, nblk;
    int n_dt, n_tiles, seg_len, n_segs, softplus;
    int grid_h, grid_w;  // row kernel, column-major visits: the patch grid
    float inv_h;         // 1 / grid_h
    // row kernel with the block's prologue: x is the conv input, filtered
    // here by the causal depthwise conv (conv_k taps, fp32 (dim, conv_k)
    // weights, optional bias) and SiLU; conv_state holds the inputs before
    // step 0 ((batch, dim, conv_k - 1) io dtype, oldest first) or is null
    const float *conv_w, *conv_b;
    const void *conv_state;
    int conv_k;
};

struct Layout {
    int n_dt, n_tiles, seg_len, n_segs;
    size_t hbuf_off, total;
};

// d_state 16 runs on the row kernel, whose persistent workgroups balance
// any number of tiles, in at most SSM_ROWS_MAX_SEGS segments; the other
// kernel takes at most SSM_SCAN_MAX_SEGS, and none when the tiles do not
// fill the CUs
bool rows_path(int64_t dstate) { return dstate == 16; }

Layout make_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t esize) {
    Layout l{};
    const bool rows = rows_path(dstate);
    const int64_t max_segs = rows ? SSM_ROWS_MAX_SEGS : SSM_SCAN_MAX_SEGS;
    l.n_dt = static_cast<int>((dim + kTile - 1) / kTile);
    l.n_tiles = static_cast<int>(batch * l.n_dt);
    const int64_t blocks = (seqlen + kTB - 1) / kTB;
    int64_t segs = (!rows && l.n_tiles < SSM_SCAN_SMALL_TILES) ? 1 : seqlen / SSM_SCAN_MIN_SEG_STEPS;
    segs = segs < 1 ? 1 : (segs > max_segs ? max_segs : segs);
    // row offsets inside a segment are 32-bit buffer offsets: keep a segment
    // of (seqlen, d_inner) below 1 GiB
    const int64_t max_rows = (int64_t(1) << 30) / (dim * esize > 0 ? dim * esize : 1);
    const int64_t need = max_rows > kTB ? (seqlen + max_rows - kTB - 1) / (max_rows - kTB) : seqlen;
    segs = segs > need ? segs : need;
    const int64_t seg_blocks = blocks > 0 ? (blocks + segs - 1) / segs : 1;
    l.seg_len = static_cast<int>(seg_blocks * kTB);
    l.n_segs = static_cast<int>(seqlen > 0 ? (seqlen + l.seg_len - 1) / l.seg_len : 1);
    auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
    // [0, 256): ticket + error word; [256, hbuf_off): per-tile progress
    l.hbuf_off = 256 + up(static_cast<size_t>(l.n_tiles) * sizeof(uint32_t));
    // carried states: 8 bytes each (the row kernel tags every value with its
    // segment; the other kernel uses the first half of the slab as floats)
    l.total = l.hbuf_off + up(static_cast<size_t>(l.n_tiles) * dstate * kTile * sizeof(uint64_t));
    return l;
}

// ---- DPP row broadcasts: lane K of every 16-lane row feeds the whole row
constexpr int kRowNewBcast = 0x150;   // DPP control row_newbcast:0

template <int K> __device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kRowNewBcast + K, 0xF, 0xF, true));
}

// acc += (lane K of each row of c) * h as a single v_fmac_f32 with a DPP
// source (the compiler folds DPP into v_mul but not into v_fmac).  c must
// come from a load, not from a VALU write just before: on gfx9 a VALU write
// needs two wait states before a DPP read of the same VGPR, and the compiler's
// hazard recognizer does not see inside inline assembly.  Every caller passes
// a value read from LDS; tests/test_dpp_hazards.py disassembles the built
// library and fails if any DPP source is written by a VALU within two wait
// states (an s_nop 1 here would cost two wait states per broadcast fma).
template <int K> __device__ __forceinline__ float fmac_row_bcast(float acc, float c, float h) {
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "+v"(acc) : "v"(c), "v"(h), "n"(K));
    return acc;
}

// One step of the wave's NPW states: breg holds B of the step in row lanes
// [0, NPW), creg holds C in row lanes [CB, CB + NPW).  Returns sum_i C_i h_i.
template <typename M, int NPW, int CB, int... I>
__device__ __forceinline__ float scan_step(std::integer_sequence<int, I...>, float (&h)[NPW],
                                           const float (&A2)[NPW], float dt, float dtx, float breg,
                                           float creg) {
    ((h[I] = M::step(dt * A2[I], h[I], dtx * row_bcast<I>(breg))), ...);
    float acc = h[0] * row_bcast<CB>(creg);
    ((acc = I > 0 ? fmac_row_bcast<CB + I>(acc, creg, h[I]) : acc), ...);
    return acc;
}

// ---- buffer loads / stores.  A wave-uniform descriptor (base and size in
// SGPRs) plus a per-lane byte offset and a scalar row offset is how gfx950
// addresses memory without per-lane 64-bit arithmetic.

#ifndef SSM_SCAN_WAVES_PER_EU
#define SSM_SCAN_WAVES_PER_EU 1   // occupancy the register allocator may assume
#endif

// FL = 1: softplus and gate known to be on at compile time (the common
// Mamba call); FL = 0 reads both flags at run time.
// TX: the storage type of x (T, or float when the caller's x is an fp32
// intermediate next to io-dtype inputs: the filtered x of the fused prologue).
template <int N, int NW, typename T, int FL, typename TX = T>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, SSM_SCAN_WAVES_PER_EU)))
void scan_fwd_kernel(Params p) {
    using M = typename MathFor<T>::type;
    static_assert(N % NW == 0 && kTB % NW == 0, "waves must split d_state and the block evenly");
    constexpr int NPW = N / NW;      // states per wave
    constexpr int PB = kTB / NW;     // steps per wave in the produce / finish phases
    constexpr int NT = NW * 64;
    constexpr int kBCV = 2 * NPW <= 16 ? 1 : 2;        // VGPRs holding one step's B and C
    constexpr int BC_HALF = (kTB * N + NT - 1) / NT;   // B (or C) values of a block staged per thread
    constexpr int BC_PER = 2 * BC_HALF;

    // LDS layouts are chosen for 128-bit reads: (Delta, Delta*x) of two
    // consecutive steps per lane and slot, partial readouts of four
    // consecutive steps, and B / C transposed to [state][step] (row stride
    // kTB + 4 floats keeps the 2*NPW rows a wave reads in distinct banks).
    static_assert(kTB % 4 == 0, "steps per block must be a multiple of 4");
    constexpr int kBCS = kTB + 4;
    __shared__ float4 sDX[2][kTB / 2][kTile];   // (Delta, Delta*x) of steps 2i, 2i+1
    __shared__ float4 sP[2][NW][kTB / 4][kTile];// partial readouts of steps 4i .. 4i+3
    __shared__ float sBC[2][2 * N][kBCS];       // [buf][n (B) | N + n (C)][step], fp32
    __shared__ uint32_t s_ticket, s_gaveup;

    using raw = typename Io<T>::raw;
    const int64_t seqlen = p.seqlen, dim = p.dim;

    const int tid = threadIdx.x, lane = tid % 64;
    // the wave index is uniform across the wave; saying so keeps every step,
    // row and state index derived from it in scalar registers
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    if (tid == 0) s_ticket = atomicAdd(&p.words[0], 1u);
    __syncthreads();
    const uint32_t ticket = __builtin_amdgcn_readfirstlane(s_ticket);   // uniform: keeps tile math scalar
    const int seg = static_cast<int>(ticket / static_cast<uint32_t>(p.n_tiles));
    const int tile = static_cast<int>(ticket % static_cast<uint32_t>(p.n_tiles));
    const int64_t b = tile / p.n_dt;
    const int64_t d0 = static_cast<int64_t>(tile % p.n_dt) * kTile;   // first channel of the tile
    const bool active = d0 + lane < dim;
    // column of this lane inside the tile; inactive lanes shadow the last channel
    const uint32_t col = active ? static_cast<uint32_t>(lane) : static_cast<uint32_t>(dim - 1 - d0);
    const int64_t d = d0 + col;
    const int n0 = w * NPW;
    const int64_t t_begin = static_cast<int64_t>(seg) * p.seg_len;
    const int64_t t_end = (t_begin + p.seg_len < seqlen) ? t_begin + p.seg_len : seqlen;
    const int steps = static_cast<int>(t_end - t_begin);   // steps of this segment (32-bit compares stay scalar)
    const int nb = (steps + kTB - 1) / kTB;
    const bool softplus_on = FL ? true : p.softplus != 0;
    const bool has_z = FL ? true : p.z != nullptr;
    uint32_t *progress = p.words + 64;

    // descriptors start at this segment's first row (and, for the (t, d)
    // tensors, at the tile's first channel); rows are scalar byte offsets
    const int64_t row0 = b * seqlen + t_begin;
    const int64_t e0 = (row0 * dim + d0) * static_cast<int64_t>(sizeof(T));
    const rsrc_t rx = make_rsrc(static_cast<const char *>(p.x) + (row0 * dim + d0) * static_cast<int64_t>(sizeof(TX)));
    const rsrc_t rd = make_rsrc(static_cast<const char *>(p.delta) + e0);
    const rsrc_t rz = make_rsrc(static_cast<const char *>(has_z ? p.z : p.delta) + e0);
    const rsrc_t ry = make_rsrc(static_cast<char *>(p.y) + e0);
    const rsrc_t rB = make_rsrc(static_cast<const char *>(p.B) + row0 * N * static_cast<int64_t>(sizeof(T)));
    const rsrc_t rC = make_rsrc(static_cast<const char *>(p.C) + row0 * N * static_cast<int64_t>(sizeof(T)));
    const uint32_t voff = col * static_cast<uint32_t>(sizeof(T));
    const uint32_t voffx = col * static_cast<uint32_t>(sizeof(TX));
    const uint32_t row_bytes_x = static_cast<uint32_t>(dim * static_cast<int64_t>(sizeof(TX)));
    // stores of lanes past d_inner use an offset beyond the descriptor's
    // range, which the buffer unit drops (no branch around the store)
    const uint32_t voff_store = active ? voff : kOffNone;
    const uint32_t row_bytes = static_cast<uint32_t>(dim * static_cast<int64_t>(sizeof(T)));
    float *hslot = p.hbuf + static_cast<int64_t>(tile) * N * kTile;

    float A2[NPW], h[NPW];
#pragma unroll
    for (int i = 0; i < NPW; ++i) A2[i] = M::prep_A(p.A[d * N + n0 + i]);
    const float bias = p.bias ? p.bias[d] : 0.0f;
    const float Dd = p.D ? p.D[d] : 0.0f;

    // ---- state entering this segment
    if (seg == 0) {
#pragma unroll
        for (int i = 0; i < NPW; ++i) h[i] = p.h0 ? p.h0[(b * dim + d) * N + n0 + i] : 0.0f;
    } else {
        // Poll with relaxed coherent loads (an acquire per poll would
        // invalidate the L2 every time) and acquire once when the flag is seen.
        // A wait that gives up records it in the workspace's error word and
        // poisons the state with NaN, so every output that depends on it is
        // NaN rather than silently wrong.
        if (tid == 0) {
            uint32_t spins = 0;
            s_gaveup = 0u;
            while (__hip_atomic_load(&progress[tile], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                   static_cast<uint32_t>(seg)) {
                if (++spins > p.spin_limit) {     // never wait unboundedly
                    __hip_atomic_store(&p.words[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    s_gaveup = 1u;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const bool gaveup = __builtin_amdgcn_readfirstlane(s_gaveup) != 0u;
#pragma unroll
        for (int i = 0; i < NPW; ++i) h[i] = gaveup ? __builtin_nanf("") : hslot[(n0 + i) * kTile + lane];
    }

    // ---- prefetch registers.  Loads are issued right after the data they
    // replace was consumed and two blocks ahead of their use.  Every load is
    // unconditional (rows clamped into the segment) so the loop body is
    // straight-line code.
    using rawx = typename Io<TX>::raw;
    struct Pre {
        raw dP[PB];            // produce phase: delta
        rawx xP[PB];           //                x
        rawx xE[PB];           // finish phase: x
        raw zE[PB];            //               z
        raw bc[BC_PER];        // B/C values this thread stages
    };
    auto clamp_step = [&](int j, int k) __attribute__((always_inline)) -> uint32_t {   // segment step of step k of block j, clamped
        const int s = j * kTB + k;
        return static_cast<uint32_t>(s < 0 ? 0 : (s < steps ? s : steps - 1));
    };
    // full: blocks jp and je lie wholly inside the segment (no clamping)
    auto load_pre = [&](Pre &r, int jp, int je, auto full) __attribute__((always_inline)) {
        constexpr bool F = decltype(full)::value;
        auto step_of = [&](int j, int k) __attribute__((always_inline)) -> uint32_t {
            return F ? static_cast<uint32_t>(j * kTB + k) : clamp_step(j, k);
        };
#pragma unroll
        for (int kk = 0; kk < PB; ++kk) {
            const uint32_t kp = step_of(jp, w * PB + kk), ke = step_of(je, w * PB + kk);
            r.dP[kk] = Io<T>::load(rd, voff, kp * row_bytes);
            r.xP[kk] = Io<TX>::load(rx, voffx, kp * row_bytes_x);
            r.xE[kk] = Io<TX>::load(rx, voffx, ke * row_bytes_x);
            if (has_z) r.zE[kk] = Io<T>::load(rz, voff, ke * row_bytes);
        }
        // B then C of the block; each loop has a uniform descriptor
#pragma unroll
        for (int m = 0; m < BC_PER; ++m) {
            int e = tid + (m % BC_HALF) * NT;
            e = e < kTB * N ? e : kTB * N - 1;
            const uint32_t off = (step_of(jp, e / N) * N + e % N) * static_cast<uint32_t>(sizeof(T));
            r.bc[m] = Io<T>::load(m < BC_HALF ? rB : rC, off, 0);
        }
    };

    // produce block j into LDS buffer j%2
    auto produce = [&](const Pre &r, int j, auto full) __attribute__((always_inline)) {
        const int buf = j & 1;
#pragma unroll
        for (int kk = 0; kk < PB; ++kk) {
            const int k = w * PB + kk;
            const bool tv = decltype(full)::value || j * kTB + k < steps;     // wave-uniform
            const float v = Io<T>::f32(r.dP[kk]) + bias;
            float dt = softplus_on ? M::softplus(v) : v;
            dt = tv ? dt : 0.0f;                     // past the end: identity step
            reinterpret_cast<float2 *>(&sDX[buf][k / 2][lane])[k % 2] = make_float2(dt, dt * Io<TX>::f32(r.xP[kk]));
        }
#pragma unroll
        for (int m = 0; m < BC_PER; ++m) {
            const int e = tid + (m % BC_HALF) * NT;
            if (e < kTB * N) sBC[buf][(m < BC_HALF ? 0 : N) + e % N][e / N] = Io<T>::f32(r.bc[m]);
        }
    };

    // Scan operands of block j (LDS buffer j%2), read in one go: Delta and
    // Delta*x per step, and B, C of the wave's states laid out so that lane q
    // of every 16-lane row holds value q of the step (B in lanes [0, NPW), C
    // after them).  The steps then run on registers only; B and C reach the
    // arithmetic through DPP row broadcasts.  Every read is 128 bits.
    struct ScanOps {
        float2 dx[kTB];
        float bcr[kTB][kBCV];
    };
    auto scan_read = [&](ScanOps &o, int j) __attribute__((always_inline)) {
        const int buf = j & 1;
        const int q = lane & 15;
#pragma unroll
        for (int k2 = 0; k2 < kTB / 2; ++k2) {
            const float4 v = sDX[buf][k2][lane];
            o.dx[2 * k2] = make_float2(v.x, v.y);
            o.dx[2 * k2 + 1] = make_float2(v.z, v.w);
        }
        // the state row each lane reads: B rows for lanes [0, NPW), C rows
        // after them (kBCV == 1); kBCV == 2 keeps B and C in two registers
        int mrow[kBCV];
        if constexpr (kBCV == 1) {
            const int qq = q < 2 * NPW ? q : 0;
            mrow[0] = qq < NPW ? n0 + qq : N + n0 + qq - NPW;
        } else {
            const int qq = q < NPW ? q : 0;
            mrow[0] = n0 + qq;
            mrow[1] = N + n0 + qq;
        }
#pragma unroll
        for (int v = 0; v < kBCV; ++v)
#pragma unroll
            for (int k4 = 0; k4 < kTB / 4; ++k4) {
                const float4 c4 = *reinterpret_cast<const float4 *>(&sBC[buf][mrow[v]][4 * k4]);
                o.bcr[4 * k4][v] = c4.x;
                o.bcr[4 * k4 + 1][v] = c4.y;
                o.bcr[4 * k4 + 2][v] = c4.z;
                o.bcr[4 * k4 + 3][v] = c4.w;
            }
    };
    auto scan = [&](const ScanOps &o, int j) __attribute__((always_inline)) {
        const int buf = j & 1;
#pragma unroll
        for (int k4 = 0; k4 < kTB / 4; ++k4) {
            float part[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = 4 * k4 + i;
                part[i] = scan_step<M, NPW, (kBCV == 1 ? NPW : 0)>(
                    std::make_integer_sequence<int, NPW>{}, h, A2, o.dx[k].x, o.dx[k].y, o.bcr[k][0],
                    o.bcr[k][kBCV - 1]);
            }
            sP[buf][w][k4][lane] = make_float4(part[0], part[1], part[2], part[3]);
        }
    };

    // finish block j: sum the partials (read early, at the top of the
    // iteration, so their LDS latency hides behind the produce phase), D skip,
    // gate, store
    struct Partials {
        float v[PB][NW];
    };
    auto finish_read = [&](Partials &pv, int j) __attribute__((always_inline)) {
        const int buf = j & 1;
        const float *base = reinterpret_cast<const float *>(&sP[buf][0][0][0]);
#pragma unroll
        for (int kk = 0; kk < PB; ++kk) {
            const int k = w * PB + kk;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww)
                pv.v[kk][ww] = base[((ww * (kTB / 4) + k / 4) * kTile + lane) * 4 + k % 4];
        }
    };
    auto finish = [&](const Pre &r, const Partials &pv, int j, auto full) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < PB; ++kk) {
            const int k = w * PB + kk;
            const int sl = j * kTB + k;
            float acc = 0.0f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) acc += pv.v[kk][ww];
            float out = fmaf(Dd, Io<TX>::f32(r.xE[kk]), acc);
            if (has_z) out *= silu(Io<T>::f32(r.zE[kk]));
            if (decltype(full)::value || sl < steps)
                Io<T>::store(out, ry, voff_store, static_cast<uint32_t>(sl) * row_bytes);
        }
    };

    // ---- the pipeline: iteration j reads the scan operands of block j-1,
    // produces block j, finishes block j-2, issues the global loads of two
    // iterations ahead and scans block j-1.  Two prefetch register sets
    // alternate, so every global load has two scan phases to arrive.  The
    // phases of an iteration are compile-time flags: the steady-state
    // iterations are straight-line code, which lets the compiler count
    // outstanding loads exactly instead of draining them at every branch.
    ScanOps so;
    auto iteration = [&](auto produce_on, auto finish_on, auto scan_on, auto full, Pre &r, int j) __attribute__((always_inline)) {
        Partials pv;
        if constexpr (decltype(scan_on)::value) scan_read(so, j - 1);
        if constexpr (decltype(finish_on)::value) finish_read(pv, j - 2);
        if constexpr (decltype(produce_on)::value) produce(r, j, full);
        if constexpr (decltype(finish_on)::value) finish(r, pv, j - 2, full);
        load_pre(r, j + 2, j, full);
        if constexpr (decltype(scan_on)::value) scan(so, j - 1);
        __syncthreads();
    };
    using on = std::true_type;
    using off = std::false_type;
    const int nfull = steps / kTB;               // blocks with no step past the segment
    Pre r0, r1;
    load_pre(r0, 0, 0, off{});
    load_pre(r1, 1, 0, off{});
    if (nb >= 3) {
        iteration(on{}, off{}, off{}, off{}, r0, 0);
        iteration(on{}, off{}, on{}, off{}, r1, 1);
        int j = 2;
        // steady state over whole blocks: no clamping, no store guards
        for (; j + 3 < nfull; j += 2) {
            iteration(on{}, on{}, on{}, on{}, r0, j);
            iteration(on{}, on{}, on{}, on{}, r1, j + 1);
        }
        for (; j + 1 < nb; j += 2) {
            iteration(on{}, on{}, on{}, off{}, r0, j);
            iteration(on{}, on{}, on{}, off{}, r1, j + 1);
        }
        if (j < nb) {          // one steady iteration left (even j): drain ends on set r1
            iteration(on{}, on{}, on{}, off{}, r0, j);
            iteration(off{}, on{}, on{}, off{}, r1, nb);
            iteration(off{}, on{}, off{}, off{}, r0, nb + 1);
        } else {               // j == nb (even): drain ends on set r0
            iteration(off{}, on{}, on{}, off{}, r0, nb);
            iteration(off{}, on{}, off{}, off{}, r1, nb + 1);
        }
    } else {
        // short segments: the same phases with run-time conditions
        for (int j = 0; j < nb + 2; ++j) {
            Pre &r = (j & 1) ? r1 : r0;
            const bool do_scan = j >= 1 && j - 1 < nb;
            Partials pv;
            if (do_scan) scan_read(so, j - 1);
            if (j >= 2) finish_read(pv, j - 2);
            if (j < nb) produce(r, j, off{});
            if (j >= 2) finish(r, pv, j - 2, off{});
            load_pre(r, j + 2, j, off{});
            if (do_scan) scan(so, j - 1);
            __syncthreads();
        }
    }

    // ---- hand the state on, or write last_state
    if (seg + 1 < p.n_segs) {
#pragma unroll
        for (int i = 0; i < NPW; ++i) hslot[(n0 + i) * kTile + lane] = h[i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // every wave's stores, then the flag
        __syncthreads();
        if (tid == 0 && p.publish)
            __hip_atomic_store(&progress[tile], static_cast<uint32_t>(seg + 1), __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else if (p.last && active) {
#pragma unroll
        for (int i = 0; i < NPW; ++i) p.last[(b * dim + d) * N + n0 + i] = h[i];
    }
}

// ===========================================================================
// d_state 16: the row kernel.
//
// A wave owns 16 channels and all 16 states of each: lane = 16 * r + c holds
// states [4r, 4r + 4) of channel c, so a 16-lane DPP row is one state group
// and a lane column is one channel.  Waves share nothing and never wait on
// each other; within a wave, the per-(t, d) work and the readout sum over
// states cross the four rows:
//   * per group of 4 steps, row r discretises step kRowStep[r] of the group
//     (softplus of delta + bias, Delta*x), two groups ahead, and the wave's
//     LDS slot gives every lane the four steps (an all-gather by the gfx950
//     lane swaps took 6 VALU swaps per group: 3% slower at the 2.8b layer);
//   * B and C of the block, staged in this wave's own LDS slice, reach the
//     arithmetic through DPP row broadcasts (lane q < 4 of row r holds
//     B[4r + q], lanes 4..7 hold C[4r + q - 4]);
//   * the four steps' partial readouts are summed across rows by a
//     reduce-scatter with the lane swaps v_permlane16_swap /
//     v_permlane32_swap (3 swaps, 3 adds; through LDS, with the output a
//     group later, it measured 3% slower) that leaves the total of step
//     kRowStep[r] in row r, which then applies the D skip and the gate and
//     stores it.
// x, delta and z of a group are loaded two blocks ahead.  Long sequences are
// cut into segments handed on through the workspace, as in the kernel above.
constexpr int kRowTB = 16;                   // steps per block (four groups of four)
#ifndef SSM_ROWS_WG_PER_CU
// persistent workgroups (4 waves each) per CU.  One: no more workgroups than
// the 320 tiles of the 2.8b layer can keep busy, so a job never waits on a
// predecessor that has not finished
#define SSM_ROWS_WG_PER_CU 1
#endif
// With at least this many tiles per CU a second persistent workgroup per CU
// always has a job whose predecessor is done.  It then fills the VALU cycles
// that one wave per SIMD leaves idle: measured 751 against 870 us at
// 16 x 2048 x 5120 (1280 tiles), equal at 640 tiles, slower at 320.
constexpr int kRowsTilesPerCuForTwo = 4;
constexpr int kRowBCS = kRowTB + 4;          // LDS row stride of the staged B / C (floats)
constexpr int kRowCOff = 16 * kRowBCS + 16;  // C rows start 16 banks after the B rows
constexpr int kRowBCWords = kRowCOff + 16 * kRowBCS;

__device__ __forceinline__ void swap16(float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// out[k] = the value row k holds, in every lane of its column
__device__ __forceinline__ void row_allgather(float v, float (&out)[4]) {
    float a = v, b = v;
    swap16(a, b);          // a: rows (0, 0, 2, 2)   b: rows (1, 1, 3, 3)
    float a2 = a, b2 = b;
    swap32(a, a2);         // a: row 0 everywhere    a2: row 2 everywhere
    swap32(b, b2);         // b: row 1 everywhere    b2: row 3 everywhere
    out[0] = a; out[1] = b; out[2] = a2; out[3] = b2;
}
// sum over the four rows of p[0..3]; row r receives the total of p[kRowStep[r]]
__device__ __forceinline__ float row_reduce_scatter(const float (&p)[4]) {
    float a = p[0], b = p[1];
    swap32(a, b);          // a + b: rows (0+2, 1+3) of p0 in rows 0-1, of p1 in rows 2-3
    const float u = a + b;
    float c = p[2], e = p[3];
    swap32(c, e);
    const float v = c + e; // the same for p2, p3
    float s0 = u, s1 = v;
    swap16(s0, s1);        // rows: (u0, v0, u2, v2) and (u1, v1, u3, v3)
    return s0 + s1;        // totals of p0, p2, p1, p3 in rows 0, 1, 2, 3
}

template <typename T> struct Wide4;          // four consecutive io elements as one load
template <> struct Wide4<bf16_t> {
    typedef uint32_t raw __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ raw load(rsrc_t r, uint32_t voff) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
    }
    static __device__ __forceinline__ float get(const raw &v, int i) {
        const uint32_t wd = v[i / 2];
        return __uint_as_float(i % 2 ? (wd & 0xffff0000u) : (wd << 16));
    }
};
template <> struct Wide4<float> {
    typedef uint32_t raw __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ raw load(rsrc_t r, uint32_t voff) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
    }
    static __device__ __forceinline__ float get(const raw &v, int i) { return __uint_as_float(v[i]); }
};

// CK = true: also record the state entering every block in p.ckpt (y may
// then be absent); a separate instantiation, so the forward proper carries
// none of it.  REV = true: the sequence is visited from its last step to its
// first (step k of the scan reads and writes row seqlen - 1 - k), the 2-D
// scan's reversed row-major order without a gathered copy.  COL = true: the
// rows are patches of a grid_h x grid_w grid visited column by column (step
// q reads and writes row (q mod grid_h) grid_w + q div grid_h, q counted
// from the end when REV), the 2-D scan's column-major orders in place.
// CONV = true: x is the input of the block's causal conv1d (up to 4 taps) +
// SiLU, which runs here on the raw x (three more rows per step, the first
// three read from the caller's window or zeros), and the filtered x that the
// scan consumes never leaves the registers.
template <typename T, int FL, bool CK = false, bool REV = false, bool COL = false, bool CONV = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4)))
void scan_rows_kernel(Params p) {
    static_assert(!CONV || (!CK && !REV && !COL), "the fused prologue runs in the forward order only");
    using M = typename MathFor<T>::type;
    using raw = typename Io<T>::raw;
    using W4 = Wide4<T>;
    constexpr int N = 16, NPL = 4, NG = kRowTB / 4;
    constexpr uint32_t es = sizeof(T);
    __shared__ __attribute__((aligned(16))) float sBC[4][2][kRowBCWords];   // per wave, double-buffered B / C
    // per wave: one group's (Delta, Delta x) of 16 channels x 4 steps,
    // [channel (stride 6: every channel in banks of its own)][step]
    constexpr int kXGS = 6;
    __shared__ __attribute__((aligned(16))) float2 sXG[4][16 * kXGS];
    __shared__ uint32_t s_ticket;

    const int64_t seqlen = p.seqlen, dim = p.dim;
    const int tid = threadIdx.x, lane = tid % 64;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    const int r = lane / 16, c = lane % 16;
    const int rstep = r == 1 ? 2 : (r == 2 ? 1 : r);   // the step of a group this row discretises / finishes
    const uint32_t n_jobs = static_cast<uint32_t>(p.n_tiles) * static_cast<uint32_t>(p.n_segs);
    // Persistent workgroups take (segment, tile) jobs in ticket order, all
    // tiles' segment s before any segment s + 1: a job's predecessor was
    // taken by a running workgroup long before, so waits are rare and short,
    // and every workgroup does the same number of jobs to within one.
    for (;;) {
    if (tid == 0) s_ticket = atomicAdd(&p.words[0], 1u);
    __syncthreads();
    const uint32_t ticket = __builtin_amdgcn_readfirstlane(s_ticket);
    if (ticket >= n_jobs) break;
    const int seg = static_cast<int>(ticket / static_cast<uint32_t>(p.n_tiles));
    const int tile = static_cast<int>(ticket % static_cast<uint32_t>(p.n_tiles));
    const int64_t b = tile / p.n_dt;
    const int64_t d0 = static_cast<int64_t>(tile % p.n_dt) * kTile;
    const int tcol = w * 16 + c;                        // channel inside the 64-channel tile
    const bool active = d0 + tcol < dim;
    const uint32_t col = active ? static_cast<uint32_t>(tcol) : static_cast<uint32_t>(dim - 1 - d0);
    const int64_t d = d0 + col;
    const int n0 = r * NPL;
    const int64_t t_begin = static_cast<int64_t>(seg) * p.seg_len;
    const int64_t t_end = (t_begin + p.seg_len < seqlen) ? t_begin + p.seg_len : seqlen;
    const int steps = static_cast<int>(t_end - t_begin);
    const int nb = (steps + kRowTB - 1) / kRowTB;
    const int nfull = steps / kRowTB;
    const bool softplus_on = FL ? true : p.softplus != 0;
    const bool has_z = FL ? true : p.z != nullptr;

    // descriptors start at the segment's lowest row: its first step, or its
    // last one when the sequence is visited backwards
    // (column-major visits: the batch row's first row, every offset below 2^31)
    const int64_t row0 = COL ? b * seqlen : (REV ? b * seqlen + (seqlen - t_end) : b * seqlen + t_begin);
    const int64_t e0 = (row0 * dim + d0) * static_cast<int64_t>(es);
    const rsrc_t rx = make_rsrc(static_cast<const char *>(p.x) + e0);
    const rsrc_t rd = make_rsrc(static_cast<const char *>(p.delta) + e0);
    const rsrc_t rz = make_rsrc(static_cast<const char *>(has_z ? p.z : p.x) + e0);
    // y may be absent when the block states are recorded: its stores then go
    // to an empty descriptor and are dropped
    const rsrc_t ry = (!CK || p.y) ? make_rsrc(static_cast<char *>(p.y) + e0) : make_rsrc(p.x, 0u);
    // B / C of the segment; rows past its end read 0
    const uint32_t bc_bytes = static_cast<uint32_t>(COL ? seqlen : steps) * N * es;
    const rsrc_t rB = make_rsrc(static_cast<const char *>(p.B) + row0 * N * static_cast<int64_t>(es), bc_bytes);
    const rsrc_t rC = make_rsrc(static_cast<const char *>(p.C) + row0 * N * static_cast<int64_t>(es), bc_bytes);
    const uint32_t row_bytes = static_cast<uint32_t>(dim * static_cast<int64_t>(es));
    const uint32_t vcol = col * es;
    // lane offset of its row in a whole group, the group's first row in the
    // scalar offset.  Backwards, group step s is row 3 - s of the group, whose
    // first row (in the scalar offset) is steps - 4 - (the group's first step):
    // never negative for a whole block, so both halves stay in the segment.
    const uint32_t voff_full = vcol + static_cast<uint32_t>(REV ? 3 - rstep : rstep) * row_bytes;
    auto soff_full = [&](int j, int g) __attribute__((always_inline)) {
        return static_cast<uint32_t>(REV ? steps - 4 - (j * kRowTB + 4 * g) : j * kRowTB + 4 * g) * row_bytes;
    };
    // the lane offset of segment step k
    auto row_off = [&](int k) __attribute__((always_inline)) {
        return vcol + static_cast<uint32_t>(REV ? steps - 1 - k : k) * row_bytes;
    };
    // column-major visits: the row (inside the batch row) of segment step k.
    // q < 2^23, so q and the fp32 quotient estimate are within one of the
    // true quotient, and one correction each way makes it exact.
    auto col_row = [&](int k) __attribute__((always_inline)) {
        const int kk = static_cast<int>(t_begin) + k;
        const int q = REV ? static_cast<int>(seqlen) - 1 - kk : kk;
        int qd = static_cast<int>(static_cast<float>(q) * p.inv_h);
        int qm = q - qd * p.grid_h;
        if (qm < 0) { qm += p.grid_h; --qd; }
        if (qm >= p.grid_h) { qm -= p.grid_h; ++qd; }
        return static_cast<uint32_t>(qm * p.grid_w + qd);
    };
    // carried states of this tile: one 64-bit word per state, the value in
    // the low half and (segment + 1) of its writer in the high half
    uint64_t *hslot = reinterpret_cast<uint64_t *>(p.hbuf) + static_cast<int64_t>(tile) * N * kTile;
    float *bc_lds = sBC[w][0];

    float A2[NPL], h[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) A2[i] = M::prep_A(p.A[d * N + n0 + i]);
    const float bias = p.bias ? p.bias[d] : 0.0f;
    const float Dd = p.D ? p.D[d] : 0.0f;

    // the prologue's filter, padded on the old side to four taps: cw[k]
    // multiplies x at step t - 3 + k; cwin[i] is x at step i - 3 before the
    // sequence (the caller's window, or zeros)
    float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cbias = 0.0f, cwin[3] = {0.0f, 0.0f, 0.0f};
    // rows before the segment the conv reads: three, except at the sequence's start
    const int halo = (CONV && t_begin > 0) ? 3 : 0;
    if constexpr (CONV) {
        const int K = p.conv_k;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (k >= 4 - K) cw[k] = p.conv_w[d * K + k - (4 - K)];
        cbias = p.conv_b ? p.conv_b[d] : 0.0f;
        if (t_begin == 0 && p.conv_state && K > 1) {
            const raw *st = static_cast<const raw *>(p.conv_state) + (b * dim + d) * (K - 1);
#pragma unroll
            for (int i = 0; i < 3; ++i)
                if (i >= 3 - (K - 1)) cwin[i] = Io<T>::f32(st[i - (3 - (K - 1))]);
        }
    }
    const rsrc_t rxc = make_rsrc(static_cast<const char *>(p.x) + e0 - static_cast<int64_t>(halo) * dim * es);

    if (seg == 0) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) h[i] = p.h0 ? p.h0[(b * dim + d) * N + n0 + i] : 0.0f;
    } else {
        // Each lane waits for its own four words to carry the previous
        // segment's tag: value and tag arrive together in one 64-bit atomic,
        // so no fence (and no cache-wide invalidate or write-back) is needed,
        // and the waves of the workgroup do not wait for one another.
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            uint64_t *slot = &hslot[(n0 + i) * kTile + tcol];
            uint64_t v = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t spins = 0;
            bool gaveup = false;
            while (static_cast<uint32_t>(v >> 32) != static_cast<uint32_t>(seg)) {
                if (++spins > p.spin_limit) {        // never wait unboundedly
                    __hip_atomic_store(&p.words[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    gaveup = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                v = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            // a give-up is recorded in the error word and poisons the state
            // (NaN), so no output that depends on it passes for a value
            h[i] = gaveup ? __builtin_nanf("") : __uint_as_float(static_cast<uint32_t>(v));
        }
    }

    // ---- per-lane raw inputs of one block: delta, x, z of step kRowStep[r]
    // of each group
    struct Pre {                                     // raw words, zero-extended at the load
        uint32_t d[NG], x[NG], z[NG];
        uint32_t off[NG];                            // column-major visits: the lane's row offset
        uint32_t xh[3][NG];                          // the prologue: x at steps s - 1, s - 2, s - 3
    };
    // the segment step this lane touches in group g of block j (clamped when
    // the block is not whole)
    auto lane_step = [&](int j, int g) __attribute__((always_inline)) {
        const int s = j * kRowTB + 4 * g + rstep;
        return s < steps ? s : steps - 1;
    };
    auto load_group = [&](Pre &pr, int j, int g, auto full) __attribute__((always_inline)) {
        if constexpr (COL) {                         // kept for the store of this step
            const uint32_t vo = vcol + col_row(lane_step(j, g)) * row_bytes;
            pr.off[g] = vo;
            pr.d[g] = Io<T>::load(rd, vo, 0);
            pr.x[g] = Io<T>::load(rx, vo, 0);
            if (has_z) pr.z[g] = Io<T>::load(rz, vo, 0);
        } else if constexpr (decltype(full)::value) {
            const uint32_t so = soff_full(j, g);
            pr.d[g] = Io<T>::load(rd, voff_full, so);
            pr.x[g] = Io<T>::load(rx, voff_full, so);
            if (has_z) pr.z[g] = Io<T>::load(rz, voff_full, so);
            if constexpr (CONV) {
                // rows s - k of a whole block: never before the halo (the
                // sequence's first blocks take the other path)
#pragma unroll
                for (int k = 1; k <= 3; ++k)
                    pr.xh[k - 1][g] = Io<T>::load(
                        rxc, voff_full, static_cast<uint32_t>(j * kRowTB + 4 * g + halo - k) * row_bytes);
            }
        } else {
            const int sl = lane_step(j, g);
            const uint32_t vo = row_off(sl);
            pr.d[g] = Io<T>::load(rd, vo, 0);
            pr.x[g] = Io<T>::load(rx, vo, 0);
            if (has_z) pr.z[g] = Io<T>::load(rz, vo, 0);
            if constexpr (CONV) {
                // before the sequence's first step the buffer reads 0; the
                // block substitutes the window
#pragma unroll
                for (int k = 1; k <= 3; ++k) {
                    const int rk = sl - k + halo;
                    pr.xh[k - 1][g] = Io<T>::load(rxc, rk >= 0 ? vcol + static_cast<uint32_t>(rk) * row_bytes : kOffNone, 0);
                }
            }
        }
    };
    // B / C of block j: lane l fetches elements [4l, 4l + 4) of each (16 steps x 16 states)
    struct BCRaw {
        typename W4::raw b, c;
    };
    auto load_bc = [&](BCRaw &v, int j) __attribute__((always_inline)) {
        // backwards, step j * 16 + lane / 4 is row steps - 1 - that step of the
        // segment; past the end the offset wraps beyond the descriptor: zeros
        uint32_t off;
        if constexpr (COL) {
            const int k = j * kRowTB + lane / 4;
            off = k < steps ? (col_row(k) * N + (lane % 4) * 4) * es : kOffNone;
        } else {
            off = REV ? static_cast<uint32_t>(((steps - 1 - (j * kRowTB + lane / 4)) * N + (lane % 4) * 4) *
                                              static_cast<int>(es))
                      : (static_cast<uint32_t>(j) * kRowTB * N + 4 * lane) * es;
        }
        v.b = W4::load(rB, off);
        v.c = W4::load(rC, off);
    };
    auto stash_bc = [&](BCRaw &v, int j) __attribute__((always_inline)) {
        asm volatile("" : "+v"(v.b), "+v"(v.c));     // widen here, not next to the load
        float *buf = bc_lds + (j & 1) * kRowBCWords;
        const int t = (4 * lane) / N, n = (4 * lane) % N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            buf[(n + i) * kRowBCS + t] = W4::get(v.b, i);
            buf[kRowCOff + (n + i) * kRowBCS + t] = W4::get(v.c, i);
        }
    };
    // the staged row this lane reads: B rows for lanes q < 4 of its DPP row,
    // C rows for q in [4, 8)
    const int q = c < 2 * NPL ? c : 0;
    const int bc_row = q < NPL ? (n0 + q) * kRowBCS : kRowCOff + (n0 + q - NPL) * kRowBCS;

    // one block: four groups; the raw inputs of block j + 2 are loaded into
    // the same registers right after each group consumed its own
    // bcq holds the staged B / C of the group about to run: each group reads
    // the next group's (the first of block j + 1 comes from the other buffer,
    // stashed at the start of block j) so the LDS latency is covered by a
    // whole group of arithmetic.
    auto widen = [](uint32_t wd) __attribute__((always_inline)) {
        return sizeof(raw) == 4 ? __uint_as_float(wd) : __uint_as_float(wd << 16);
    };
    // ---- the per-(t, d) values of a group, two groups ahead: lane (r, c)
    // discretises step kRowStep[r] of channel c (Delta, Delta x, and its own
    // x for the D skip), writes (Delta, Delta x) to its wave's LDS slot at
    // [c][step] and reads its channel's four steps straight back into the
    // register set of the group's parity.  A wave's LDS operations run in
    // order, so no barrier is needed, and the round trip runs under a whole
    // group of arithmetic (a lane-swap all-gather took six VALU swaps per
    // group).
    float2 *xg = &sXG[w][0];
    float4 xg01[2], xg23[2];                         // (Delta, Delta x) of steps 0, 1 / 2, 3, per group parity
    float xvg[2];                                    // this lane's x (filtered by the prologue), per group parity
    // (win: the group may lie outside whole blocks, so it may hold the
    // sequence's first steps, whose conv window comes from the caller, or
    // steps past the segment's end; false when it lies in a whole block,
    // which holds neither)
    auto prepare = [&](const Pre &q, int jj, int gg, auto win) __attribute__((always_inline)) {
        // pin the first use of the group's raw inputs here: otherwise the
        // scheduler hoists their widening next to the loads two blocks ahead
        // and the wave waits for memory it does not need yet.  The pinned
        // words are widened straight from 32 bits (a bf16 load zero-extends,
        // and the shift drops the upper half anyway).
        uint32_t dw = q.d[gg], xw = q.x[gg];
        asm volatile("" : "+v"(dw), "+v"(xw));
        const int sl = jj * kRowTB + 4 * gg + rstep;
        const float v = widen(dw) + bias;
        float dt = softplus_on ? M::softplus(v) : v;
        if constexpr (decltype(win)::value)
            dt = sl < steps ? dt : 0.0f;             // past the end: identity step
        float xv = widen(xw);
        if constexpr (CONV) {
            uint32_t h1 = q.xh[0][gg], h2 = q.xh[1][gg], h3 = q.xh[2][gg];
            asm volatile("" : "+v"(h1), "+v"(h2), "+v"(h3));
            float x1 = widen(h1), x2 = widen(h2), x3 = widen(h3);   // x at s - 1, s - 2, s - 3
            if (decltype(win)::value && t_begin == 0 && jj == 0) {   // steps before 0: the caller's window
                x1 = sl >= 1 ? x1 : cwin[2];
                x2 = sl >= 2 ? x2 : (sl == 1 ? cwin[2] : cwin[1]);
                x3 = sl >= 3 ? x3 : (sl == 2 ? cwin[2] : (sl == 1 ? cwin[1] : cwin[0]));
            }
            xv = silu(fmaf(cw[3], xv, fmaf(cw[2], x1, fmaf(cw[1], x2, fmaf(cw[0], x3, cbias)))));
        }
        xg[c * kXGS + rstep] = make_float2(dt, dt * xv);
        __builtin_amdgcn_wave_barrier();
        xg01[gg & 1] = *reinterpret_cast<const float4 *>(&xg[c * kXGS]);
        xg23[gg & 1] = *reinterpret_cast<const float4 *>(&xg[c * kXGS + 2]);
        xvg[gg & 1] = xv;
    };

    // one block: four groups; the raw inputs of block j + 2 are loaded into
    // the same registers right after each group consumed its own (nx holds
    // block j + 1's, whose first two groups are prepared in this block's last two)
    // bcq holds the staged B / C of the group about to run: each group reads
    // the next group's (the first of block j + 1 comes from the other buffer,
    // stashed at the start of block j) so the LDS latency is covered by a
    // whole group of arithmetic.
    auto block = [&](Pre &pr, const Pre &nx, BCRaw &bcn, float4 &bcq, int j, auto full) __attribute__((always_inline)) {
        constexpr bool F = decltype(full)::value;
        if (CK && active) {                         // the state entering this block
            const int64_t blk = t_begin / kRowTB + j;
            *reinterpret_cast<float4 *>(p.ckpt + ((b * p.nblk + blk) * dim + d) * N + n0) =
                make_float4(h[0], h[1], h[2], h[3]);
        }
        stash_bc(bcn, j + 1);                       // loaded one block ago
        load_bc(bcn, j + 2);
        const float *buf = bc_lds + (j & 1) * kRowBCWords + bc_row;
        const float *nbuf = bc_lds + ((j + 1) & 1) * kRowBCWords + bc_row;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float4 bc4 = bcq;
            bcq = *reinterpret_cast<const float4 *>(g + 1 < NG ? buf + 4 * (g + 1) : nbuf);
            const int sl = j * kRowTB + 4 * g + rstep;
            const float bcs[4] = {bc4.x, bc4.y, bc4.z, bc4.w};
            float part[4];
            float xv;
            uint32_t zw;
            if constexpr (!CONV) {
                zw = pr.z[g];                        // (raw word, pinned as above)
                asm volatile("" : "+v"(zw));
                // this group's values, prepared two groups ago
                const float4 e01 = xg01[g & 1], e23 = xg23[g & 1];
                const float dts[4] = {e01.x, e01.z, e23.x, e23.z};
                const float dtxs[4] = {e01.y, e01.w, e23.y, e23.w};
                xv = xvg[g & 1];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    part[k] = scan_step<M, NPL, NPL>(std::make_integer_sequence<int, NPL>{}, h, A2, dts[k],
                                                     dtxs[k], bcs[k], bcs[k]);
                // the group after next: in this block, or among the next block's first two
                if (g + 2 < NG)
                    prepare(pr, j, g + 2, std::integral_constant<bool, !F>{});
                else
                    prepare(nx, j + 1, g + 2 - NG, std::integral_constant<bool, !F>{});
            } else {
                // with the conv prologue (registers already tight) the group is
                // discretised here and all-gathered by lane swaps: the LDS form
                // two groups ahead measured 4% slower in this instantiation
                uint32_t dw = pr.d[g], xw = pr.x[g];
                zw = pr.z[g];
                asm volatile("" : "+v"(dw), "+v"(xw), "+v"(zw));
                const float v = widen(dw) + bias;
                float dt = softplus_on ? M::softplus(v) : v;
                dt = (F || sl < steps) ? dt : 0.0f;  // past the end: identity step
                uint32_t h1 = pr.xh[0][g], h2 = pr.xh[1][g], h3 = pr.xh[2][g];
                asm volatile("" : "+v"(h1), "+v"(h2), "+v"(h3));
                float x1 = widen(h1), x2 = widen(h2), x3 = widen(h3);   // x at s - 1, s - 2, s - 3
                if (!F && t_begin == 0) {            // steps before 0: the caller's window
                    x1 = sl >= 1 ? x1 : cwin[2];
                    x2 = sl >= 2 ? x2 : (sl == 1 ? cwin[2] : cwin[1]);
                    x3 = sl >= 3 ? x3 : (sl == 2 ? cwin[2] : (sl == 1 ? cwin[1] : cwin[0]));
                }
                xv = silu(fmaf(cw[3], widen(xw), fmaf(cw[2], x1, fmaf(cw[1], x2, fmaf(cw[0], x3, cbias)))));
                float dts[4], dtxs[4];
                row_allgather(dt, dts);
                row_allgather(dt * xv, dtxs);
                // group step k lives in row kRowStep^-1(k): 0 -> 0, 1 -> 2, 2 -> 1, 3 -> 3
                constexpr int src_row[4] = {0, 2, 1, 3};
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    part[k] = scan_step<M, NPL, NPL>(std::make_integer_sequence<int, NPL>{}, h, A2,
                                                     dts[src_row[k]], dtxs[src_row[k]], bcs[k], bcs[k]);
            }
            float out = fmaf(Dd, xv, row_reduce_scatter(part));
            if (has_z) out *= silu(widen(zw));
            if constexpr (COL) {
                Io<T>::store(out, ry, (active && (F || sl < steps)) ? pr.off[g] : kOffNone, 0);
            } else if constexpr (F) {
                Io<T>::store(out, ry, active ? voff_full : kOffNone, soff_full(j, g));
            } else {
                const uint32_t vo = (active && sl < steps) ? row_off(sl) : kOffNone;
                Io<T>::store(out, ry, vo, 0);
            }
            load_group(pr, j + 2, g, std::integral_constant<bool, F>{});
            asm volatile("" ::: "memory");
        }
    };

    Pre p0, p1;
    BCRaw bca, bcb;
    {
        // Start the job with nothing in flight and issue in the steady
        // state's order (B/C of block 1 before the inputs of blocks 0 and 1):
        // the wait counts the compiler derives at the loop head then stay as
        // partial as inside the loop.
        __builtin_amdgcn_s_waitcnt(0);
        using off = std::false_type;
        load_bc(bca, 0);
        load_bc(bcb, 1);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            load_group(p0, 0, g, off{});
            asm volatile("" ::: "memory");           // keep the per-group issue order
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            load_group(p1, 1, g, off{});
            asm volatile("" ::: "memory");
        }
        stash_bc(bca, 0);
    }
    float4 bcq = *reinterpret_cast<const float4 *>(bc_lds + bc_row);   // block 0, group 0
    if constexpr (!CONV) {
        prepare(p0, 0, 0, std::true_type{});
        prepare(p0, 0, 1, std::true_type{});
    }
    // bcb carries block j + 1 into block j (stashed there), then block j + 2
    int j = 0;
    if (CONV && t_begin == 0) {
        // the first two blocks of a sequence read the conv window before
        // step 0: they take the path with per-lane row checks
        block(p0, p1, bcb, bcq, 0, std::false_type{});
        if (nb > 1) block(p1, p0, bcb, bcq, 1, std::false_type{});
        j = 2;
    }
    for (; j + 1 < nb && j + 3 < nfull; j += 2) {
        block(p0, p1, bcb, bcq, j, std::true_type{});
        block(p1, p0, bcb, bcq, j + 1, std::true_type{});
    }
    for (; j + 1 < nb; j += 2) {
        block(p0, p1, bcb, bcq, j, std::false_type{});
        block(p1, p0, bcb, bcq, j + 1, std::false_type{});
    }
    if (j < nb) block(p0, p1, bcb, bcq, j, std::false_type{});

    if (seg + 1 < p.n_segs) {
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (p.publish) __hip_atomic_store(&hslot[(n0 + i) * kTile + tcol],
                               (static_cast<uint64_t>(seg + 1) << 32) | __float_as_uint(h[i]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else if (p.last && active) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) p.last[(b * dim + d) * N + n0 + i] = h[i];
    }
    __syncthreads();                                 // every wave is done with s_ticket
    }
}

// seqlen == 0: last_state = h0 (or 0)
__global__ __launch_bounds__(256) void copy_state_kernel(const float *h0, float *last, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) last[i] = h0 ? h0[i] : 0.0f;
}

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *w, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) w[i] = 0u;
}

template <int N, int NW, typename T, int FL, typename TX = T> hipError_t launch(const ScanArgs &a, hipStream_t s) {
    const Layout l = make_layout(a.batch, a.seqlen, a.dim, N, sizeof(TX) > sizeof(T) ? sizeof(TX) : sizeof(T));
    char *ws = static_cast<char *>(a.workspace);
    Params p;
    p.x = a.x; p.delta = a.delta; p.z = a.z; p.B = a.B; p.C = a.C;
    p.A = a.A; p.D = a.D; p.bias = a.delta_bias; p.h0 = a.h0;
    p.y = a.y; p.last = a.last_state;
    p.words = reinterpret_cast<uint32_t *>(ws);
    p.hbuf = reinterpret_cast<float *>(ws + l.hbuf_off);
    p.seqlen = a.seqlen; p.dim = a.dim;
    p.n_dt = l.n_dt; p.n_tiles = l.n_tiles; p.seg_len = l.seg_len; p.n_segs = l.n_segs;
    p.softplus = a.softplus;
    p.ckpt = nullptr;
    p.nblk = 0;
    p.spin_limit = a.test_spin_limit ? a.test_spin_limit : kSpinLimit;
    p.publish = a.test_spin_limit ? 0 : 1;
    const int64_t nclear = static_cast<int64_t>(l.hbuf_off / sizeof(uint32_t));   // ticket + progress
    hipLaunchKernelGGL(clear_words_kernel, dim3(static_cast<unsigned>((nclear + 255) / 256)), dim3(256), 0, s,
                       p.words, nclear);
    const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(l.n_tiles) * l.n_segs);
    hipLaunchKernelGGL((scan_fwd_kernel<N, NW, T, FL, TX>), dim3(grid), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
}

template <typename T, int FL, bool CK, bool REV = false, bool COL = false, bool CONV = false>
hipError_t launch_rows(const ScanArgs &a, hipStream_t s) {
    const Layout l = make_layout(a.batch, a.seqlen, a.dim, 16, sizeof(T));
    char *ws = static_cast<char *>(a.workspace);
    Params p;
    p.x = a.x; p.delta = a.delta; p.z = a.z; p.B = a.B; p.C = a.C;
    p.A = a.A; p.D = a.D; p.bias = a.delta_bias; p.h0 = a.h0;
    p.y = a.y; p.last = a.last_state;
    p.words = reinterpret_cast<uint32_t *>(ws);
    p.hbuf = reinterpret_cast<float *>(ws + l.hbuf_off);
    p.seqlen = a.seqlen; p.dim = a.dim;
    p.n_dt = l.n_dt; p.n_tiles = l.n_tiles; p.seg_len = l.seg_len; p.n_segs = l.n_segs;
    p.softplus = a.softplus;
    p.spin_limit = a.test_spin_limit ? a.test_spin_limit : kSpinLimit;
    p.publish = a.test_spin_limit ? 0 : 1;
    p.ckpt = a.ckpt;
    p.nblk = (a.seqlen + kRowTB - 1) / kRowTB;
    p.grid_h = static_cast<int>(a.grid_h);
    p.grid_w = static_cast<int>(a.grid_w);
    p.inv_h = a.grid_h > 0 ? 1.0f / static_cast<float>(a.grid_h) : 0.0f;
    p.conv_w = a.conv_w; p.conv_b = a.conv_b; p.conv_state = a.conv_state;
    p.conv_k = static_cast<int>(a.conv_k);
    // ticket, error word and the tagged carried states (tag 0 = not written)
    const int64_t nclear = static_cast<int64_t>(l.total / sizeof(uint32_t));
    hipLaunchKernelGGL(clear_words_kernel, dim3(static_cast<unsigned>((nclear + 255) / 256)), dim3(256), 0, s,
                       p.words, nclear);
    // persistent: one workgroup per CU (two with enough tiles), never more than jobs
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const int64_t jobs = static_cast<int64_t>(l.n_tiles) * l.n_segs;
    const int per_cu = l.n_tiles >= kRowsTilesPerCuForTwo * cus ? 2 * SSM_ROWS_WG_PER_CU : SSM_ROWS_WG_PER_CU;
    const int64_t workers = static_cast<int64_t>(cus) * per_cu;
    const unsigned grid = static_cast<unsigned>(jobs < workers ? jobs : workers);
    hipLaunchKernelGGL((scan_rows_kernel<T, FL, CK, REV, COL, CONV>), dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---- dispatch inside one translation unit's share
// d_state 16, forward order: the plain forward, its checkpointing form and
// the fused prologue.  With softplus and gate on (the Mamba layer) the kernel
// has both flags fixed at compile time.
template <typename T> hipError_t dispatch_rows_main(const ScanArgs &a, hipStream_t s) {
    const bool fl = a.softplus && a.z;
    if (a.conv_w)
        return fl ? launch_rows<T, 1, false, false, false, true>(a, s) : launch_rows<T, 0, false, false, false, true>(a, s);
    if (a.ckpt) return fl ? launch_rows<T, 1, true>(a, s) : launch_rows<T, 0, true>(a, s);
    return fl ? launch_rows<T, 1, false>(a, s) : launch_rows<T, 0, false>(a, s);
}
// d_state 16, the 2-D orders visited in place
template <typename T> hipError_t dispatch_rows_2d(const ScanArgs &a, hipStream_t s) {
    const bool fl = a.softplus && a.z;
    if (a.column_major && a.reverse)
        return fl ? launch_rows<T, 1, false, true, true>(a, s) : launch_rows<T, 0, false, true, true>(a, s);
    if (a.column_major)
        return fl ? launch_rows<T, 1, false, false, true>(a, s) : launch_rows<T, 0, false, false, true>(a, s);
    return fl ? launch_rows<T, 1, false, true>(a, s) : launch_rows<T, 0, false, true>(a, s);
}
// every other d_state; TX is x's storage type
template <typename T, typename TX> hipError_t dispatch_general(const ScanArgs &a, hipStream_t s) {
    switch (a.dstate) {
#define SSM_CASE(NN) \
    case NN: return launch<NN, waves_for<NN>(), T, 0, TX>(a, s);
        SSM_CASE(1) SSM_CASE(2) SSM_CASE(3) SSM_CASE(4) SSM_CASE(5) SSM_CASE(6) SSM_CASE(7)
        SSM_CASE(8) SSM_CASE(9) SSM_CASE(10) SSM_CASE(11) SSM_CASE(12) SSM_CASE(13)
        SSM_CASE(14) SSM_CASE(15)
#undef SSM_CASE
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// The shares, one per translation unit.
hipError_t scan_rows_main_bf16(const ScanArgs &a, hipStream_t s);
hipError_t scan_rows_main_f32(const ScanArgs &a, hipStream_t s);
hipError_t scan_rows_2d_bf16(const ScanArgs &a, hipStream_t s);
hipError_t scan_rows_2d_f32(const ScanArgs &a, hipStream_t s);
hipError_t scan_general_bf16(const ScanArgs &a, hipStream_t s);
hipError_t scan_general_bf16_xf32(const ScanArgs &a, hipStream_t s);
hipError_t scan_general_f32(const ScanArgs &a, hipStream_t s);

}  // namespace ssm
