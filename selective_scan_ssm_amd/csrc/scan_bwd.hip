// Backward of the selective scan: the gradient of
//   h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t,  y_t = (C_t . h_t + D x_t) SiLU(z_t),
//   Delta_t = softplus(delta_t + bias)
// with respect to every input, given dL/dy and dL/dlast_state.  The pages
// train through this scan (the youngju.dev guide's training loop calls
// loss.backward(); the "Windows SM1" page trains its scalar-state model with
// autograd) but print no backward: the kernels compute the exact reverse-mode
// derivative of the forward definition, statement by statement.
//
// Four launches:
//   1. checkpoints   -- the forward recurrence again, writing the state that
//                       enters every block of kBT steps and no output: the
//                       forward row kernel at d_state 16, ckpt_kernel else.
//   2. bwd_carry     -- the sequence of every (channel tile, batch row) is cut
//                       into S time segments.  For each segment but the first
//                       this pass runs the adjoint alone (no contributions)
//                       from zero at the segment's end to its start, and sums
//                       Delta over the segment.  The adjoint is linear, so the
//                       adjoint entering segment s from later times follows
//                       from these in a fixed order:
//                         carry_{S-1} = dL/dlast,
//                         carry_{s-1} = glocal_s + exp(A sum_s Delta) carry_s.
//   3. bwd_kernel    -- one workgroup per (tile, batch row, segment) walks the
//                       segment's blocks from last to first, starting from its
//                       carry.  For a block it recomputes the kBT states from
//                       the checkpoint (kept in registers), then runs the
//                       adjoint g = dL/dh backwards through them:
//                       g += dy C ;  contributions ;  g *= a.
//   4. bwd_reduce    -- sums the per-tile partials of dB, dC (over channel
//                       tiles) and of dA, dD, dbias (over batch rows and
//                       segments).
// The segments exist for the chip's sake: a sweep is sequential in time, and
// one workgroup per (tile, batch row) leaves most of the 256 CUs idle or
// alone (a lone workgroup issues at about two thirds of the rate of a pair).
// S is a function of the shape only, so results do not depend on the device.
//
// Work split of 1 and 2 (the forward general kernel's split): a workgroup of
// four waves owns 64 channels of one batch row (lane = channel) for the whole
// sequence; wave w owns states [w NPW, w NPW + NPW).  Per-(t, d) work (softplus,
// gate, their derivatives) is split over the waves by step and shared through
// LDS; the per-state partial sums (d Delta, dx and the readout needed by dz)
// meet in LDS and are added in a fixed order.  dB and dC sum over channels,
// i.e. over the 64 lanes: a butterfly reduce-scatter (v_permlane32_swap,
// v_permlane16_swap, then DPP row rotations and mirrors) leaves each lane one
// channel-sum, written as a per-tile partial.  Results are deterministic.
#include <mutex>

#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

constexpr int kBT = 16;        // steps per block
constexpr int kBWaves = 4;     // waves per workgroup
constexpr int kBTile = 64;     // channels per workgroup
constexpr int kBThreads = kBWaves * 64;

struct BwdParams {
    const void *x, *delta, *z, *B, *C, *dout;
    const float *A, *D, *bias, *h0, *dlast;
    void *dx, *ddelta, *dz;
    float *ckpt;        // (batch, nblk, dim, N): the state entering each block
    float *dBp, *dCp;   // (n_dt, batch, seqlen, N): per-tile channel sums
    float *dAp;         // (batch, dim, N)
    float *dDp, *dbp;   // (batch, dim)
    float *dh0;         // (batch, dim, N) or null
    float *glocal;      // (batch, S, dim, N): segment adjoints from zero (segments 1..S-1)
    float *sdelta;      // (batch, S, dim): sum of Delta over each segment
    int64_t seqlen, dim;
    int n_dt, nblk, N, softplus;
    int S, sblk;        // segments per sequence, blocks per segment (the last may be shorter)
};

__device__ __forceinline__ float sigmoid_f(float v) { return fast_rcp(1.0f + fast_exp2(-v * kLog2e)); }

// ---- lane exchange
__device__ __forceinline__ void bswap32(float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void bswap16(float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
constexpr int kDppRor8 = 0x128;        // row_ror:8   (lane i <-> i ^ 8 within a row)
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror (i <-> 7 - i within 8 lanes)
constexpr int kDppQuad2301 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppQuad1032 = 0xB1;     // quad_perm [1,0,3,2]
// (every pattern used here pairs lanes inside a row, so no source lane is out
// of bounds; bound_ctrl on lets the compiler fold the move into the add that
// consumes it, v_add_f32_dpp)
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// One butterfly stage inside a 16-lane row: lanes whose `bit` is 0 keep the
// lower half of the R values, the others the upper half, and each adds the
// matching half of its partner (the lane the DPP pattern pairs it with, which
// differs in `bit`).  Both pair sums are formed in every lane (own + partner,
// one DPP add each) and the lane keeps its half's: one select per kept value.
// With one value left the stage sums both lanes.
template <int R, int CTRL>
__device__ __forceinline__ void dpp_stage(float (&v)[R], float (&out)[R > 1 ? R / 2 : 1], bool upper) {
    if constexpr (R == 1) {
        out[0] = v[0] + dpp<CTRL>(v[0]);
    } else {
#pragma unroll
        for (int m = 0; m < R / 2; ++m) {
            const float lo = v[m] + dpp<CTRL>(v[m]);
            const float hi = v[m + R / 2] + dpp<CTRL>(v[m + R / 2]);
            out[m] = upper ? hi : lo;
        }
    }
}

// Sum over the 64 lanes of each of V values (V = 4, 8 or 16); lane l returns
// the total of value  l >> (6 - log2 V).
template <int V> __device__ __forceinline__ float wave_reduce_scatter(float (&v)[V]) {
    static_assert(V == 4 || V == 8 || V == 16, "V values per lane");
    const int lane = threadIdx.x & 63;
    float s32[V / 2];
#pragma unroll
    for (int m = 0; m < V / 2; ++m) {          // lanes 0-31 keep m, 32-63 keep m + V/2
        float a = v[m], b = v[m + V / 2];
        bswap32(a, b);
        s32[m] = a + b;
    }
    float s16[V / 4];
#pragma unroll
    for (int m = 0; m < V / 4; ++m) {          // rows 0, 2 keep m, rows 1, 3 keep m + V/4
        float a = s32[m], b = s32[m + V / 4];
        bswap16(a, b);
        s16[m] = a + b;
    }
    constexpr int R3 = V / 4;
    float s8[R3 > 1 ? R3 / 2 : 1];
    dpp_stage<R3, kDppRor8>(s16, s8, (lane >> 3) & 1);
    constexpr int R4 = R3 > 1 ? R3 / 2 : 1;
    float s4[R4 > 1 ? R4 / 2 : 1];
    dpp_stage<R4, kDppHalfMirror>(s8, s4, (lane >> 2) & 1);
    constexpr int R5 = R4 > 1 ? R4 / 2 : 1;
    float s2[1];
    static_assert(R5 == 1, "at most 16 values");
    dpp_stage<1, kDppQuad2301>(s4, s2, false);
    float s1[1];
    dpp_stage<1, kDppQuad1032>(s2, s1, false);
    return s1[0];
}

template <int NPW> struct PowV { static constexpr int v = (4 * NPW <= 4) ? 4 : (4 * NPW <= 8 ? 8 : 16); };

// ===========================================================================
// 1. checkpoints: the state entering each block
template <typename IO, int NPW>
__global__ __launch_bounds__(kBThreads) void ckpt_kernel(BwdParams p) {
    using M = typename MathFor<IO>::type;
    using R = typename Io<IO>::raw;
    constexpr uint32_t es = sizeof(IO);
    __shared__ float2 sDX[2][kBT][kBTile];            // (Delta, Delta x)
    __shared__ float sB[2][kBT][16];

    const int tid = threadIdx.x, lane = tid % 64;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    const int b = blockIdx.y;
    const int64_t T = p.seqlen, dim = p.dim;
    const int N = p.N;
    const int64_t ch = static_cast<int64_t>(blockIdx.x) * kBTile + lane;
    const bool active = ch < dim;
    const int64_t chc = active ? ch : dim - 1;

    float A2[NPW], h[NPW];
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int n = w * NPW + i;
        A2[i] = n < N ? M::prep_A(p.A[chc * N + n]) : 0.0f;
        h[i] = (n < N && p.h0 && active) ? p.h0[(b * dim + chc) * N + n] : 0.0f;
    }
    const float bias = p.bias ? p.bias[chc] : 0.0f;

    const int64_t row0 = static_cast<int64_t>(b) * T;
    const rsrc_t rx = make_rsrc(static_cast<const char *>(p.x) + row0 * dim * es, static_cast<uint32_t>(T * dim * es));
    const rsrc_t rd = make_rsrc(static_cast<const char *>(p.delta) + row0 * dim * es, static_cast<uint32_t>(T * dim * es));
    const rsrc_t rB = make_rsrc(static_cast<const char *>(p.B) + row0 * N * es, static_cast<uint32_t>(T * N * es));

    // wave w discretises steps 4w .. 4w+3 of a block; thread tid stages B of
    // step tid / 16, state tid % 16 (zero past N or past the sequence).  The
    // raw words of a block are loaded one block ahead of their conversion.
    struct Raw {
        R d[4], x[4];
        R b;
    };
    auto load_raw = [&](Raw &r, int blk) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t t = static_cast<int64_t>(blk) * kBT + 4 * w + k;
            const uint32_t vo = (active && t < T) ? static_cast<uint32_t>((t * dim + ch) * es) : kOffNone;
            r.x[k] = Io<IO>::load(rx, vo, 0);
            r.d[k] = Io<IO>::load(rd, vo, 0);
        }
        const int k = tid / 16, n = tid % 16;
        const int64_t t = static_cast<int64_t>(blk) * kBT + k;
        const uint32_t bo = (n < N && t < T) ? static_cast<uint32_t>((t * N + n) * es) : kOffNone;
        r.b = Io<IO>::load(rB, bo, 0);
    };
    auto produce = [&](const Raw &r, int blk, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int kk = 4 * w + k;
            const int64_t t = static_cast<int64_t>(blk) * kBT + kk;
            const bool in = active && t < T;
            const float xv = Io<IO>::f32(r.x[k]);
            const float v = Io<IO>::f32(r.d[k]) + bias;
            float dt = p.softplus ? M::softplus(v) : v;
            dt = in ? dt : 0.0f;
            sDX[buf][kk][lane] = make_float2(dt, dt * xv);
        }
        sB[buf][tid / 16][tid % 16] = Io<IO>::f32(r.b);
    };

    float *ck = p.ckpt + (static_cast<int64_t>(b) * p.nblk * dim + ch) * N;
    Raw raw;
    if (p.nblk > 0) {
        load_raw(raw, 0);
        produce(raw, 0, 0);
    }
    if (p.nblk > 1) load_raw(raw, 1);
    __syncthreads();
    for (int blk = 0; blk < p.nblk; ++blk) {
        const int cur = blk & 1;
        if (active) {
#pragma unroll
            for (int i = 0; i < NPW; ++i)
                if (w * NPW + i < N) ck[static_cast<int64_t>(blk) * dim * N + w * NPW + i] = h[i];
        }
#pragma unroll
        for (int k = 0; k < kBT; ++k) {
            const float2 q = sDX[cur][k][lane];
#pragma unroll
            for (int i = 0; i < NPW; ++i) h[i] = M::step(q.x * A2[i], h[i], q.y * sB[cur][k][w * NPW + i]);
        }
        if (blk + 1 < p.nblk) {
            produce(raw, blk + 1, cur ^ 1);          // loaded during this block's scan
            if (blk + 2 < p.nblk) load_raw(raw, blk + 2);
        }
        __syncthreads();
    }
}

// ===========================================================================
// 2. segment carries: the adjoint of each segment from zero at its end
//
// One workgroup per (tile, batch row, segment s >= 1), the sweep's work split:
// wave w owns states [w NPW, w NPW + NPW) of 64 channels (lane = channel) and
// discretises steps 4w .. 4w+3 of each block (Delta and dL/d(pre-gate y),
// shared through LDS, double buffered: one barrier per block).  Per step,
// latest first:  g += dy' C ;  g *= exp(Delta A)  -- the sweep's own adjoint
// without its contributions.
template <typename IO, int NPW, bool GATE>
__global__ __launch_bounds__(kBThreads) void bwd_carry_kernel(BwdParams p) {
    using M = typename MathFor<IO>::type;
    using R = typename Io<IO>::raw;
    constexpr uint32_t es = sizeof(IO);
    __shared__ float2 sG[2][kBT][kBTile];             // (Delta, dy')
    __shared__ float sC[2][kBT][16];
    __shared__ float sS[kBWaves][kBTile];

    const int tid = threadIdx.x, lane = tid % 64;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    const int b = blockIdx.y;
    const int seg = blockIdx.z + 1;
    const int64_t T = p.seqlen, dim = p.dim;
    const int N = p.N;
    constexpr bool gate = GATE;
    const int64_t ch = static_cast<int64_t>(blockIdx.x) * kBTile + lane;
    const bool active = ch < dim;
    const int64_t chc = active ? ch : dim - 1;
    const int blk_lo = seg * p.sblk;
    const int blk_hi = min(p.nblk, blk_lo + p.sblk);   // exclusive, > blk_lo

    float A2[NPW], g[NPW];
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int n = w * NPW + i;
        A2[i] = n < N ? M::prep_A(p.A[chc * N + n]) : 0.0f;
        g[i] = 0.0f;
    }
    const float bias = p.bias ? p.bias[chc] : 0.0f;

    const int64_t row0 = static_cast<int64_t>(b) * T;
    const uint32_t io_bytes = static_cast<uint32_t>(T * dim * es);
    const int64_t ebase = row0 * dim * es;
    const rsrc_t rd = make_rsrc(static_cast<const char *>(p.delta) + ebase, io_bytes);
    const rsrc_t rz = make_rsrc(static_cast<const char *>(gate ? p.z : p.delta) + ebase, io_bytes);
    const rsrc_t rg = make_rsrc(static_cast<const char *>(p.dout) + ebase, io_bytes);
    const rsrc_t rC = make_rsrc(static_cast<const char *>(p.C) + row0 * N * es, static_cast<uint32_t>(T * N * es));

    struct Raw {
        R d[4], z[4], g[4];
        R c;
    };
    auto load_raw = [&](Raw &r, int blk) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t t = static_cast<int64_t>(blk) * kBT + 4 * w + k;
            const uint32_t vo = (active && t < T) ? static_cast<uint32_t>((t * dim + ch) * es) : kOffNone;
            r.d[k] = Io<IO>::load(rd, vo, 0);
            r.z[k] = gate ? Io<IO>::load(rz, vo, 0) : R(0);
            r.g[k] = Io<IO>::load(rg, vo, 0);
        }
        const int k = tid / 16, n = tid % 16;
        const int64_t t = static_cast<int64_t>(blk) * kBT + k;
        const uint32_t co = (n < N && t < T) ? static_cast<uint32_t>((t * N + n) * es) : kOffNone;
        r.c = Io<IO>::load(rC, co, 0);
    };
    float dsum = 0.0f;                               // Delta over this wave's steps
    auto produce = [&](const Raw &r, int blk, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int kk = 4 * w + k;
            const int64_t t = static_cast<int64_t>(blk) * kBT + kk;
            const bool in = active && t < T;
            const float v = Io<IO>::f32(r.d[k]) + bias;
            float dt = p.softplus ? M::softplus(v) : v;
            float dy = Io<IO>::f32(r.g[k]);
            if (gate) {
                const float zv = Io<IO>::f32(r.z[k]);
                dy *= zv * sigmoid_f(zv);
            }
            dt = in ? dt : 0.0f;
            dy = in ? dy : 0.0f;
            dsum += dt;
            sG[buf][kk][lane] = make_float2(dt, dy);
        }
        sC[buf][tid / 16][tid % 16] = Io<IO>::f32(r.c);
    };

    // A block's sweep is short next to a load's latency, so the raw inputs
    // are loaded two blocks ahead, alternately into ra and rb: entering the
    // sweep of block blk, r holds block blk - 1 (converted into LDS after the
    // sweep) and the other set block blk - 2.
    auto iteration = [&](int blk, Raw &r) __attribute__((always_inline)) {
        const int cur = (blk_hi - 1 - blk) & 1;
#pragma unroll
        for (int k = kBT - 1; k >= 0; --k) {
            const float2 q = sG[cur][k][lane];
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
                g[i] = fmaf(q.y, sC[cur][k][w * NPW + i], g[i]);
                g[i] = M::apply(M::factor(q.x * A2[i]), g[i], 0.0f);
            }
        }
        if (blk > blk_lo) {
            produce(r, blk - 1, cur ^ 1);
            if (blk - 3 >= blk_lo) load_raw(r, blk - 3);
        }
        __syncthreads();
    };
    Raw ra, rb;
    load_raw(ra, blk_hi - 1);
    produce(ra, blk_hi - 1, 0);
    if (blk_hi - 2 >= blk_lo) load_raw(ra, blk_hi - 2);
    if (blk_hi - 3 >= blk_lo) load_raw(rb, blk_hi - 3);
    __syncthreads();
    for (int blk = blk_hi - 1; blk >= blk_lo; blk -= 2) {
        iteration(blk, ra);
        if (blk - 1 >= blk_lo) iteration(blk - 1, rb);
    }

    const int64_t row = static_cast<int64_t>(b) * p.S + seg;
    if (active) {
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int n = w * NPW + i;
            if (n < N) p.glocal[(row * dim + ch) * N + n] = g[i];
        }
    }
    sS[w][lane] = dsum;
    __syncthreads();
    if (w == 0 && active) {
        float t = 0.0f;
#pragma unroll
        for (int u = 0; u < kBWaves; ++u) t += sS[u][lane];
        p.sdelta[row * dim + ch] = t;
    }
}

// ===========================================================================
// 3. the reverse sweep
//
// Two waves per SIMD: two workgroups per CU (76 KB of LDS each), at most 256
// registers per lane.
constexpr int kBwdPerCU = 2;

template <typename IO, int NPW, bool GATE>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(kBwdPerCU, kBwdPerCU))) void bwd_kernel(BwdParams p) {
    using M = typename MathFor<IO>::type;
    using R = typename Io<IO>::raw;
    constexpr uint32_t es = sizeof(IO);
    constexpr int V = PowV<NPW>::v;                   // dB / dC values per 4-step chunk, padded
    __shared__ float4 sP[kBT][kBTile];                // (Delta, Delta x, dL/d(pre-gate y), x)
    __shared__ float2 sE[kBT][kBTile];                // (dDelta/d(delta), dL/dz per unit pre-gate y)
    __shared__ float sB[kBT][16], sC[kBT][16];
    __shared__ float2 sQ[kBWaves][kBT][kBTile];       // per-wave (dL/dDelta, dx) partials
    __shared__ float sY[kBWaves][kBT][kBTile];        // per-wave readout partials (for dz)
    __shared__ float2 sAcc[kBWaves][kBTile];

    const int tid = threadIdx.x, lane = tid % 64;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    const int b = blockIdx.y;
    const int64_t T = p.seqlen, dim = p.dim;
    const int N = p.N;
    constexpr bool gate = GATE;
    const int64_t ch = static_cast<int64_t>(blockIdx.x) * kBTile + lane;
    const bool active = ch < dim;
    const int64_t chc = active ? ch : dim - 1;

    const int seg = blockIdx.z;
    const int blk_lo = seg * p.sblk;
    const int blk_hi = min(p.nblk, blk_lo + p.sblk);     // exclusive

    float A2[NPW], Ar[NPW], g[NPW], dA[NPW];
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int n = w * NPW + i;
        const bool vn = n < N;
        Ar[i] = vn ? p.A[chc * N + n] : 0.0f;
        A2[i] = M::prep_A(Ar[i]);
        g[i] = (vn && active && p.dlast) ? p.dlast[(b * dim + chc) * N + n] : 0.0f;
        dA[i] = 0.0f;
    }
    // the adjoint entering this segment from later times, later segments first
    for (int j = p.S - 1; j > seg; --j) {
        const int64_t row = static_cast<int64_t>(b) * p.S + j;
        const float sd = p.sdelta[row * dim + chc];
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int n = w * NPW + i;
            const float gl = n < N ? p.glocal[(row * dim + chc) * N + n] : 0.0f;
            g[i] = M::apply(M::factor(sd * A2[i]), g[i], gl);
        }
    }
    const float bias = p.bias ? p.bias[chc] : 0.0f;
    const float Dd = p.D ? p.D[chc] : 0.0f;

    const int64_t row0 = static_cast<int64_t>(b) * T;
    const uint32_t io_bytes = static_cast<uint32_t>(T * dim * es);
    const int64_t ebase = row0 * dim * es;
    const rsrc_t rx = make_rsrc(static_cast<const char *>(p.x) + ebase, io_bytes);
    const rsrc_t rd = make_rsrc(static_cast<const char *>(p.delta) + ebase, io_bytes);
    const rsrc_t rz = make_rsrc(static_cast<const char *>(gate ? p.z : p.x) + ebase, io_bytes);
    const rsrc_t rg = make_rsrc(static_cast<const char *>(p.dout) + ebase, io_bytes);
    const rsrc_t rdx = make_rsrc(static_cast<char *>(p.dx) + ebase, io_bytes);
    const rsrc_t rdd = make_rsrc(static_cast<char *>(p.ddelta) + ebase, io_bytes);
    const rsrc_t rdz = make_rsrc(static_cast<char *>(gate ? p.dz : p.dx) + ebase, gate ? io_bytes : 0u);
    const uint32_t bc_bytes = static_cast<uint32_t>(T * N * es);
    const rsrc_t rB = make_rsrc(static_cast<const char *>(p.B) + row0 * N * es, bc_bytes);
    const rsrc_t rC = make_rsrc(static_cast<const char *>(p.C) + row0 * N * es, bc_bytes);
    // checkpoints of batch row b; one block's (dim x N fp32, < 2 GiB) are read
    // through a descriptor of their own, lane offsets out of range for
    // inactive lanes (loads return 0, no branch)
    const float *ckrow = p.ckpt + static_cast<int64_t>(b) * p.nblk * dim * N;
    const uint32_t ck_bytes = static_cast<uint32_t>(dim * N * 4);
    const uint32_t ck_off = active ? static_cast<uint32_t>((ch * N + w * NPW) * 4) : kOffNone;

    // raw inputs of wave w's four steps of a block, B / C of (step tid/16,
    // state tid%16), and the checkpoint of the block
    struct Raw {
        R d[4], x[4], z[4], g[4];
        R b, c;
        float ck[NPW];
    };
    auto step_off = [&](int blk, int k) __attribute__((always_inline)) -> uint32_t {
        const int64_t t = static_cast<int64_t>(blk) * kBT + 4 * w + k;
        return (active && t < T) ? static_cast<uint32_t>((t * dim + ch) * es) : kOffNone;
    };
    auto load_raw = [&](Raw &r, int blk) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t vo = step_off(blk, k);
            r.d[k] = Io<IO>::load(rd, vo, 0);
            r.x[k] = Io<IO>::load(rx, vo, 0);
            r.z[k] = gate ? Io<IO>::load(rz, vo, 0) : R(0);
            r.g[k] = Io<IO>::load(rg, vo, 0);
        }
        const int k = tid / 16, n = tid % 16;
        const int64_t t = static_cast<int64_t>(blk) * kBT + k;
        const uint32_t bo = (n < N && t < T) ? static_cast<uint32_t>((t * N + n) * es) : kOffNone;
        r.b = Io<IO>::load(rB, bo, 0);
        r.c = Io<IO>::load(rC, bo, 0);
        const rsrc_t rck = make_rsrc(ckrow + static_cast<int64_t>(blk) * dim * N, ck_bytes);
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const float v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rck, ck_off + 4 * i, 0, 0));
            r.ck[i] = w * NPW + i < N ? v : 0.0f;
        }
    };
    // per-(t, d) discretisation of wave w's steps, and B / C staging
    auto produce = [&](const Raw &r, int blk) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int kk = 4 * w + k;
            const int64_t t = static_cast<int64_t>(blk) * kBT + kk;
            const bool in = active && t < T;
            const float xv = Io<IO>::f32(r.x[k]);
            const float v = Io<IO>::f32(r.d[k]) + bias;
            float dt = p.softplus ? M::softplus(v) : v;
            const float dsp = p.softplus ? sigmoid_f(v) : 1.0f;     // dDelta / d(delta)
            const float dout = Io<IO>::f32(r.g[k]);
            float dy = dout, ez = 0.0f;
            if (gate) {
                // y = y_pre SiLU(z): dL/dy_pre = dout SiLU(z), and
                // dL/dz = dout y_pre s (1 + z (1 - s)), s = sigmoid(z)
                const float zv = Io<IO>::f32(r.z[k]);
                const float sz = sigmoid_f(zv);
                dy *= zv * sz;
                ez = dout * sz * fmaf(zv, 1.0f - sz, 1.0f);
            }
            dt = in ? dt : 0.0f;
            dy = in ? dy : 0.0f;
            sP[kk][lane] = make_float4(dt, dt * xv, dy, xv);
            sE[kk][lane] = make_float2(dsp, ez);
        }
        sB[tid / 16][tid % 16] = Io<IO>::f32(r.b);
        sC[tid / 16][tid % 16] = Io<IO>::f32(r.c);
    };

    float dD_acc = 0.0f, db_acc = 0.0f;
    // the partial sums of dB / dC of one 4-step chunk, reduced over the 64
    // channels and written as this tile's partial
    const int64_t part0 = (static_cast<int64_t>(blockIdx.x) * gridDim.y + b) * T * N;
    auto flush = [&](float (&vals)[V], float *dst, int blk, int kc) __attribute__((always_inline)) {
        const float s = wave_reduce_scatter<V>(vals);
        constexpr int shift = V == 16 ? 2 : (V == 8 ? 3 : 4);
        const int idx = lane >> shift;
        const int kk = idx / NPW, i = idx % NPW;
        const int64_t t = static_cast<int64_t>(blk) * kBT + 4 * kc + kk;
        const int n = w * NPW + i;
        if ((lane & ((1 << shift) - 1)) == 0 && idx < 4 * NPW && n < N && t < T) dst[part0 + t * N + n] = s;
    };

    // steps [s0, s0 + kBT/2) of block blk from the state hin entering them:
    // recompute and keep the states and decay factors, write the readout
    // partials, then run the adjoint back through them
    auto sweep_half = [&](int s0, const float (&hin)[NPW], int blk) __attribute__((always_inline)) {
        constexpr int H = kBT / 2;
        float hs[H + 1][NPW], fk[H][NPW];
#pragma unroll
        for (int i = 0; i < NPW; ++i) hs[0][i] = hin[i];
#pragma unroll
        for (int k = 0; k < H; ++k) {
            const float4 q = sP[s0 + k][lane];
            float yv = 0.0f;
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
                fk[k][i] = M::factor(q.x * A2[i]);
                hs[k + 1][i] = M::apply(fk[k][i], hs[k][i], q.y * sB[s0 + k][w * NPW + i]);
                yv = fmaf(sC[s0 + k][w * NPW + i], hs[k + 1][i], yv);
            }
            if (gate) sY[w][s0 + k][lane] = yv;
        }
#pragma unroll
        for (int kc = H / 4 - 1; kc >= 0; --kc) {
            float vB[V], vC[V];
#pragma unroll
            for (int m = 0; m < V; ++m) vB[m] = vC[m] = 0.0f;
#pragma unroll
            for (int kk = 3; kk >= 0; --kk) {
                const int k = 4 * kc + kk, st = s0 + k;
                const float4 q = sP[st][lane];           // Delta, Delta x, dy, x
                // dL/dDelta = sum_n g (A a h_{t-1}) + x sum_n g B, dx = Delta sum_n g B
                float ddt = 0.0f, sgb = 0.0f;
#pragma unroll
                for (int i = 0; i < NPW; ++i) {
                    const float bk = sB[st][w * NPW + i], ck = sC[st][w * NPW + i];
                    g[i] = fmaf(q.z, ck, g[i]);                      // dL/dh_t
                    sgb = fmaf(g[i], bk, sgb);
                    vB[kk * NPW + i] = g[i] * q.y;
                    vC[kk * NPW + i] = q.z * hs[k + 1][i];
                    g[i] = M::apply(fk[k][i], g[i], 0.0f);           // dL/dh_{t-1} = a_t dL/dh_t
                    // dL/d(Delta A) of this step: g a_t h_{t-1}, i.e. the
                    // decayed adjoint times the previous state
                    const float qa = g[i] * hs[k][i];
                    ddt = fmaf(qa, Ar[i], ddt);
                    dA[i] = fmaf(qa, q.x, dA[i]);
                }
                sQ[w][st][lane] = make_float2(fmaf(sgb, q.w, ddt), sgb * q.x);
            }
            flush(vB, p.dBp, blk, s0 / 4 + kc);
            flush(vC, p.dCp, blk, s0 / 4 + kc);
        }
    };

    // one set of raw inputs: those of the next block (earlier in time) are in
    // flight during a block's sweep and converted into LDS after it; what the
    // per-step finish needs was staged by produce, the checkpoint kept apart
    Raw raw;
    float ck[NPW];
    if (blk_hi > blk_lo) {
        load_raw(raw, blk_hi - 1);
        produce(raw, blk_hi - 1);
    }
#pragma unroll
    for (int i = 0; i < NPW; ++i) ck[i] = raw.ck[i];
    __syncthreads();
    for (int blk = blk_hi - 1; blk >= blk_lo; --blk) {
        if (blk > blk_lo) load_raw(raw, blk - 1);   // in flight during the sweep

        // ---- the block in two halves of kBT / 2 steps, the later half first:
        // the state entering the later half is recomputed (not kept) from the
        // checkpoint, then each half keeps its states and decay factors in
        // registers while the adjoint runs back through it
        float hmid[NPW];
#pragma unroll
        for (int i = 0; i < NPW; ++i) hmid[i] = ck[i];
#pragma unroll
        for (int k = 0; k < kBT / 2; ++k) {
            const float4 q = sP[k][lane];
#pragma unroll
            for (int i = 0; i < NPW; ++i) hmid[i] = M::step(q.x * A2[i], hmid[i], q.y * sB[k][w * NPW + i]);
        }
        sweep_half(kBT / 2, hmid, blk);
        sweep_half(0, ck, blk);
        __syncthreads();

        // ---- finish wave w's steps: sum the four waves' partials in order
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int kk = 4 * w + k;
            const int64_t t = static_cast<int64_t>(blk) * kBT + kk;
            const bool in = active && t < T;
            const float4 q = sP[kk][lane];
            const float2 e = sE[kk][lane];
            float ddt = 0.0f, dxs = 0.0f, yv = 0.0f;
#pragma unroll
            for (int u = 0; u < kBWaves; ++u) {
                const float2 s = sQ[u][kk][lane];
                ddt += s.x;
                dxs += s.y;
                if (gate) yv += sY[u][kk][lane];
            }
            const float dv = ddt * e.x;
            const float dxv = fmaf(q.z, Dd, dxs);
            const uint32_t vo = step_off(blk, k);
            Io<IO>::store(dxv, rdx, vo, 0);
            Io<IO>::store(dv, rdd, vo, 0);
            if (gate) Io<IO>::store(e.y * fmaf(Dd, q.w, yv), rdz, vo, 0);   // dL/dz
            if (in) {
                dD_acc = fmaf(q.z, q.w, dD_acc);
                db_acc += dv;
            }
        }
        if (blk > blk_lo) {
            produce(raw, blk - 1);
#pragma unroll
            for (int i = 0; i < NPW; ++i) ck[i] = raw.ck[i];
        }
        __syncthreads();
    }

    // ---- per-chain and per-(b, d) results: partials of this segment; the
    // first segment's final adjoint is dL/dh0
    const int64_t prow = static_cast<int64_t>(b) * p.S + seg;
    if (active) {
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int n = w * NPW + i;
            if (n < N) {
                p.dAp[(prow * dim + ch) * N + n] = dA[i];
                if (p.dh0 && seg == 0) p.dh0[(b * dim + ch) * N + n] = g[i];
            }
        }
    }
    sAcc[w][lane] = make_float2(dD_acc, db_acc);
    __syncthreads();
    if (w == 0 && active) {
        float sd = 0.0f, sb = 0.0f;
#pragma unroll
        for (int u = 0; u < kBWaves; ++u) {
            sd += sAcc[u][lane].x;
            sb += sAcc[u][lane].y;
        }
        p.dDp[prow * dim + ch] = sd;
        p.dbp[prow * dim + ch] = sb;
    }
}

// ===========================================================================
// 4. reductions: dB, dC over the channel tiles; dA, dD, dbias over the rows
// of partials (batch row x segment)
struct ReduceParams {
    const float *dBp, *dCp, *dAp, *dDp, *dbp;
    void *dB, *dC;
    float *dA, *dD, *dbias;
    int64_t n_btn, n_dn, dim;
    int n_dt, rows;          // rows of dA / dD / dbias partials: batch x segments
};

template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(ReduceParams r) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < r.n_btn; e += stride) {
        float sb = 0.0f, sc = 0.0f;
        for (int j = 0; j < r.n_dt; ++j) {
            sb += r.dBp[j * r.n_btn + e];
            sc += r.dCp[j * r.n_btn + e];
        }
        static_cast<T *>(r.dB)[e] = from_f32<T>(sb);
        static_cast<T *>(r.dC)[e] = from_f32<T>(sc);
    }
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < r.n_dn; e += stride) {
        float s = 0.0f;
        for (int bb = 0; bb < r.rows; ++bb) s += r.dAp[bb * r.n_dn + e];
        r.dA[e] = s;
    }
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < r.dim; e += stride) {
        float sd = 0.0f, sb = 0.0f;
        for (int bb = 0; bb < r.rows; ++bb) {
            sd += r.dDp[bb * r.dim + e];
            sb += r.dbp[bb * r.dim + e];
        }
        if (r.dD) r.dD[e] = sd;
        if (r.dbias) r.dbias[e] = sb;
    }
}

// ---- segments
// Cost model of a segmentation, in units of one block swept by one of a pair
// of workgroups sharing a CU: rounds of kBwdCUs x per_cu workgroups, a lone
// workgroup on a CU at 1.58 / 2 of a pair's time (measured: one workgroup per
// CU runs 1.58x slower per unit of work than two), a prologue of about a
// quarter block plus the carry combination, and the carry pass at about a
// fifth of the sweep per block it covers.  S depends on the shape only.
constexpr int kBwdCUs = 256;
constexpr int kBwdMaxSeg = 64;
struct BwdPlan {
    int S, sblk;
};
BwdPlan bwd_plan(int64_t units0, int64_t nblk, int per_cu) {
    BwdPlan best{1, static_cast<int>(nblk)};
    if (nblk <= 1 || units0 <= 0) return best;
    const int64_t slots = static_cast<int64_t>(kBwdCUs) * per_cu;
    double best_cost = 0.0;
    const int64_t smax = nblk < kBwdMaxSeg ? nblk : kBwdMaxSeg;
    for (int64_t S = 1; S <= smax; ++S) {
        const int64_t sblk = (nblk + S - 1) / S;
        if ((nblk + sblk - 1) / sblk != S) continue;   // the same split as a smaller S
        const int64_t units = units0 * S;
        const int64_t full = units / slots, rem = units % slots;
        const double rounds = static_cast<double>(full) +
                              (rem == 0 ? 0.0 : ((per_cu == 2 && rem <= kBwdCUs) ? 0.79 : 1.0));
        const double cost = rounds * (static_cast<double>(sblk) + 0.25 + 0.02 * static_cast<double>(S)) +
                            0.2 * static_cast<double>(units0) * static_cast<double>(nblk - sblk) /
                                static_cast<double>(slots);
        if (S == 1 || cost < best_cost - 1e-9) {
            best_cost = cost;
            best = BwdPlan{static_cast<int>(S), static_cast<int>(sblk)};
        }
    }
    return best;
}

// ---- the side stream
// When the backward computes its own checkpoints, the carry pass (which reads
// delta, z, dL/dy and C) does not depend on them and runs beside the
// checkpoint pass on a library-owned stream of each device, at the default
// priority.  The checkpoint pass is one persistent workgroup per CU (116
// registers, 21 KB of LDS), so up to two carry workgroups share each CU with it
// and use issue slots a lone wave per SIMD leaves idle.  The fork and the join
// are events recorded on the caller's stream and on the side stream; the whole
// enqueue sequence of one call runs under a lock, so concurrent calls from
// several host threads cannot interleave their fork and join records.
constexpr int kMaxDevices = 64;
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// the current device's side stream and events, created on first use unless
// `create` is false (then *out is null when they do not exist yet); the
// caller holds g_side_mu
hipError_t side_stream(SideStream **out, bool create) {
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    SideStream &ss = g_side[dev];
    if (!ss.stream) {
        if (!create) return hipSuccess;
        hipStream_t st = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        if ((e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&f, hipEventDisableTiming)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&j, hipEventDisableTiming)) != hipSuccess) {
            if (f) (void)hipEventDestroy(f);
            (void)hipStreamDestroy(st);
            return e;
        }
        ss.stream = st;
        ss.fork = f;
        ss.join = j;
    }
    *out = &ss;
    return hipSuccess;
}

// ---- workspace
struct BwdLayout {
    int64_t nblk, n_dt;
    BwdPlan plan;
    size_t fwd_off, fwd_bytes, ckpt_off, dBp_off, dCp_off, dAp_off, dDp_off, dbp_off, gl_off, sd_off, total;
};
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
// At d_state 16 the checkpoints come from the forward row kernel (run with no
// y), which needs its own workspace; other widths use ckpt_kernel.
bool ckpt_by_forward(int64_t N) { return N == 16; }
ScanArgs ckpt_forward_args(int64_t batch, int64_t seqlen, int64_t dim, int64_t N, int bf16) {
    ScanArgs f{};
    f.batch = batch; f.seqlen = seqlen; f.dim = dim; f.dstate = N; f.bf16 = bf16;
    return f;
}
BwdLayout bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t N, int bf16) {
    BwdLayout l;
    l.nblk = (seqlen + kBT - 1) / kBT;
    l.n_dt = (dim + kBTile - 1) / kBTile;
    l.plan = bwd_plan(l.n_dt * batch, l.nblk, kBwdPerCU);
    const size_t rows = size_t(batch) * l.plan.S;
    size_t o = 0;
    l.fwd_off = 0;
    l.fwd_bytes = (ckpt_by_forward(N) && batch > 0 && dim > 0 && seqlen > 0)
                      ? scan_fwd_workspace(ckpt_forward_args(batch, seqlen, dim, N, bf16)) : 0;
    o = align256(l.fwd_bytes);
    l.ckpt_off = o; o = align256(o + sizeof(float) * size_t(batch) * l.nblk * dim * N);
    l.dBp_off = o;  o = align256(o + sizeof(float) * size_t(l.n_dt) * batch * seqlen * N);
    l.dCp_off = o;  o = align256(o + sizeof(float) * size_t(l.n_dt) * batch * seqlen * N);
    l.dAp_off = o;  o = align256(o + sizeof(float) * rows * dim * N);
    l.dDp_off = o;  o = align256(o + sizeof(float) * rows * dim);
    l.dbp_off = o;  o = align256(o + sizeof(float) * rows * dim);
    const size_t grows = l.plan.S > 1 ? rows : 0;
    l.gl_off = o;   o = align256(o + sizeof(float) * grows * dim * N);
    l.sd_off = o;   o = align256(o + sizeof(float) * grows * dim);
    l.total = o;
    return l;
}

template <typename T, int NPW> hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s) {
    const BwdLayout l = bwd_layout(a.batch, a.seqlen, a.dim, a.dstate, a.bf16);
    // batch == 0 or d_inner == 0 leaves only the reduction, which writes the
    // zero sums (dB, dC over no channel, dA, dD, dbias over no batch row)
    char *ws = static_cast<char *>(a.workspace);
    BwdParams p;
    p.x = a.x; p.delta = a.delta; p.z = a.z; p.B = a.B; p.C = a.C; p.dout = a.dout;
    p.A = a.A; p.D = a.D; p.bias = a.delta_bias; p.h0 = a.h0; p.dlast = a.dlast;
    p.dx = a.dx; p.ddelta = a.ddelta; p.dz = a.dz;
    // checkpoints recorded by the caller's forward, or computed here
    p.ckpt = a.ckpt_in ? const_cast<float *>(a.ckpt_in) : reinterpret_cast<float *>(ws + l.ckpt_off);
    p.dBp = reinterpret_cast<float *>(ws + l.dBp_off);
    p.dCp = reinterpret_cast<float *>(ws + l.dCp_off);
    p.dAp = reinterpret_cast<float *>(ws + l.dAp_off);
    p.dDp = reinterpret_cast<float *>(ws + l.dDp_off);
    p.dbp = reinterpret_cast<float *>(ws + l.dbp_off);
    p.dh0 = a.dh0;
    p.glocal = reinterpret_cast<float *>(ws + l.gl_off);
    p.sdelta = reinterpret_cast<float *>(ws + l.sd_off);
    p.seqlen = a.seqlen; p.dim = a.dim;
    p.n_dt = static_cast<int>(l.n_dt); p.nblk = static_cast<int>(l.nblk);
    p.N = static_cast<int>(a.dstate); p.softplus = a.softplus;
    p.S = l.plan.S; p.sblk = l.plan.sblk;
    if (l.n_dt > 0 && a.batch > 0) {
        const dim3 grid(static_cast<unsigned>(l.n_dt), static_cast<unsigned>(a.batch));
        const dim3 cgrid(static_cast<unsigned>(l.n_dt), static_cast<unsigned>(a.batch),
                         static_cast<unsigned>(p.S - 1));
        auto launch_carry = [&](hipStream_t st) {
            if (a.z) hipLaunchKernelGGL((bwd_carry_kernel<T, NPW, true>), cgrid, dim3(kBThreads), 0, st, p);
            else hipLaunchKernelGGL((bwd_carry_kernel<T, NPW, false>), cgrid, dim3(kBThreads), 0, st, p);
            return hipGetLastError();
        };
        // the carry pass beside the checkpoint pass (side stream), or before
        // the sweep on the caller's stream when the checkpoints are given
        std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
        SideStream *side = nullptr;
        bool beside = p.S > 1 && !a.ckpt_in;
        // once the carry pass is on the side stream, the caller's stream waits
        // for it on every way out, errors included (the caller may free the
        // buffers it reads as soon as its stream says so)
        bool forked = false;
        auto join = [&]() -> hipError_t {
            if (!forked) return hipSuccess;
            forked = false;
            const hipError_t e = hipStreamWaitEvent(s, side->join, 0);
            side_lock.unlock();
            return e;
        };
        if (beside) {
            // creating a stream or an event may be refused while `s` is being
            // captured into a graph: a capture before any uncaptured call on
            // this device runs the carry pass on `s` instead
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            hipError_t e = hipStreamIsCapturing(s, &cs);
            if (e != hipSuccess) return e;
            side_lock.lock();
            e = side_stream(&side, cs == hipStreamCaptureStatusNone);
            if (e != hipSuccess) return e;
            beside = side != nullptr;
        }
        if (beside) {
            hipError_t e = hipEventRecord(side->fork, s);
            if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
            if (e == hipSuccess) e = launch_carry(side->stream);
            if (e == hipSuccess) {
                e = hipEventRecord(side->join, side->stream);
                if (e != hipSuccess) (void)hipStreamSynchronize(side->stream);
            }
            if (e != hipSuccess) return e;
            forked = true;
        }
        if (a.ckpt_in) {
            // nothing to do: the forward recorded them
        } else if (ckpt_by_forward(a.dstate)) {
            ScanArgs f = ckpt_forward_args(a.batch, a.seqlen, a.dim, a.dstate, a.bf16);
            f.x = a.x; f.delta = a.delta; f.z = a.z; f.B = a.B; f.C = a.C;
            f.delta_bias = a.delta_bias; f.A = a.A; f.D = a.D; f.h0 = a.h0;
            f.y = nullptr; f.last_state = nullptr;
            f.softplus = a.softplus;
            f.workspace = ws + l.fwd_off; f.workspace_bytes = l.fwd_bytes;
            f.ckpt = p.ckpt;
            if (a.seqlen > 0) {
                const hipError_t e = launch_scan_fwd(f, s);
                if (e != hipSuccess) {
                    (void)join();
                    return e;
                }
            }
        } else {
            hipLaunchKernelGGL((ckpt_kernel<T, NPW>), grid, dim3(kBThreads), 0, s, p);
        }
        if (beside) {
            const hipError_t e = join();
            if (e != hipSuccess) return e;
        } else if (p.S > 1) {
            if (side_lock.owns_lock()) side_lock.unlock();
            const hipError_t e = launch_carry(s);
            if (e != hipSuccess) return e;
        }
        const dim3 sgrid(static_cast<unsigned>(l.n_dt), static_cast<unsigned>(a.batch),
                         static_cast<unsigned>(p.S));
        if (a.z) hipLaunchKernelGGL((bwd_kernel<T, NPW, true>), sgrid, dim3(kBThreads), 0, s, p);
        else hipLaunchKernelGGL((bwd_kernel<T, NPW, false>), sgrid, dim3(kBThreads), 0, s, p);
    }
    ReduceParams r;
    r.dBp = p.dBp; r.dCp = p.dCp; r.dAp = p.dAp; r.dDp = p.dDp; r.dbp = p.dbp;
    r.dB = a.dB; r.dC = a.dC; r.dA = a.dA; r.dD = a.dD; r.dbias = a.ddelta_bias;
    r.n_btn = a.batch * a.seqlen * a.dstate;
    r.n_dn = a.dim * a.dstate;
    r.dim = a.dim;
    r.n_dt = static_cast<int>(l.n_dt);
    r.rows = static_cast<int>(a.batch * l.plan.S);
    const int64_t most = r.n_btn > r.n_dn ? r.n_btn : r.n_dn;
    const int64_t blocks = (most + 255) / 256;
    hipLaunchKernelGGL(bwd_reduce_kernel<T>, dim3(static_cast<unsigned>(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096)),
                       dim3(256), 0, s, r);
    return hipGetLastError();
}

// the checkpoint pass alone, for a forward that records them at d_state != 16
template <typename T, int NPW> hipError_t launch_ckpt_t(const ScanArgs &f, hipStream_t s) {
    BwdParams p{};
    p.x = f.x; p.delta = f.delta; p.B = f.B;
    p.A = f.A; p.bias = f.delta_bias; p.h0 = f.h0;
    p.ckpt = f.ckpt;
    p.seqlen = f.seqlen; p.dim = f.dim;
    const int64_t n_dt = (f.dim + kBTile - 1) / kBTile;
    p.n_dt = static_cast<int>(n_dt);
    p.nblk = static_cast<int>((f.seqlen + kBT - 1) / kBT);
    p.N = static_cast<int>(f.dstate); p.softplus = f.softplus;
    const dim3 grid(static_cast<unsigned>(n_dt), static_cast<unsigned>(f.batch));
    hipLaunchKernelGGL((ckpt_kernel<T, NPW>), grid, dim3(kBThreads), 0, s, p);
    return hipGetLastError();
}

template <typename T> hipError_t launch_ckpt_npw(const ScanArgs &f, hipStream_t s) {
    switch ((f.dstate + 3) / 4) {
    case 1: return launch_ckpt_t<T, 1>(f, s);
    case 2: return launch_ckpt_t<T, 2>(f, s);
    case 3: return launch_ckpt_t<T, 3>(f, s);
    default: return launch_ckpt_t<T, 4>(f, s);
    }
}

template <typename T> hipError_t launch_bwd_npw(const BwdArgs &a, hipStream_t s) {
    switch ((a.dstate + 3) / 4) {
    case 1: return launch_bwd_t<T, 1>(a, s);
    case 2: return launch_bwd_t<T, 2>(a, s);
    case 3: return launch_bwd_t<T, 3>(a, s);
    default: return launch_bwd_t<T, 4>(a, s);
    }
}

}  // namespace

size_t scan_bwd_workspace(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int bf16) {
    return bwd_layout(batch, seqlen, dim, dstate, bf16).total;
}

void scan_bwd_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int bf16, int *segments,
                   int *blocks_per_segment) {
    const BwdLayout l = bwd_layout(batch, seqlen, dim, dstate, bf16);
    *segments = l.plan.S;
    *blocks_per_segment = l.plan.sblk;
}

hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t s) {
    return a.bf16 ? launch_bwd_npw<bf16_t>(a, s) : launch_bwd_npw<float>(a, s);
}

hipError_t launch_scan_fwd_ckpt(const ScanArgs &a, hipStream_t s) {
    // d_state 16: the row kernel writes y, last_state and the checkpoints in one pass
    if (ckpt_by_forward(a.dstate)) return launch_scan_fwd(a, s);
    ScanArgs f = a;
    f.ckpt = nullptr;
    const hipError_t e = launch_scan_fwd(f, s);
    if (e != hipSuccess || a.batch == 0 || a.dim == 0 || a.seqlen == 0) return e;
    return a.bf16 ? launch_ckpt_npw<bf16_t>(a, s) : launch_ckpt_npw<float>(a, s);
}

}  // namespace ssm
