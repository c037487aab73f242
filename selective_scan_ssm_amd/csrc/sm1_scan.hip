// d_state = 1 forward scan ("SM1", the scalar-state Mamba-1 scan of the
// "Windows SM1 (Scalar Mamba1)" page: h_t = dA_t h_{t-1} + dBx_t, y = h C,
// whose closed form is a cumulative product and a cumulative sum).
//
// With one state per channel there are only batch * d_inner independent
// chains (12288 at the 130M shape): walking each chain through time on one
// lane leaves most of the chip idle, so time is split.  One step is the
// affine map h -> f h + u, and such maps compose associatively:
//     (P1, H1) then (P2, H2)  =  (P2 P1, P2 H1 + H2),  identity (1, 0)
// (the (decay, offset) operator behind the parallel scan of the youngju.dev
// guide, section 5 "Hardware-Aware Algorithm").  Because A is diagonal, the
// decay of a run of steps is exp(A * sum Delta): one exp per run.
//
// Work split.  A workgroup owns 64 consecutive channels of one batch row for
// the whole sequence and walks it in rounds of 128 steps:
//   * lane = channel, so every load and store instruction of a wave moves one
//     contiguous row segment (256 bytes fp32, 128 bytes bf16); wave w of the
//     16 takes sub-chunk w of the round, 8 consecutive steps;
//   * pass 1: each lane discretises its 8 steps (softplus, decay factor,
//     Delta B x), keeps them in registers and folds them into its sub-chunk's
//     aggregate (P, H);
//   * the 16 aggregates of a channel meet in LDS; every lane folds the ones
//     before its sub-chunk into the state entering the round, which gives its
//     own incoming state, and all 16 into the state leaving the round (the
//     carry, kept in a register: no workgroup ever waits on another);
//   * pass 2 replays the 8 steps from the incoming state and writes
//     y = (C h + D x) SiLU(z).
// The next round's delta, x and z are loaded while the current one computes;
// B and C of a round are widened once into LDS two rounds ahead.  Every input
// byte is read once and every output byte written once; one barrier per round.
// Full-row accesses matter more here than filling every CU: at the SM1
// workload the 192 workgroups of 16 waves stream faster than 768 workgroups
// of 16-channel tiles whose wave accesses are split over four 64-byte rows.
#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

#ifndef SSM_SM1_WAVES
#define SSM_SM1_WAVES 16                     // waves per workgroup = sub-chunks per round
#endif
#ifndef SSM_SM1_STEPS
#define SSM_SM1_STEPS 8                      // steps per sub-chunk
#endif

constexpr int kWaves = SSM_SM1_WAVES;
constexpr int kThreads = kWaves * 64;
constexpr int kTileC = 64;                   // channels per workgroup (lane = channel)
constexpr int kSub = kWaves;                 // sub-chunks per round (one per wave)
constexpr int kL = SSM_SM1_STEPS;
constexpr int kRound = kSub * kL;            // steps per round
static_assert(2 * kRound <= kThreads, "one B or C value per thread");

struct Sm1Params {
    const void *x, *delta, *z, *B, *C;
    void *y;
    const float *A, *D, *bias, *h0;
    float *last;
    int64_t seqlen;
    int dim, n_ct;
};

template <typename T, bool SP, bool GATE>
__global__ __launch_bounds__(kThreads) void sm1_scan_kernel(Sm1Params p) {
    using M = typename MathFor<T>::type;
    using R = typename Io<T>::raw;
    constexpr uint32_t es = sizeof(T);
    __shared__ float2 sPH[2][kSub][kTileC];          // sub-chunk aggregates
    __shared__ float4 sBC[3][2][kRound / 4];          // B, C of a round, widened

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    const int c = tid % 64;                          // channel within the tile
    const int s = w;                                 // sub-chunk of this wave
    const int b = static_cast<int>(blockIdx.x) / p.n_ct;
    const int ct = static_cast<int>(blockIdx.x) - b * p.n_ct;
    const int ch = ct * kTileC + c;
    const bool cvalid = ch < p.dim;
    const int chc = cvalid ? ch : p.dim - 1;

    const float Ac = M::prep_A(p.A[chc]);
    const float bias = p.bias ? p.bias[chc] : 0.0f;
    const float Dc = p.D ? p.D[chc] : 0.0f;
    const int64_t bd = static_cast<int64_t>(b) * p.dim;
    float h_in = p.h0 ? p.h0[bd + chc] : 0.0f;

    // Addressing inside a round: row (s*kL + i), column ch, as a vector offset
    // from a descriptor that starts at the round's first row and ends at its
    // last valid one.  The buffer unit checks the vector offset against that
    // range, so steps past the sequence read 0 and store nothing, and lanes
    // past d_inner, whose offsets start at 2 GiB, do the same.  The kL offsets
    // are computed once and kept in registers; every round, full or partial,
    // uses the same instructions.
    const uint32_t row_bytes = static_cast<uint32_t>(p.dim) * es;
    const uint32_t voff = cvalid ? static_cast<uint32_t>(s * kL) * row_bytes + static_cast<uint32_t>(ch) * es
                                 : kOffNone;
    uint32_t vo[kL];
#pragma unroll
    for (int i = 0; i < kL; ++i) {
        vo[i] = voff + static_cast<uint32_t>(i) * row_bytes;
        asm volatile("" : "+v"(vo[i]));              // keep, do not recompute per access
    }
    const char *xb = static_cast<const char *>(p.x);
    const char *db = static_cast<const char *>(p.delta);
    const char *zb = static_cast<const char *>(GATE ? p.z : p.x);
    char *yb = static_cast<char *>(p.y);
    const char *Bb = static_cast<const char *>(p.B);
    const char *Cb = static_cast<const char *>(p.C);
    const int n_rounds = static_cast<int>((p.seqlen + kRound - 1) / kRound);

    // steps of round r; 0 past the last round, whose loads then go through an
    // empty descriptor and return zeros without touching memory
    auto steps_in = [&](int r) {
        const int64_t rem = p.seqlen - static_cast<int64_t>(r) * kRound;
        return static_cast<int>(rem < kRound ? (rem > 0 ? rem : 0) : kRound);
    };
    auto row_of = [&](int r) { return static_cast<int64_t>(b) * p.seqlen + static_cast<int64_t>(r) * kRound; };
    auto io_rsrc = [&](const char *base, int r) {
        return make_rsrc(base + row_of(r) * static_cast<int64_t>(row_bytes),
                         static_cast<uint32_t>(steps_in(r)) * row_bytes);
    };
    // load kL steps of one tensor for round r
    auto load_steps = [&](R (&dst)[kL], const char *base, int r) {
        const rsrc_t rs = io_rsrc(base, r);
#pragma unroll
        for (int i = 0; i < kL; ++i) dst[i] = Io<T>::template load<kStream>(rs, vo[i], 0);
    };
    // B and C of a round: the first kRound threads fetch step tid of B, the
    // next kRound step tid - kRound of C.  The choice is taken from the wave
    // index so that the descriptor stays in scalar registers.
    static_assert(kRound % 64 == 0, "B/C loads split at a wave boundary");
    const bool bc_c = w >= kRound / 64;
    const int bc_k = bc_c ? tid - kRound : tid;
    auto load_bc = [&](R &v, int r) {
        const uint32_t n = static_cast<uint32_t>(steps_in(r)) * es;
        const int64_t e0 = row_of(r) * es;
        v = Io<T>::load(make_rsrc((bc_c ? Cb : Bb) + e0, n), static_cast<uint32_t>(bc_k) * es, 0);
    };
    auto stash_bc = [&](R v, int r) {
        if (w < 2 * kRound / 64) reinterpret_cast<float *>(sBC[r % 3][bc_c ? 1 : 0])[bc_k] = Io<T>::f32(v);
    };

    struct Raw { R d[kL], x[kL], z[kL]; };
    R bcnext;
    auto round = [&](Raw &cur, Raw &next, int r) {
        const int left = steps_in(r);
        // the next round's delta, x and gate input and the B, C two rounds
        // ahead go in flight while this round computes.  They are issued on
        // every round, past the end through empty descriptors, so that the
        // number of accesses in flight is the same on every path through the
        // loop and the compiler's wait counts stay exact.
        load_steps(next.d, db, r + 1);
        load_steps(next.x, xb, r + 1);
        if constexpr (GATE) load_steps(next.z, zb, r + 1);
        if (r + 1 < n_rounds) stash_bc(bcnext, r + 1);
        load_bc(bcnext, r + 2);
        // ---- pass 1: discretise, keep (f, u), fold into the aggregate
        float f[kL], u[kL];
        float S = 0.0f, H = 0.0f;
#pragma unroll
        for (int j = 0; j < kL / 4; ++j) {
            const float4 b4 = sBC[r % 3][0][s * (kL / 4) + j];
            const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = 4 * j + k;
                const float v = Io<T>::f32(cur.d[i]) + bias;
                float dt = SP ? M::softplus(v) : v;
                dt = s * kL + i < left ? dt : 0.0f;  // past the end: identity step
                S += dt;
                f[i] = M::factor(dt * Ac);
                u[i] = dt * bv[k] * Io<T>::f32(cur.x[i]);
                H = M::apply(f[i], H, u[i]);
            }
        }
        sPH[r & 1][s][c] = make_float2(M::factor(S * Ac), H);
        __syncthreads();

        // ---- carry: compose the sub-chunk aggregates of this channel in
        // order (s is the wave index, so the prefix split is uniform).  The
        // round's partial sums are built apart from the carried state and
        // meet it once, so the long-lived state takes two roundings per round
        // instead of two per sub-chunk.
        float Pp = M::kIdentity, Hp = 0.0f, Ps = M::kIdentity, Hs = 0.0f;
#pragma unroll
        for (int k = 0; k < kSub; ++k) {
            if (k == s) { Ps = Pp; Hs = Hp; }        // aggregate of sub-chunks 0 .. s-1
            const float2 ph = sPH[r & 1][k][c];
            Hp = M::apply(ph.x, Hp, ph.y);
            Pp = M::compose(Pp, ph.x);
        }
        const float hs = M::apply(Ps, h_in, Hs);     // state entering this sub-chunk
        h_in = M::apply(Pp, h_in, Hp);               // state leaving the round

        // ---- pass 2: replay from the incoming state, write y
        const rsrc_t ry = make_rsrc(yb + row_of(r) * static_cast<int64_t>(row_bytes),
                                    static_cast<uint32_t>(left) * row_bytes);
        float h = hs;
#pragma unroll
        for (int j = 0; j < kL / 4; ++j) {
            const float4 c4 = sBC[r % 3][1][s * (kL / 4) + j];
            const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = 4 * j + k;
                h = M::apply(f[i], h, u[i]);
                float o = fmaf(cv[k], h, Dc * Io<T>::f32(cur.x[i]));
                if constexpr (GATE) o *= silu(Io<T>::f32(cur.z[i]));
                Io<T>::template store<kStream>(o, ry, vo[i], 0);
            }
        }
    };

    // prologue: round 0's delta, x and z, B/C of round 0 in LDS, B/C of round 1
    Raw ra, rb;
    load_steps(ra.d, db, 0);
    load_steps(ra.x, xb, 0);
    if constexpr (GATE) load_steps(ra.z, zb, 0);
    {
        R bc0;
        load_bc(bc0, 0);
        stash_bc(bc0, 0);
    }
    load_bc(bcnext, 1);
    // Drain the prologue's loads: the loop then starts with nothing in
    // flight, as after a steady-state round, so the compiler's wait counts
    // inside the loop stay those of the steady state.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // rounds alternate between the two register sets (no copies)
    for (int r = 0; r < n_rounds; r += 2) {
        round(ra, rb, r);
        if (r + 1 < n_rounds) round(rb, ra, r + 1);
    }
    if (p.last && w == 0 && cvalid) p.last[bd + ch] = h_in;
}

// The kernel's 32-bit round offsets need kRound rows of d_inner to span
// less than 2 GiB (inactive lanes start at 2 GiB and must not wrap); the
// tile count must fit an int.
bool tiled_ok(int64_t batch, int64_t seqlen, int64_t dim, int bf16) {
    const int64_t es = bf16 ? 2 : 4;
    const int64_t n_ct = (dim + kTileC - 1) / kTileC;
    return seqlen > 0 && dim * es * kRound < (int64_t(1) << 31) && batch * n_ct < (int64_t(1) << 31);
}

template <typename T, bool SP, bool GATE> hipError_t launch_t(const ScanArgs &a, hipStream_t s) {
    Sm1Params p{};
    p.x = a.x; p.delta = a.delta; p.z = a.z; p.B = a.B; p.C = a.C; p.y = a.y;
    p.A = a.A; p.D = a.D; p.bias = a.delta_bias; p.h0 = a.h0; p.last = a.last_state;
    p.seqlen = a.seqlen;
    p.dim = static_cast<int>(a.dim);
    p.n_ct = static_cast<int>((a.dim + kTileC - 1) / kTileC);
    const unsigned grid = static_cast<unsigned>(a.batch * p.n_ct);
    hipLaunchKernelGGL((sm1_scan_kernel<T, SP, GATE>), dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename T> hipError_t launch_flags(const ScanArgs &a, hipStream_t s) {
    const bool sp = a.softplus != 0, gate = a.z != nullptr;
    if (sp && gate) return launch_t<T, true, true>(a, s);
    if (sp) return launch_t<T, true, false>(a, s);
    if (gate) return launch_t<T, false, true>(a, s);
    return launch_t<T, false, false>(a, s);
}

}  // namespace

size_t sm1_workspace(int64_t batch, int64_t seqlen, int64_t dim, int bf16) {
    if (tiled_ok(batch, seqlen, dim, bf16)) return 0;
    ScanArgs g{};
    g.batch = batch; g.seqlen = seqlen; g.dim = dim; g.dstate = 1; g.bf16 = bf16;
    return scan_fwd_workspace(g);                     // the general kernel's needs
}

hipError_t launch_sm1_scan(const ScanArgs &a, hipStream_t s) {
    if (a.batch == 0 || a.dim == 0) return hipSuccess;
    ScanArgs g = a;
    g.dstate = 1;
    if (!tiled_ok(a.batch, a.seqlen, a.dim, a.bf16)) return launch_scan_fwd(g, s);   // T = 0, huge d_inner
    if (a.bf16) return launch_flags<bf16_t>(g, s);
    return launch_flags<float>(g, s);
}

}  // namespace ssm
