// d_state = 1 forward scan ("SM1", the scalar-state Mamba-1 scan of the
// "Windows SM1 (Scalar Mamba1)" page: h_t = dA_t h_{t-1} + dBx_t, y = h C,
// whose closed form is a cumulative product and a cumulative sum).
//
// With one state per channel there are only batch * d_inner independent
// chains (12288 at the 130M shape), far too few to keep HBM busy by walking
// each chain through time, so time is split.  The recurrence composes as the
// affine map h -> P h + H, and maps compose associatively:
//     (P1, H1) then (P2, H2)  =  (P2 P1, P2 H1 + H2),  identity (1, 0)
// (the (decay, offset) operator behind the parallel scan of the youngju.dev
// guide, section 5 "Hardware-Aware Algorithm").
//
// Work split (one workgroup = 64 channels x 128 steps of one batch row):
//   * lane = (channel group g of 4 channels, sub-chunk s of 8 steps); each
//     lane loads its 4 channels with one 128-bit (fp32) / 64-bit (bf16) load
//     per step, discretises, and scans its 8 steps sequentially, keeping the
//     decay factors and inputs in registers;
//   * the 4 sub-chunks of a wave (the 4 lanes of a quad) are scanned with two
//     DPP quad permutations; wave totals go through LDS to later waves;
//   * the carry between workgroups is chained: each workgroup publishes its
//     aggregate, then looks back over its predecessors' published aggregates /
//     inclusive prefixes (decoupled look-back) and publishes its own prefix.
//     Chunk order comes from an atomic ticket, so a workgroup only ever waits
//     on workgroups that are already running;
//   * a second pass over the registers applies the incoming state and writes
//     y = (C h + D x) SiLU(z) with the same wide stores.
// Every input byte is read once and every output byte written once.
#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kCPL = 4;                      // channels per lane
constexpr int kGroups = 16;                  // channel groups per workgroup
constexpr int kTileC = kGroups * kCPL;       // 64 channels
constexpr int kSubPerWave = 4;               // quad position = sub-chunk within the wave
constexpr int kSub = kWaves * kSubPerWave;   // 16 sub-chunks
constexpr int kL = 8;                        // steps per sub-chunk
constexpr int kChunkT = kSub * kL;           // 128 steps per workgroup
constexpr uint32_t kSpinLimit = 1u << 22;    // bounded wait on a predecessor

// DPP quad_perm controls: take the value of quad lane (q-1) / (q-2)
constexpr int kQuadShr1 = 0x90;   // [0,0,1,2]
constexpr int kQuadShr2 = 0x44;   // [0,1,0,1]

enum : uint32_t { kFlagEmpty = 0, kFlagAggregate = 1, kFlagPrefix = 2 };

struct Layout {
    int n_ct, n_tiles, n_chunks;
    size_t flags_off, agg_off, pre_off, total;
};

Layout make_layout(int64_t batch, int64_t seqlen, int64_t dim) {
    Layout l{};
    l.n_ct = static_cast<int>((dim + kTileC - 1) / kTileC);
    l.n_tiles = static_cast<int>(batch * l.n_ct);
    l.n_chunks = static_cast<int>((seqlen + kChunkT - 1) / kChunkT);
    const size_t nflags = static_cast<size_t>(l.n_tiles) * l.n_chunks;
    auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
    l.flags_off = 256;                                   // [0]: ticket counter
    l.agg_off = l.flags_off + up(nflags * sizeof(uint32_t));
    l.pre_off = l.agg_off + up(nflags * kTileC * sizeof(float2));
    l.total = l.pre_off + up(nflags * kTileC * sizeof(float));
    return l;
}

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <typename T> __device__ __forceinline__ void load4(const T *p, float (&v)[4]);
template <> __device__ __forceinline__ void load4<float>(const float *p, float (&v)[4]) {
    const float4 q = *reinterpret_cast<const float4 *>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
template <> __device__ __forceinline__ void load4<bf16_t>(const bf16_t *p, float (&v)[4]) {
    const uint2 q = *reinterpret_cast<const uint2 *>(p);
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
}
template <typename T> __device__ __forceinline__ void store4(T *p, const float (&v)[4]);
template <> __device__ __forceinline__ void store4<float>(float *p, const float (&v)[4]) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t *p, const float (&v)[4]) {
    uint2 q;
    q.x = static_cast<uint32_t>(from_f32<bf16_t>(v[0]).bits) | (static_cast<uint32_t>(from_f32<bf16_t>(v[1]).bits) << 16);
    q.y = static_cast<uint32_t>(from_f32<bf16_t>(v[2]).bits) | (static_cast<uint32_t>(from_f32<bf16_t>(v[3]).bits) << 16);
    *reinterpret_cast<uint2 *>(p) = q;
}

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *w, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) w[i] = 0u;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void sm1_chunked_kernel(
    const T *__restrict__ x, const T *__restrict__ delta, const T *__restrict__ z,
    const T *__restrict__ Bv, const T *__restrict__ Cv, const float *__restrict__ A,
    const float *__restrict__ Dv, const float *__restrict__ bias, const float *__restrict__ h0,
    T *__restrict__ y, float *__restrict__ last, uint32_t *__restrict__ ws_words,
    float2 *__restrict__ agg, float *__restrict__ pre, int64_t seqlen, int64_t dim,
    int n_ct, int n_tiles, int n_chunks, int softplus_flag) {
    using M = typename MathFor<T>::type;
    __shared__ uint32_t s_ticket;
    __shared__ float2 s_wave[kWaves][kTileC];   // wave totals per channel
    __shared__ float s_hin[kTileC];             // state entering this chunk

    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    if (tid == 0) s_ticket = atomicAdd(&ws_words[0], 1u);
    __syncthreads();
    const uint32_t ticket = s_ticket;
    const int chunk = static_cast<int>(ticket / static_cast<uint32_t>(n_tiles));
    const int tile = static_cast<int>(ticket % static_cast<uint32_t>(n_tiles));
    const int64_t b = tile / n_ct;
    const int ct = tile % n_ct;
    uint32_t *flags = ws_words + 64;            // flags start 256 bytes in
    const int64_t slot = static_cast<int64_t>(tile) * n_chunks + chunk;

    const int g = lane / kSubPerWave, sq = lane % kSubPerWave;
    const int s = wave * kSubPerWave + sq;
    const int64_t c_raw = static_cast<int64_t>(ct) * kTileC + g * kCPL;
    const bool cvalid = c_raw < dim;             // dim % 4 == 0: all 4 or none
    const int64_t c0 = cvalid ? c_raw : dim - kCPL;
    const int64_t t_first = static_cast<int64_t>(chunk) * kChunkT + s * kL;
    const bool softplus_on = softplus_flag != 0;

    float Ac[kCPL], bc[kCPL], Dc[kCPL];
#pragma unroll
    for (int k = 0; k < kCPL; ++k) {
        Ac[k] = M::prep_A(A[c0 + k]);
        bc[k] = bias ? bias[c0 + k] : 0.0f;
        Dc[k] = Dv ? Dv[c0 + k] : 0.0f;
    }

    // ---- pass 1: loads, discretisation, local scan of this lane's 8 steps
    float xs[kL][kCPL], ds[kL][kCPL], zs[kL][kCPL], Ct[kL], Bt[kL];
#pragma unroll
    for (int i = 0; i < kL; ++i) {
        const int64_t t = t_first + i;
        const int64_t tt = t < seqlen ? t : seqlen - 1;
        const int64_t row = (b * seqlen + tt) * dim + c0;
        load4<T>(x + row, xs[i]);
        load4<T>(delta + row, ds[i]);
        if (z) load4<T>(z + row, zs[i]);
        Bt[i] = to_f32(Bv[b * seqlen + tt]);
        Ct[i] = to_f32(Cv[b * seqlen + tt]);
    }
    float f[kL][kCPL], u[kL][kCPL];
    float P[kCPL], H[kCPL], S[kCPL];
#pragma unroll
    for (int k = 0; k < kCPL; ++k) { H[k] = 0.0f; S[k] = 0.0f; }
#pragma unroll
    for (int i = 0; i < kL; ++i) {
        const bool tv = t_first + i < seqlen;
#pragma unroll
        for (int k = 0; k < kCPL; ++k) {
            const float v = ds[i][k] + bc[k];
            float dt = softplus_on ? M::softplus(v) : v;
            dt = tv ? dt : 0.0f;                     // past the end: identity step
            S[k] += dt;
            f[i][k] = M::factor(dt * Ac[k]);
            u[i][k] = dt * Bt[i] * xs[i][k];
            H[k] = M::apply(f[i][k], H[k], u[i][k]);
            xs[i][k] *= Dc[k];                       // keep D x for the epilogue
        }
    }
#pragma unroll
    for (int k = 0; k < kCPL; ++k) P[k] = M::decay(S[k] * Ac[k]);   // product of the 8 decays

    // ---- scan over the 4 sub-chunks of the wave (quad lanes), inclusive
#pragma unroll
    for (int k = 0; k < kCPL; ++k) {
        float Pp = dpp<kQuadShr1>(P[k]), Hp = dpp<kQuadShr1>(H[k]);
        if (sq >= 1) { H[k] = fmaf(P[k], Hp, H[k]); P[k] *= Pp; }
        Pp = dpp<kQuadShr2>(P[k]); Hp = dpp<kQuadShr2>(H[k]);
        if (sq >= 2) { H[k] = fmaf(P[k], Hp, H[k]); P[k] *= Pp; }
    }
    // exclusive prefix inside the wave
    float Pe[kCPL], He[kCPL];
#pragma unroll
    for (int k = 0; k < kCPL; ++k) {
        Pe[k] = dpp<kQuadShr1>(P[k]);
        He[k] = dpp<kQuadShr1>(H[k]);
        if (sq == 0) { Pe[k] = 1.0f; He[k] = 0.0f; }
    }
    if (sq == kSubPerWave - 1) {
#pragma unroll
        for (int k = 0; k < kCPL; ++k) s_wave[wave][g * kCPL + k] = make_float2(P[k], H[k]);
    }
    __syncthreads();

    // ---- carry across waves, then the chained carry across workgroups
    if (wave == 0) {
        const int ch = lane;
        float Pt = 1.0f, Ht = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float2 a = s_wave[w][ch];
            Ht = fmaf(a.x, Ht, a.y);
            Pt *= a.x;
        }
        const int64_t chg = static_cast<int64_t>(ct) * kTileC + ch;
        float h_in;
        if (chunk == 0) {
            h_in = (h0 && chg < dim) ? h0[b * dim + chg] : 0.0f;
        } else {
            agg[slot * kTileC + ch] = make_float2(Pt, Ht);
            __hip_atomic_store(&flags[slot], kFlagAggregate, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            float Pa = 1.0f, Ha = 0.0f;
            int k = chunk - 1;
            uint32_t spins = 0;
            h_in = 0.0f;
            while (true) {
                const int64_t ks = static_cast<int64_t>(tile) * n_chunks + k;
                // relaxed coherent poll; one acquire fence once a flag is seen
                const uint32_t fl = __hip_atomic_load(&flags[ks], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (fl != kFlagEmpty) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                if (fl == kFlagPrefix) {
                    h_in = fmaf(Pa, pre[ks * kTileC + ch], Ha);
                    break;
                }
                if (fl == kFlagAggregate) {
                    const float2 a = agg[ks * kTileC + ch];
                    Ha = fmaf(Pa, a.y, Ha);
                    Pa *= a.x;
                    --k;
                    spins = 0;
                    if (k < 0) break;                 // unreachable: chunk 0 publishes a prefix
                    continue;
                }
                if (++spins > kSpinLimit) {           // never wait unboundedly
                    ws_words[1] = 1u;                 // error word for the host
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        const float h_out = fmaf(Pt, h_in, Ht);
        pre[slot * kTileC + ch] = h_out;
        __hip_atomic_store(&flags[slot], kFlagPrefix, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        s_hin[ch] = h_in;
        if (last && chunk == n_chunks - 1 && chg < dim) last[b * dim + chg] = h_out;
    }
    __syncthreads();

    // ---- pass 2: apply the incoming state and write y
    float Pw = 1.0f, Hw = 0.0f;
    float h[kCPL];
#pragma unroll
    for (int k = 0; k < kCPL; ++k) {
        Pw = 1.0f; Hw = 0.0f;
        for (int w = 0; w < wave; ++w) {             // waves before this one
            const float2 a = s_wave[w][g * kCPL + k];
            Hw = fmaf(a.x, Hw, a.y);
            Pw *= a.x;
        }
        // state entering this lane's sub-chunk
        h[k] = fmaf(Pe[k], fmaf(Pw, s_hin[g * kCPL + k], Hw), He[k]);
    }
#pragma unroll
    for (int i = 0; i < kL; ++i) {
        const int64_t t = t_first + i;
        float out[kCPL];
#pragma unroll
        for (int k = 0; k < kCPL; ++k) {
            h[k] = M::apply(f[i][k], h[k], u[i][k]);
            float o = fmaf(Ct[i], h[k], xs[i][k]);
            if (z) o *= silu(zs[i][k]);
            out[k] = o;
        }
        if (cvalid && t < seqlen) store4<T>(y + (b * seqlen + t) * dim + c0, out);
    }
}

template <typename T> hipError_t launch_chunked(const ScanArgs &a, hipStream_t s) {
    const Layout l = make_layout(a.batch, a.seqlen, a.dim);
    char *ws = static_cast<char *>(a.workspace);
    uint32_t *words = reinterpret_cast<uint32_t *>(ws);
    const int64_t nclear = static_cast<int64_t>(l.agg_off / sizeof(uint32_t));   // counter + flags
    hipLaunchKernelGGL(clear_words_kernel, dim3(static_cast<unsigned>((nclear + 255) / 256)), dim3(256), 0, s,
                       words, nclear);
    const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(l.n_tiles) * l.n_chunks);
    hipLaunchKernelGGL((sm1_chunked_kernel<T>), dim3(grid), dim3(kThreads), 0, s,
                       static_cast<const T *>(a.x), static_cast<const T *>(a.delta),
                       static_cast<const T *>(a.z), static_cast<const T *>(a.B),
                       static_cast<const T *>(a.C), a.A, a.D, a.delta_bias, a.h0,
                       static_cast<T *>(a.y), a.last_state, words,
                       reinterpret_cast<float2 *>(ws + l.agg_off), reinterpret_cast<float *>(ws + l.pre_off),
                       a.seqlen, a.dim, l.n_ct, l.n_tiles, l.n_chunks, a.softplus);
    return hipGetLastError();
}

bool aligned_to(const void *p, size_t n) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % n == 0; }

// The chunked kernel needs 4-channel vector access: d_inner % 4 == 0 and the
// (batch, seqlen, d_inner) tensors aligned to 4 elements.
bool chunked_ok(const ScanArgs &a) {
    const size_t vec = a.bf16 ? 8 : 16;
    return a.seqlen > 0 && a.dim % kCPL == 0 && aligned_to(a.x, vec) && aligned_to(a.delta, vec) &&
           aligned_to(a.z, vec) && aligned_to(a.y, vec) &&
           static_cast<int64_t>(make_layout(a.batch, a.seqlen, a.dim).n_tiles) *
                   make_layout(a.batch, a.seqlen, a.dim).n_chunks < (int64_t(1) << 31);
}

}  // namespace

size_t sm1_workspace(int64_t batch, int64_t seqlen, int64_t dim, int bf16) {
    ScanArgs g{};
    g.batch = batch; g.seqlen = seqlen; g.dim = dim; g.dstate = 1; g.bf16 = bf16;
    const size_t general = scan_fwd_workspace(g);                 // fallback path
    const size_t chunked = seqlen > 0 ? make_layout(batch, seqlen, dim).total : 0;
    return general > chunked ? general : chunked;
}

hipError_t launch_sm1_scan(const ScanArgs &a, hipStream_t s) {
    if (a.batch == 0 || a.dim == 0) return hipSuccess;
    ScanArgs g = a;
    g.dstate = 1;
    if (!chunked_ok(g)) return launch_scan_fwd(g, s);   // T = 0, ragged d_inner, unaligned views
    if (a.workspace == nullptr || a.workspace_bytes < make_layout(a.batch, a.seqlen, a.dim).total)
        return hipErrorInvalidValue;
    if (a.bf16) return launch_chunked<bf16_t>(g, s);
    return launch_chunked<float>(g, s);
}

}  // namespace ssm
