// One recurrent decode step of the selective scan on gfx950: the recurrence
// of the youngju.dev guide (section 2 discrete recurrence, section 5
// selective_scan) taken for a single token, with the constant-size state
// read and written in place (the O(1)-per-token inference of the
// "Windows SM1 (Scalar Mamba1)" page).
//
// The step streams the (batch, d_inner, d_state) fp32 state once in and once
// out; everything else is small, so the kernel is HBM-bound.  Each chain
// (b, d) is served by one quad of lanes: lane q of the quad owns states
// [q*NPL, q*NPL + NPL), so for d_state = 16 a quad reads and writes one
// contiguous 64-byte state row with 16-byte non-temporal accesses and a wave
// moves 1 KiB of contiguous state per access; at d_state 16 a thread serves
// the same channel of two batch rows, which halves the A-row reads and keeps
// two state loads in flight.  The readout sum over n is reduced inside the
// quad with two DPP row-quad permutations.
#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

constexpr int kThreads = 256;
constexpr int kQuad = 4;

// quad_perm DPP controls: lanes exchange with lane^1 and lane^2 of their quad
constexpr int kQuadXor1 = 0xB1;   // [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // [2,3,0,1]

__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kQuadXor1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kQuadXor2, 0xF, 0xF, true));
    return v;
}

// 4 consecutive B or C values of one batch row, widened
__device__ __forceinline__ void load4_io(const float *p, float (&v)[4]) {
    const float4 q = *reinterpret_cast<const float4 *>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void load4_io(const bf16_t *p, float (&v)[4]) {
    const uint2 q = *reinterpret_cast<const uint2 *>(p);
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
}

// Any d_state: one workgroup = 64 chains (channels cb*64 .. cb*64+63) of one
// batch row; block index = b * n_cblk + cb.
template <int N, typename T>
__global__ __launch_bounds__(kThreads) void state_update_kernel(StepArgs a, int n_cblk) {
    using M = typename MathFor<T>::type;
    constexpr int NPL = (N + kQuad - 1) / kQuad;   // states per lane
    const int b = static_cast<int>(blockIdx.x) / n_cblk;
    const int cb = static_cast<int>(blockIdx.x) - b * n_cblk;
    const int tid = threadIdx.x, q = tid % kQuad;
    const int d_raw = cb * (kThreads / kQuad) + tid / kQuad;
    const bool active = d_raw < a.dim;
    const int d = active ? d_raw : static_cast<int>(a.dim) - 1;   // keep the quad's DPP partners valid
    const int64_t c = static_cast<int64_t>(b) * a.dim + d;          // chain (b, d)

    const T *x = static_cast<const T *>(a.x);
    const T *dl = static_cast<const T *>(a.delta);
    const T *Bm = static_cast<const T *>(a.B) + static_cast<int64_t>(b) * N;
    const T *Cm = static_cast<const T *>(a.C) + static_cast<int64_t>(b) * N;
    float *st = a.state + c * N;
    const float *Ad = a.A + static_cast<int64_t>(d) * N;

    float hs[NPL], Av[NPL], Bv[NPL], Cv[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int n = q * NPL + i;
        const int nn = n < N ? n : N - 1;
        hs[i] = st[nn];
        Av[i] = Ad[nn];
        Bv[i] = to_f32(Bm[nn]);
        Cv[i] = to_f32(Cm[nn]);
    }
    const float xv = to_f32(x[c]);
    const float v = to_f32(dl[c]) + (a.delta_bias ? a.delta_bias[d] : 0.0f);
    const float dt = a.softplus ? M::softplus(v) : v;
    const float dtx = dt * xv;

    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int n = q * NPL + i;
        if (n < N) {
            hs[i] = M::step(dt * M::prep_A(Av[i]), hs[i], dtx * Bv[i]);
            part = fmaf(Cv[i], hs[i], part);
        }
    }
    if (active) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const int n = q * NPL + i;
            if (n < N) st[n] = hs[i];
        }
    }
    const float acc = quad_sum(part);
    if (q == 0 && active) {
        float out = acc + (a.D ? a.D[d] * xv : 0.0f);
        if (a.z) out *= silu(to_f32(static_cast<const T *>(a.z)[c]));
        static_cast<T *>(a.y)[c] = from_f32<T>(out);
    }
}

// d_state 16, 16-byte aligned state and A rows: a thread serves one lane
// quarter of KB chains that share a channel (batch rows bg*KB .. bg*KB+KB-1),
// so the channel's A row, bias and D are loaded once for KB chains and KB
// state loads are in flight per thread.  Block index = bg * n_cblk + cb.
#ifndef SSM_DECODE_ROWS
#define SSM_DECODE_ROWS 2
#endif
template <typename T, int KB>
__global__ __launch_bounds__(kThreads) void state_update_rows_kernel(StepArgs a, int n_cblk) {
    using M = typename MathFor<T>::type;
    typedef float f4v __attribute__((ext_vector_type(4)));
    constexpr int N = 16;
    const int bg = static_cast<int>(blockIdx.x) / n_cblk;
    const int cb = static_cast<int>(blockIdx.x) - bg * n_cblk;
    const int tid = threadIdx.x, q = tid % kQuad;
    const int d_raw = cb * (kThreads / kQuad) + tid / kQuad;
    const bool active = d_raw < a.dim;
    const int d = active ? d_raw : static_cast<int>(a.dim) - 1;   // keep the quad's DPP partners valid
    const int b0 = bg * KB;
    const int nb = static_cast<int>(a.batch - b0 < KB ? a.batch - b0 : KB);   // rows of this group (uniform)

    const float4 a4 = *reinterpret_cast<const float4 *>(a.A + static_cast<int64_t>(d) * N + q * 4);
    const float A2[4] = {M::prep_A(a4.x), M::prep_A(a4.y), M::prep_A(a4.z), M::prep_A(a4.w)};
    const float bias = a.delta_bias ? a.delta_bias[d] : 0.0f;
    const float Dd = a.D ? a.D[d] : 0.0f;
    const T *x = static_cast<const T *>(a.x);
    const T *dl = static_cast<const T *>(a.delta);
    const T *zp = static_cast<const T *>(a.z);

    // every load of the group first, then the arithmetic
    f4v hs[KB];
    float Bv[KB][4], Cv[KB][4], xv[KB], dv[KB], zv[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int b = b0 + (k < nb ? k : 0);
        const int64_t c = static_cast<int64_t>(b) * a.dim + d;
        hs[k] = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(a.state + c * N + q * 4));
        load4_io(static_cast<const T *>(a.B) + static_cast<int64_t>(b) * N + q * 4, Bv[k]);
        load4_io(static_cast<const T *>(a.C) + static_cast<int64_t>(b) * N + q * 4, Cv[k]);
        xv[k] = to_f32(x[c]);
        dv[k] = to_f32(dl[c]);
        zv[k] = zp ? to_f32(zp[c]) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        if (k >= nb) break;                                // uniform
        const int64_t c = static_cast<int64_t>(b0 + k) * a.dim + d;
        const float v = dv[k] + bias;
        const float dt = a.softplus ? M::softplus(v) : v;
        const float dtx = dt * xv[k];
        float part = 0.0f;
        f4v h = hs[k];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = M::step(dt * A2[i], h[i], dtx * Bv[k][i]);
            part = fmaf(Cv[k][i], h[i], part);
        }
        if (active) __builtin_nontemporal_store(h, reinterpret_cast<f4v *>(a.state + c * N + q * 4));
        const float acc = quad_sum(part);
        if (q == 0 && active) {
            float out = fmaf(Dd, xv[k], acc);
            if (zp) out *= silu(zv[k]);
            static_cast<T *>(a.y)[c] = from_f32<T>(out);
        }
    }
}

bool aligned_to(const void *p, size_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

template <int N, typename T> hipError_t launch(const StepArgs &a, hipStream_t s) {
    const int n_cblk = static_cast<int>((a.dim + kThreads / kQuad - 1) / (kThreads / kQuad));
    const dim3 grid(static_cast<unsigned>(a.batch * n_cblk));
    if constexpr (N == 16) {
        const size_t bc = sizeof(T) * 4;
        if (aligned_to(a.state, 16) && aligned_to(a.A, 16) && aligned_to(a.B, bc) && aligned_to(a.C, bc)) {
            constexpr int KB = SSM_DECODE_ROWS;
            const dim3 g2(static_cast<unsigned>((a.batch + KB - 1) / KB * n_cblk));
            hipLaunchKernelGGL((state_update_rows_kernel<T, KB>), g2, dim3(kThreads), 0, s, a, n_cblk);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((state_update_kernel<N, T>), grid, dim3(kThreads), 0, s, a, n_cblk);
    return hipGetLastError();
}

template <typename T> hipError_t dispatch_n(const StepArgs &a, hipStream_t s) {
    switch (a.dstate) {
#define SSM_CASE(NN) \
    case NN: return launch<NN, T>(a, s);
        SSM_CASE(1) SSM_CASE(2) SSM_CASE(3) SSM_CASE(4) SSM_CASE(5) SSM_CASE(6) SSM_CASE(7)
        SSM_CASE(8) SSM_CASE(9) SSM_CASE(10) SSM_CASE(11) SSM_CASE(12) SSM_CASE(13)
        SSM_CASE(14) SSM_CASE(15) SSM_CASE(16)
#undef SSM_CASE
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_state_update(const StepArgs &a, hipStream_t s) {
    if (a.batch == 0 || a.dim == 0) return hipSuccess;
    if (a.bf16) return dispatch_n<bf16_t>(a, s);
    return dispatch_n<float>(a, s);
}

}  // namespace ssm
