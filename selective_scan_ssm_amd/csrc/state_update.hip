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
// contiguous 64-byte state row with 16-byte accesses and a wave moves 1 KiB
// of contiguous state per access.  The readout sum over n is reduced inside
// the quad with two DPP row-quad permutations.
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

template <int N, typename T>
__global__ __launch_bounds__(kThreads) void state_update_kernel(StepArgs a) {
    using M = typename MathFor<T>::type;
    constexpr int NPL = (N + kQuad - 1) / kQuad;   // states per lane
    const int64_t chains = a.batch * a.dim;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t c_raw = gid / kQuad;
    const int q = static_cast<int>(gid % kQuad);
    const bool active = c_raw < chains;
    const int64_t c = active ? c_raw : chains - 1;   // keep the quad's DPP partners valid
    const int64_t b = c / a.dim, d = c % a.dim;

    const T *x = static_cast<const T *>(a.x);
    const T *dl = static_cast<const T *>(a.delta);
    const T *Bm = static_cast<const T *>(a.B);
    const T *Cm = static_cast<const T *>(a.C);

    const float xv = to_f32(x[c]);
    const float v = to_f32(dl[c]) + (a.delta_bias ? a.delta_bias[d] : 0.0f);
    const float dt = a.softplus ? M::softplus(v) : v;
    const float dtx = dt * xv;

    float part = 0.0f;
    float hs[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int n = q * NPL + i;
        if (n < N) hs[i] = a.state[c * N + n];
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int n = q * NPL + i;
        if (n < N) {
            const float hn = M::step(dt * M::prep_A(a.A[d * N + n]), hs[i], dtx * to_f32(Bm[b * N + n]));
            hs[i] = hn;
            part = fmaf(to_f32(Cm[b * N + n]), hn, part);
        }
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int n = q * NPL + i;
        if (n < N && active) a.state[c * N + n] = hs[i];
    }
    const float acc = quad_sum(part);
    if (q == 0 && active) {
        float out = acc + (a.D ? a.D[d] * xv : 0.0f);
        if (a.z) out *= silu(to_f32(static_cast<const T *>(a.z)[c]));
        static_cast<T *>(a.y)[c] = from_f32<T>(out);
    }
}

template <int N, typename T> hipError_t launch(const StepArgs &a, hipStream_t s) {
    const int64_t threads = a.batch * a.dim * kQuad;
    const dim3 grid(static_cast<unsigned>((threads + kThreads - 1) / kThreads));
    hipLaunchKernelGGL((state_update_kernel<N, T>), grid, dim3(kThreads), 0, s, a);
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
