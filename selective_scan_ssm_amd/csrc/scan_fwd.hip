// Forward selective scan for 1 <= d_state <= 16 on gfx950.
//
// Recurrence per (b, d) chain (youngju.dev guide, section 2 ZOH + discrete
// recurrence; section 5 selective_scan with Delta*B*x input, D skip, SiLU(z)
// gate of the block):
//     h[n] <- exp(Delta_t A[d,n]) h[n] + Delta_t B[b,t,n] x[b,t,d]
//     y     = (sum_n C[b,t,n] h[n] + D[d] x) * SiLU(z)
//
// Mapping: one lane owns one (b, d) chain and keeps all N states in VGPRs for
// the whole sequence, so each (t, d, n) item costs (bf16 io) one v_exp_f32 and
// three VALU ops plus one FMA of the readout, and the per-element work (softplus,
// Delta*x, D*x, SiLU, bf16 conversion) is paid once per N items.  A wave
// covers 64 consecutive channels of one batch row, so B[b,t,:] and C[b,t,:]
// are wave-uniform and come in through scalar loads; x, delta, z are read
// along d (128 contiguous bytes per wave for bf16) and prefetched one chunk
// of kChunk steps ahead so the memory latency hides behind the recurrence.
#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

constexpr int kWave = 64;
constexpr int kChunk = 8;

// Widen B and C to fp32 once (they are tiny: batch * seqlen * d_state values)
// so the scan can take them straight from scalar loads with no unpacking.
template <typename T>
__global__ __launch_bounds__(256) void widen_bc_kernel(const T *__restrict__ B, const T *__restrict__ C,
                                                      float *__restrict__ Bf, float *__restrict__ Cf,
                                                      int64_t count) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < count) {
        Bf[i] = to_f32(B[i]);
        Cf[i] = to_f32(C[i]);
    }
}

// Pointers come in as separate __restrict__ kernel parameters: that is what
// lets the compiler prove B/C are never written and read them with scalar
// loads into SGPRs.
template <int N, typename T>
__global__ __launch_bounds__(kWave) void scan_fwd_chain_kernel(
    const T *__restrict__ x_in, const T *__restrict__ delta_in, const T *__restrict__ z_in,
    const float *__restrict__ Bf, const float *__restrict__ Cf, const float *__restrict__ A_in,
    const float *__restrict__ D_in, const float *__restrict__ bias_in, const float *__restrict__ h0_in,
    T *__restrict__ y_out, float *__restrict__ last_out, int64_t seqlen, int64_t dim, int softplus_flag) {
    using M = typename MathFor<T>::type;
    const int64_t b = blockIdx.y;
    const int64_t d_raw = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
    const bool active = d_raw < dim;
    const int64_t d = active ? d_raw : dim - 1;   // inactive lanes shadow the last channel

    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = M::prep_A(A_in[d * N + n]);
        h[n] = h0_in ? h0_in[(b * dim + d) * N + n] : 0.0f;
    }
    const float bias = bias_in ? bias_in[d] : 0.0f;
    const float Dd = D_in ? D_in[d] : 0.0f;
    const bool has_z = z_in != nullptr;
    const bool softplus_on = softplus_flag != 0;

    const int64_t row0 = b * seqlen;   // first (b, t) row
    const T *xp = x_in + row0 * dim + d;
    const T *dp = delta_in + row0 * dim + d;
    const T *zp = has_z ? z_in + row0 * dim + d : xp;
    const float *Bp = Bf + row0 * N;
    const float *Cp = Cf + row0 * N;
    T *yp = y_out + row0 * dim + d;

    T xs[kChunk], ds[kChunk], zs[kChunk];
    if (seqlen > 0) {
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            const int64_t t = k < seqlen ? k : seqlen - 1;
            xs[k] = xp[t * dim];
            ds[k] = dp[t * dim];
            zs[k] = has_z ? zp[t * dim] : xs[k];
        }
    }

    for (int64_t t0 = 0; t0 < seqlen; t0 += kChunk) {
        // prefetch the next chunk (clamped to a valid row; unused past the end)
        T xn[kChunk], dn[kChunk], zn[kChunk];
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            int64_t t = t0 + kChunk + k;
            t = t < seqlen ? t : seqlen - 1;
            xn[k] = xp[t * dim];
            dn[k] = dp[t * dim];
            zn[k] = has_z ? zp[t * dim] : xn[k];
        }
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            const int64_t t = t0 + k;
            if (t < seqlen) {
                const float xv = to_f32(xs[k]);
                const float v = to_f32(ds[k]) + bias;
                const float dt = softplus_on ? M::softplus(v) : v;
                const float dtx = dt * xv;
                float acc = 0.0f;
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float Bn = Bp[t * N + n];
                    const float Cn = Cp[t * N + n];
                    h[n] = M::step(dt * A2[n], h[n], dtx * Bn);
                    acc = fmaf(Cn, h[n], acc);
                }
                float out = fmaf(Dd, xv, acc);
                if (has_z) out *= silu(to_f32(zs[k]));
                if (active) yp[t * dim] = from_f32<T>(out);
            }
        }
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            xs[k] = xn[k];
            ds[k] = dn[k];
            zs[k] = zn[k];
        }
    }

    if (last_out && active) {
#pragma unroll
        for (int n = 0; n < N; ++n) last_out[(b * dim + d) * N + n] = h[n];
    }
}

// fp32 copies of B and C live in the workspace when the io dtype is bf16.
size_t bc_count(const ScanArgs &a) { return static_cast<size_t>(a.batch * a.seqlen * a.dstate); }
size_t bc_bytes(const ScanArgs &a) { return (bc_count(a) * sizeof(float) + 255) & ~size_t(255); }

template <int N, typename T> hipError_t launch_chain(const ScanArgs &a, hipStream_t s) {
    const float *Bf = static_cast<const float *>(a.B);
    const float *Cf = static_cast<const float *>(a.C);
    if (a.bf16 && a.seqlen > 0) {
        if (a.workspace == nullptr || a.workspace_bytes < 2 * bc_bytes(a)) return hipErrorInvalidValue;
        float *wb = static_cast<float *>(a.workspace);
        float *wc = reinterpret_cast<float *>(static_cast<char *>(a.workspace) + bc_bytes(a));
        const int64_t cnt = static_cast<int64_t>(bc_count(a));
        hipLaunchKernelGGL((widen_bc_kernel<T>), dim3(static_cast<unsigned>((cnt + 255) / 256)), dim3(256),
                           0, s, static_cast<const T *>(a.B), static_cast<const T *>(a.C), wb, wc, cnt);
        Bf = wb;
        Cf = wc;
    }
    const dim3 grid(static_cast<unsigned>((a.dim + kWave - 1) / kWave), static_cast<unsigned>(a.batch));
    hipLaunchKernelGGL((scan_fwd_chain_kernel<N, T>), grid, dim3(kWave), 0, s,
                       static_cast<const T *>(a.x), static_cast<const T *>(a.delta),
                       static_cast<const T *>(a.z), Bf, Cf, a.A, a.D, a.delta_bias, a.h0,
                       static_cast<T *>(a.y), a.last_state, a.seqlen, a.dim, a.softplus);
    return hipGetLastError();
}

template <typename T> hipError_t dispatch_n(const ScanArgs &a, hipStream_t s) {
    switch (a.dstate) {
#define SSM_CASE(NN) \
    case NN: return launch_chain<NN, T>(a, s);
        SSM_CASE(1) SSM_CASE(2) SSM_CASE(3) SSM_CASE(4) SSM_CASE(5) SSM_CASE(6) SSM_CASE(7)
        SSM_CASE(8) SSM_CASE(9) SSM_CASE(10) SSM_CASE(11) SSM_CASE(12) SSM_CASE(13)
        SSM_CASE(14) SSM_CASE(15) SSM_CASE(16)
#undef SSM_CASE
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t scan_fwd_workspace(const ScanArgs &a) { return a.bf16 && a.seqlen > 0 ? 2 * bc_bytes(a) : 0; }

hipError_t launch_scan_fwd(const ScanArgs &a, hipStream_t s) {
    if (a.batch == 0 || a.dim == 0) return hipSuccess;
    if (a.bf16) return dispatch_n<bf16_t>(a, s);
    return dispatch_n<float>(a, s);
}

}  // namespace ssm
