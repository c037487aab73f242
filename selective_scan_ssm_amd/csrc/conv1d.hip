// The causal depthwise convolution (+ SiLU) that produces the scan's input x
// in a Mamba block (youngju.dev guide, section 5, "complete Mamba
// implementation": nn.Conv1d with one filter per channel, kernel size d_conv,
// causal padding, then SiLU), and its decode form with a rolling window of
// the last width - 1 inputs.
//     out[b, t, d] = bias[d] + sum_{k<K} w[d, k] x[b, t - (K - 1) + k, d]
// with the inputs before step 0 taken from the caller's state (or 0).
//
// HBM-bound: every input is read once from HBM and every output written
// once.  This is the stand-alone form (its output is the scan's input); the
// same filter also runs inside the d_state-16 scan kernel when the caller
// asks for both at once (ssm_conv_scan_fwd), where the filtered x never
// leaves the registers.  Below d_state 16 that call runs this kernel with an
// fp32 output in its workspace, which the scan then reads.
//
// conv1d_kernel: a lane owns VEC consecutive channels (VEC = 4 when d_inner
// and the pointers allow 8- or 16-byte accesses, else 1) and a wave 64*VEC
// channels of one time chunk of kChunk steps; the K - 1 inputs before the
// chunk are read again (3 of 128 rows at K = 4).  Rows are loaded eight steps
// ahead of their use.
#include <type_traits>

#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

#ifndef SSM_CONV_CHUNK
#define SSM_CONV_CHUNK 128
#endif
#ifndef SSM_CONV_AHEAD
#define SSM_CONV_AHEAD 8
#endif
constexpr int kChunk = SSM_CONV_CHUNK;   // steps per wave
constexpr int kAhead = SSM_CONV_AHEAD;   // rows in flight per lane
static_assert(kChunk % kAhead == 0, "chunks end on a load group");
constexpr int kConvWaves = 4;      // waves per workgroup (consecutive chunks)

struct ConvParams {
    const void *x;
    const float *w, *bias;
    const void *state_in;
    void *out;
    int64_t seqlen, dim;
    int silu;
};

template <typename T, int VEC> struct Row;
template <typename T> struct Row<T, 1> {
    using raw = typename Io<T>::raw;
    static __device__ __forceinline__ void load(raw (&r)[1], rsrc_t rs, uint32_t off) { r[0] = Io<T>::load(rs, off, 0); }
    static __device__ __forceinline__ float get(const raw (&r)[1], int) { return Io<T>::f32(r[0]); }
};
template <> struct Row<bf16_t, 4> {
    typedef uint32_t raw __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ void load(raw (&r)[1], rsrc_t rs, uint32_t off) {
        r[0] = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kStream);
    }
    static __device__ __forceinline__ float get(const raw (&r)[1], int i) {
        const uint32_t wd = r[0][i / 2];
        return __uint_as_float(i % 2 ? (wd & 0xffff0000u) : (wd << 16));
    }
};
template <> struct Row<float, 4> {
    typedef uint32_t raw __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ void load(raw (&r)[1], rsrc_t rs, uint32_t off) {
        r[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kStream);
    }
    static __device__ __forceinline__ float get(const raw (&r)[1], int i) { return __uint_as_float(r[0][i]); }
};

template <typename T, int VEC> __device__ __forceinline__ void store_row(const float (&v)[VEC], rsrc_t rs, uint32_t off);
template <> __device__ __forceinline__ void store_row<float, 1>(const float (&v)[1], rsrc_t rs, uint32_t off) {
    Io<float>::store<kStream>(v[0], rs, off, 0);
}
template <> __device__ __forceinline__ void store_row<bf16_t, 1>(const float (&v)[1], rsrc_t rs, uint32_t off) {
    Io<bf16_t>::store<kStream>(v[0], rs, off, 0);
}
template <> __device__ __forceinline__ void store_row<float, 4>(const float (&v)[4], rsrc_t rs, uint32_t off) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    u4 q = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(q, rs, off, 0, kStream);
}
template <> __device__ __forceinline__ void store_row<bf16_t, 4>(const float (&v)[4], rsrc_t rs, uint32_t off) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    u2 q = {static_cast<uint32_t>(from_f32<bf16_t>(v[0]).bits) | (static_cast<uint32_t>(from_f32<bf16_t>(v[1]).bits) << 16),
            static_cast<uint32_t>(from_f32<bf16_t>(v[2]).bits) | (static_cast<uint32_t>(from_f32<bf16_t>(v[3]).bits) << 16)};
    __builtin_amdgcn_raw_buffer_store_b64(q, rs, off, 0, kStream);
}

// TO: the type of out -- T, or float for an fp32 intermediate that the scan
// reads next (the fused prologue at d_state below 16).
template <typename T, int K, int VEC, typename TO = T>
__global__ __launch_bounds__(kConvWaves * 64) void conv1d_kernel(ConvParams p) {
    using RW = Row<T, VEC>;
    using raw = typename RW::raw;
    constexpr uint32_t es = sizeof(T);
    constexpr int H = K - 1;
    const int lane = threadIdx.x % 64;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int b = blockIdx.z;
    const int64_t T_ = p.seqlen, dim = p.dim;
    const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * 64 + lane) * VEC;   // first channel of the lane
    const bool active = c0 < dim;                  // VEC = 4 only when dim % 4 == 0
    const int64_t cc = active ? c0 : 0;
    const int64_t t0 = (static_cast<int64_t>(blockIdx.y) * kConvWaves + w) * kChunk;
    if (t0 >= T_) return;                          // whole wave past the sequence (uniform)
    const int64_t t1 = t0 + kChunk < T_ ? t0 + kChunk : T_;

    float wt[VEC][K], bias[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
#pragma unroll
        for (int k = 0; k < K; ++k) wt[v][k] = p.w[(cc + v) * K + k];
        bias[v] = p.bias ? p.bias[cc + v] : 0.0f;
    }
    const int64_t base = static_cast<int64_t>(b) * T_ * dim * es;
    const uint32_t bytes = static_cast<uint32_t>(T_ * dim * es);
    const rsrc_t rx = make_rsrc(static_cast<const char *>(p.x) + base, bytes);
    constexpr uint32_t eo = sizeof(TO);
    const rsrc_t ro = make_rsrc(static_cast<char *>(p.out) + static_cast<int64_t>(b) * T_ * dim * eo,
                                static_cast<uint32_t>(T_ * dim * eo));
    auto row_off = [&](int64_t t) -> uint32_t {
        return (active && t >= 0 && t < T_) ? static_cast<uint32_t>((t * dim + c0) * es) : kOffNone;
    };
    auto out_off = [&](int64_t t) -> uint32_t {
        return (active && t >= 0 && t < T_) ? static_cast<uint32_t>((t * dim + c0) * eo) : kOffNone;
    };

    // the K - 1 inputs before the chunk: from x, or from the state before the sequence
    float hist[VEC][H > 0 ? H : 1];
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const int64_t t = t0 - H + j;
        if (t >= 0) {
            raw r[1];
            RW::load(r, rx, row_off(t));
#pragma unroll
            for (int v = 0; v < VEC; ++v) hist[v][j] = RW::get(r, v);
        } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v)
                hist[v][j] = (p.state_in && active)
                                 ? Io<T>::f32(static_cast<const typename Io<T>::raw *>(p.state_in)
                                                  [((static_cast<int64_t>(b) * dim + cc + v) * H) + (H + t)])
                                 : 0.0f;
        }
    }

    raw cur[kAhead][1], nxt[kAhead][1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) RW::load(cur[i], rx, row_off(t0 + i));
    for (int64_t ts = t0; ts < t1; ts += kAhead) {
#pragma unroll
        for (int i = 0; i < kAhead; ++i) RW::load(nxt[i], rx, row_off(ts + kAhead + i));
#pragma unroll
        for (int i = 0; i < kAhead; ++i) {
            float o[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const float xv = RW::get(cur[i], v);
                float acc = fmaf(wt[v][H], xv, bias[v]);
#pragma unroll
                for (int j = 0; j < H; ++j) acc = fmaf(wt[v][j], hist[v][j], acc);
                o[v] = p.silu ? silu(acc) : acc;
#pragma unroll
                for (int j = 0; j + 1 < H; ++j) hist[v][j] = hist[v][j + 1];
                if (H > 0) hist[v][H > 0 ? H - 1 : 0] = xv;
            }
            store_row<TO, VEC>(o, ro, out_off(ts + i));  // rows past the sequence are dropped
        }
#pragma unroll
        for (int i = 0; i < kAhead; ++i) cur[i][0] = nxt[i][0];
    }
}

// The window after the sequence: the last K - 1 inputs of (state_in, x).
template <typename T>
__global__ __launch_bounds__(256) void conv_state_out_kernel(ConvParams p, void *state_out, int H, int64_t batch) {
    using raw = typename Io<T>::raw;
    const int64_t n = batch * p.dim * H;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t j = i % H, bd = i / H, d = bd % p.dim, b = bd / p.dim;
    const int64_t s = p.seqlen - H + j;              // step of the extended sequence
    raw v;
    if (s >= 0)
        v = static_cast<const raw *>(p.x)[(b * p.seqlen + s) * p.dim + d];
    else
        v = p.state_in ? static_cast<const raw *>(p.state_in)[bd * H + (H + s)] : raw(0);
    static_cast<raw *>(state_out)[i] = v;
}

// One decode token per channel: out = filter over (window, x); the window
// shifts by one and takes x.
template <typename T, int K>
__global__ __launch_bounds__(256) void conv_update_kernel(void *state, const void *x, const float *w,
                                                          const float *bias, void *out, int silu_on,
                                                          int64_t batch, int64_t dim) {
    using raw = typename Io<T>::raw;
    constexpr int H = K - 1;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= batch * dim) return;
    const int64_t d = i % dim;
    raw *st = static_cast<raw *>(state) + i * H;
    const raw xr = static_cast<const raw *>(x)[i];
    float acc = bias ? bias[d] : 0.0f;
    raw win[H > 0 ? H : 1];
#pragma unroll
    for (int k = 0; k < H; ++k) {
        win[k] = st[k];
        acc = fmaf(w[d * K + k], Io<T>::f32(win[k]), acc);
    }
    acc = fmaf(w[d * K + H], Io<T>::f32(xr), acc);
    const float o = silu_on ? silu(acc) : acc;
    if constexpr (sizeof(raw) == 2)
        static_cast<raw *>(out)[i] = from_f32<bf16_t>(o).bits;
    else
        static_cast<raw *>(out)[i] = __float_as_uint(o);
#pragma unroll
    for (int k = 0; k + 1 < H; ++k) st[k] = win[k + 1];
    if (H > 0) st[H > 0 ? H - 1 : 0] = xr;
}

template <typename T, int K, int VEC, typename TO = T> hipError_t launch_conv_t(const ConvArgs &a, hipStream_t s) {
    ConvParams p;
    p.x = a.x; p.w = a.weight; p.bias = a.bias; p.state_in = a.state_in; p.out = a.out;
    p.seqlen = a.seqlen; p.dim = a.dim; p.silu = a.silu;
    if (a.seqlen > 0) {
        const int64_t chunks = (a.seqlen + kChunk - 1) / kChunk;
        const dim3 grid(static_cast<unsigned>((a.dim + 64 * VEC - 1) / (64 * VEC)),
                        static_cast<unsigned>((chunks + kConvWaves - 1) / kConvWaves),
                        static_cast<unsigned>(a.batch));
        hipLaunchKernelGGL((conv1d_kernel<T, K, VEC, TO>), grid, dim3(kConvWaves * 64), 0, s, p);
    }
    if (a.state_out && K > 1) {
        const int64_t n = a.batch * a.dim * (K - 1);
        hipLaunchKernelGGL(conv_state_out_kernel<T>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                           p, a.state_out, K - 1, a.batch);
    }
    return hipGetLastError();
}

template <typename T, int K> hipError_t launch_conv_k(const ConvArgs &a, hipStream_t s) {
    const size_t vec_bytes = 4 * sizeof(T);
    const size_t out_bytes = 4 * (a.out_f32 ? sizeof(float) : sizeof(T));
    const bool vec = a.dim % 4 == 0 && reinterpret_cast<uintptr_t>(a.x) % vec_bytes == 0 &&
                     reinterpret_cast<uintptr_t>(a.out) % out_bytes == 0;
    if (a.out_f32 && !std::is_same<T, float>::value)
        return vec ? launch_conv_t<T, K, 4, float>(a, s) : launch_conv_t<T, K, 1, float>(a, s);
    return vec ? launch_conv_t<T, K, 4>(a, s) : launch_conv_t<T, K, 1>(a, s);
}

template <typename T> hipError_t launch_conv_dt(const ConvArgs &a, hipStream_t s) {
    switch (a.width) {
    case 1: return launch_conv_k<T, 1>(a, s);
    case 2: return launch_conv_k<T, 2>(a, s);
    case 3: return launch_conv_k<T, 3>(a, s);
    default: return launch_conv_k<T, 4>(a, s);
    }
}

template <typename T> hipError_t launch_update_dt(const ConvUpdateArgs &a, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>((a.batch * a.dim + 255) / 256);
    switch (a.width) {
    case 1: hipLaunchKernelGGL((conv_update_kernel<T, 1>), dim3(grid), dim3(256), 0, s, a.state, a.x, a.weight, a.bias, a.out, a.silu, a.batch, a.dim); break;
    case 2: hipLaunchKernelGGL((conv_update_kernel<T, 2>), dim3(grid), dim3(256), 0, s, a.state, a.x, a.weight, a.bias, a.out, a.silu, a.batch, a.dim); break;
    case 3: hipLaunchKernelGGL((conv_update_kernel<T, 3>), dim3(grid), dim3(256), 0, s, a.state, a.x, a.weight, a.bias, a.out, a.silu, a.batch, a.dim); break;
    default: hipLaunchKernelGGL((conv_update_kernel<T, 4>), dim3(grid), dim3(256), 0, s, a.state, a.x, a.weight, a.bias, a.out, a.silu, a.batch, a.dim); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv1d(const ConvArgs &a, hipStream_t s) {
    return a.bf16 ? launch_conv_dt<bf16_t>(a, s) : launch_conv_dt<float>(a, s);
}

hipError_t launch_conv_state_out(const ConvArgs &a, hipStream_t s) {
    if (!a.state_out || a.width <= 1 || a.batch == 0 || a.dim == 0) return hipSuccess;
    ConvParams p{};
    p.x = a.x; p.state_in = a.state_in; p.seqlen = a.seqlen; p.dim = a.dim;
    const int64_t n = a.batch * a.dim * (a.width - 1);
    const dim3 grid(static_cast<unsigned>((n + 255) / 256));
    if (a.bf16)
        hipLaunchKernelGGL(conv_state_out_kernel<bf16_t>, grid, dim3(256), 0, s, p, a.state_out, a.width - 1, a.batch);
    else
        hipLaunchKernelGGL(conv_state_out_kernel<float>, grid, dim3(256), 0, s, p, a.state_out, a.width - 1, a.batch);
    return hipGetLastError();
}

hipError_t launch_conv1d_update(const ConvUpdateArgs &a, hipStream_t s) {
    return a.bf16 ? launch_update_dt<bf16_t>(a, s) : launch_update_dt<float>(a, s);
}

}  // namespace ssm
