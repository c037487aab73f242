// Device helpers shared by the gfx950 selective-scan kernels: io-dtype
// loads/stores, the fp32 elementwise pieces of the discretisation (softplus,
// SiLU) and the hardware transcendental wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- io dtypes
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v.bits) << 16);
}

// fp32 -> io dtype, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
    __bf16 h = static_cast<__bf16>(v);
    bf16_t r;
    r.bits = __builtin_bit_cast(uint16_t, h);
    return r;
}

// ------------------------------------------------------ hardware transcendentals
// v_exp_f32 computes 2^x, v_log_f32 log2(x), v_rcp_f32 1/x (about 1 ulp).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// log(1 + e) for e in [0, 1], accurate for tiny e: with u = 1 + e rounded,
// log1p(e) = log(u) * e / (u - 1) (Goldberg, "What every computer scientist
// should know about floating-point arithmetic", Theorem 4); u == 1 means
// log1p(e) = e to working precision.
__device__ __forceinline__ float log1p_small(float e) {
    const float u = 1.0f + e;
    const float um1 = u - 1.0f;
    const float r = fast_log2(u) * kLn2 * e * fast_rcp(um1);
    return um1 == 0.0f ? e : r;
}

// softplus(v) = log(1 + exp(v)) = max(v, 0) + log(1 + exp(-|v|)).
__device__ __forceinline__ float softplus(float v) {
    const float e = fast_exp2(-fabsf(v) * kLog2e);
    return fmaxf(v, 0.0f) + log1p_small(e);
}

// SiLU(z) = z / (1 + exp(-z)); exp overflow to +inf gives the correct -0 limit.
__device__ __forceinline__ float silu(float z) {
    return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

}  // namespace ssm
