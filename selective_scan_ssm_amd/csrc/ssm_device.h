// Device helpers shared by the gfx950 selective-scan kernels: io-dtype
// conversions, the fp32 elementwise pieces of the discretisation (softplus,
// the per-state decay, SiLU) in two precisions, and hardware transcendental
// wrappers.
//
// Two math policies:
//   FastMath    -- v_exp_f32 / v_log_f32 / v_rcp_f32 straight from the
//                  hardware.  Used for bf16 io, whose output rounding (2^-9)
//                  is orders of magnitude above their error.
//   PreciseMath -- used for fp32 io.  Two hardware shortcuts are not good
//                  enough there:
//                  * v_exp_f32 is about 0.1 ulp biased below 1 for small
//                    arguments, and a decay close to 1 is multiplied into the
//                    state thousands of times, so the bias compounds
//                    (~T * 0.1 ulp).  The decay is instead applied as
//                    h + expm1(Delta*A) * h with an accurate expm1, so no
//                    near-1 factor is ever rounded.
//                  * log1p in softplus is taken from a series instead of
//                    v_log_f32 near 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLn2Hi = 0.693147182464599609375f;   // float(ln 2)
constexpr float kLn2Lo = -1.904654323148236e-09f;    // ln 2 - kLn2Hi

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

// ------------------------------------------------------------ buffer access
// Raw buffer descriptors: 32-bit byte offsets from a per-wave base, and the
// buffer unit's range check (offset >= num_records) makes loads return 0 and
// drops stores, so tails and inactive lanes need no branch.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr uint32_t kOffNone = 0x80000000u; // an offset beyond every descriptor's range

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes = 0x7fffffffu) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

// Cache policy bits of a buffer access: kStream marks data read or written
// once (non-temporal), which an HBM-bound kernel streams past the caches.
constexpr int kCached = 0;
constexpr int kStream = 2;

template <typename T> struct Io;
template <> struct Io<bf16_t> {
    using raw = uint16_t;
    template <int CP = kCached>
    static __device__ __forceinline__ raw load(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, CP);
    }
    static __device__ __forceinline__ float f32(raw v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
    template <int CP = kCached>
    static __device__ __forceinline__ void store(float v, rsrc_t r, uint32_t voff, uint32_t soff) {
        __builtin_amdgcn_raw_buffer_store_b16(from_f32<bf16_t>(v).bits, r, voff, soff, CP);
    }
};
template <> struct Io<float> {
    using raw = uint32_t;
    template <int CP = kCached>
    static __device__ __forceinline__ raw load(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, CP);
    }
    static __device__ __forceinline__ float f32(raw v) { return __uint_as_float(v); }
    template <int CP = kCached>
    static __device__ __forceinline__ void store(float v, rsrc_t r, uint32_t voff, uint32_t soff) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, CP);
    }
};
// ------------------------------------------------------ hardware transcendentals
// v_exp_f32 computes 2^x, v_log_f32 log2(x), v_rcp_f32 1/x (within 1 ulp).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// SiLU(z) = z / (1 + exp(-z)); exp overflow to +inf gives the correct -0 limit.
// Its error does not accumulate anywhere, so one form serves both policies.
__device__ __forceinline__ float silu(float z) {
    return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

// ----------------------------------------------------------- accurate pieces
// expm1(x) to a few ulp for any x (overflow above ~88): x = k ln2 + r with
// |r| <= ln2/2 (two-part ln2), expm1(r) by its Taylor series through r^7
// (truncation < 1.5e-8 relative), then expm1(x) = 2^k expm1(r) + (2^k - 1).
__device__ __forceinline__ float expm1_accurate(float x) {
    const float k = rintf(x * kLog2e);
    float r = fmaf(-k, kLn2Hi, x);
    r = fmaf(-k, kLn2Lo, r);
    float q = fmaf(r, 1.0f / 5040.0f, 1.0f / 720.0f);
    q = fmaf(r, q, 1.0f / 120.0f);
    q = fmaf(r, q, 1.0f / 24.0f);
    q = fmaf(r, q, 1.0f / 6.0f);
    q = fmaf(r, q, 0.5f);
    q = fmaf(r, q, 1.0f);
    const float p = r * q;                                   // expm1(r)
    const float scale = __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(k));
    return fmaf(scale, p, scale - 1.0f);
}

// log(1 + e) for e in [0, 1]: with s = e / (2 + e) <= 1/3,
// log1p(e) = 2 atanh(s) = 2 s (1 + s^2/3 + s^4/5 + ... + s^12/13)
// (truncation < 1.4e-8 relative).
__device__ __forceinline__ float log1p_unit(float e) {
    const float s = e * fast_rcp(2.0f + e);
    const float w = s * s;
    float q = fmaf(w, 1.0f / 13.0f, 1.0f / 11.0f);
    q = fmaf(w, q, 1.0f / 9.0f);
    q = fmaf(w, q, 1.0f / 7.0f);
    q = fmaf(w, q, 1.0f / 5.0f);
    q = fmaf(w, q, 1.0f / 3.0f);
    q = fmaf(w, q, 1.0f);
    return 2.0f * s * q;
}

// ------------------------------------------------------------- math policies
struct FastMath {
    // softplus(v) = max(v, 0) + log(1 + e), e = exp(-|v|) in (0, 1], with
    // log(1 + e) taken as log2 of the rounded fp32 sum 1 + e, times ln 2.  The
    // rounding of 1 + e costs at most 2^-24 absolutely: the result keeps an
    // absolute error below 1e-7 everywhere (far under bf16 resolution), while
    // for v below about -10, where Delta itself is under 5e-5, the relative
    // error of that tiny Delta grows.  Five VALU slots fewer per value than a
    // separate small-e branch.
    static __device__ __forceinline__ float softplus(float v) {
        const float e = fast_exp2(-fabsf(v) * kLog2e);
        return fmaf(fast_log2(1.0f + e), kLn2, fmaxf(v, 0.0f));
    }
    // the per-state decay factor exp(Delta * A), with A pre-scaled by log2(e)
    static constexpr bool kScaledA = true;
    static __device__ __forceinline__ float prep_A(float a) { return a * kLog2e; }
    // one recurrence step h <- exp(Delta A) h + u, arg = Delta * prep_A(A)
    static __device__ __forceinline__ float step(float arg, float h, float u) {
        return fmaf(fast_exp2(arg), h, u);
    }
    // exp(A * S) as a plain factor (aggregates of several steps)
    static __device__ __forceinline__ float decay(float arg) { return fast_exp2(arg); }
    // the same step split in two, for kernels that keep the factor between passes
    static __device__ __forceinline__ float factor(float arg) { return fast_exp2(arg); }
    static __device__ __forceinline__ float apply(float f, float h, float u) { return fmaf(f, h, u); }
    // factor of two runs of steps in sequence (decay product)
    static __device__ __forceinline__ float compose(float f1, float f2) { return f1 * f2; }
    static constexpr float kIdentity = 1.0f;
};

struct PreciseMath {
    static __device__ __forceinline__ float softplus(float v) {
        return fmaxf(v, 0.0f) + ssm::log1p_unit(fast_exp2(-fabsf(v) * kLog2e));
    }
    static constexpr bool kScaledA = false;
    static __device__ __forceinline__ float prep_A(float a) { return a; }
    // (h + expm1(Delta A) h) + u: the near-1 factor exp(Delta A) is never
    // rounded, and exp(Delta A) h comes out of one fma (no h + u - h
    // cancellation when the decay is fast)
    static __device__ __forceinline__ float step(float arg, float h, float u) {
        return fmaf(expm1_accurate(arg), h, h) + u;
    }
    static __device__ __forceinline__ float decay(float arg) { return expm1_accurate(arg) + 1.0f; }
    static __device__ __forceinline__ float factor(float arg) { return expm1_accurate(arg); }
    static __device__ __forceinline__ float apply(float f, float h, float u) { return fmaf(f, h, h) + u; }
    // (1 + f1)(1 + f2) - 1 without forming the near-1 products
    static __device__ __forceinline__ float compose(float f1, float f2) { return fmaf(f1, f2, f1 + f2); }
    static constexpr float kIdentity = 0.0f;
};

template <typename T> struct MathFor;
template <> struct MathFor<float> { using type = PreciseMath; };
template <> struct MathFor<bf16_t> { using type = FastMath; };

}  // namespace ssm
