// The Mamba-2 multi-head scan (youngju.dev guide, section 6 "Mamba 2": the
// SSM with one scalar decay per head is a semiseparable matrix, evaluated in
// chunks -- matrix products inside a chunk, the recurrence between chunks).
//
// Per (batch b, head h) and channel p of the head, with
//   Delta_t = softplus(dt[b,t,h] + dt_bias[h]),  a_t = Delta_t A[h],
//   S[p, n] <- exp(a_t) S[p, n] + Delta_t x[t, p] B[t, n],
//   y[t, p]  = (sum_n C[t, n] S[p, n] + D[h] x[t, p]) SiLU(z[t, p]).
// B and C (one per step) are shared by all heads.
//
// One workgroup (4 waves) owns (b, h, a tile of PT channels) and walks the
// sequence in chunks of Q = 64 steps, keeping the state S (PT x N, fp32) in
// MFMA accumulators.  With s_t the prefix sum of a over the chunk (fp64) and
// S_in the state entering the chunk, chunk c is three products:
//   G^T = B C^T (Q x Q; only s <= t blocks), masked into
//   M[t, s] = G[t, s] Delta_s exp(s_t - s_s)  (s <= t), 0 above,
//   Y^T   = X^T M^T + (S_in C^T) diag(exp(s_t))             (PT x Q)
//   S^T   = exp(s_Q) S_in^T + (B diag(w))^T X, w_s = Delta_s exp(s_Q - s_s).
// bf16 io uses v_mfma_f32_16x16x32_bf16 (M, S_in and B w rounded to bf16 as
// operands, every sum and the carried state in fp32); fp32 io uses
// v_mfma_f32_16x16x4_f32 with fp32 operands throughout.
//
// The prefix sums are taken in fp64 so that exp(s_t - s_s) keeps full fp32
// accuracy even when the chunk's total decay is large (an fp32 prefix would
// lose |s| * 2^-24 absolutely in every difference).
//
// bf16 operands that are computed (M, S_in, B w) are carried as two bf16
// terms, hi = bf16(v) and lo = bf16(v - hi), and each product with them is two
// MFMAs: a single bf16 rounding of these operands costs up to 3e-2 relative
// error in y at the layer shapes, the two-term form about 2^-17.  x, z, B, C
// are bf16 already and enter exactly.
//
// LDS: C and B natural (rows t / s, n contiguous), B w and X transposed (rows
// n / p, s contiguous), M (rows t, s contiguous), S_in (rows p, n contiguous;
// two buffers, written by one chunk and read by the next).  Every MFMA
// operand fragment is then one contiguous read along its K axis.  Three
// barriers per chunk: before staging (the previous chunk's readers are done),
// after staging, after M.
#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

constexpr int kQ = 64;          // chunk length (steps)
// Waves per workgroup: 4, one per 16-step block of a chunk, each owning that
// block's output tiles for every 16-channel block of the workgroup; or
// (WIDE) 4 per 16-channel block, one output tile each.  The wide form halves
// each wave's chain of dependent LDS reads and MFMAs, which pays when there is
// at most one workgroup per CU; with more, two narrow workgroups share a CU
// better (the wide one saturates a CU's LDS on its own).
template <int PT, bool WIDE> constexpr int waves_for() { return WIDE ? 4 * (PT / 16) : 4; }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// MFMA operand policy per io dtype: LDS element, K per instruction, K
// elements held per lane, fragment load and the instruction.
//   16x16 output tile: lane l holds rows 4 (l / 16) + v (v < 4) of column l % 16;
//   operand A lane l holds row l % 16, K elements KPL (l / 16) .. + KPL - 1;
//   operand B lane l holds column l % 16, the same K elements.
template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
    using E = uint16_t;
    static constexpr int KB = 32, KPL = 8;
    // a computed operand is carried as hi + lo (two bf16 terms, 16 significant bits)
    static constexpr int NS = 2;
    using frag = bf16x8_t;
    static __device__ __forceinline__ frag load(const E *p) {
        return __builtin_bit_cast(frag, *reinterpret_cast<const u16x8_t *>(p));
    }
    static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ E enc(float v) { return from_f32<bf16_t>(v).bits; }
    static __device__ __forceinline__ float dec(E v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
    // term q of v: q = 0 the bf16 rounding of v, q = 1 the rounding of what is left
    static __device__ __forceinline__ float term(float v, int q) {
        const float hi = dec(enc(v));
        return q == 0 ? hi : v - hi;
    }
    // four consecutive elements to LDS (8 bytes)
    static __device__ __forceinline__ void put4(E *p, float a, float b, float c, float d) {
        const u32x2_t q = {static_cast<uint32_t>(enc(a)) | (static_cast<uint32_t>(enc(b)) << 16),
                           static_cast<uint32_t>(enc(c)) | (static_cast<uint32_t>(enc(d)) << 16)};
        *reinterpret_cast<u32x2_t *>(p) = q;
    }
    // two consecutive elements to LDS (4 bytes)
    static __device__ __forceinline__ void put2(E *p, E a, E b) {
        *reinterpret_cast<uint32_t *>(p) = static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
    }
};
template <> struct Mma<float> {
    using E = float;
    static constexpr int KB = 4, KPL = 1;
    static constexpr int NS = 1;
    static __device__ __forceinline__ float term(float v, int) { return v; }
    using frag = float;
    static __device__ __forceinline__ frag load(const E *p) { return *p; }
    static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ E enc(float v) { return v; }
    static __device__ __forceinline__ float dec(E v) { return v; }
    static __device__ __forceinline__ void put4(E *p, float a, float b, float c, float d) {
        *reinterpret_cast<f32x4_t *>(p) = f32x4_t{a, b, c, d};
    }
    static __device__ __forceinline__ void put2(E *p, E a, E b) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<f2 *>(p) = f2{a, b};
    }
};

// Chunk prefix sums of a_t = Delta_t A in "scaled" units: log2 units (a
// log2(e)) with fp32 sums for FastMath, natural units with fp64 sums for
// PreciseMath.  exp of a difference d of two prefixes, and of the carried
// state's decay over a chunk, in those units.
template <typename M> struct Steps;
template <> struct Steps<FastMath> {
    using real = float;
    static constexpr float kScale = kLog2e;
    static __device__ __forceinline__ float ex(float d) { return fast_exp2(d); }
    static __device__ __forceinline__ f32x4_t decay(float d, f32x4_t h) { return h * fast_exp2(d); }
    // inclusive prefix over the 64 lanes: row_shr 1, 2, 4, 8 inside each row of
    // 16 lanes (bound_ctrl: 0 from outside the row), then the row totals
    template <int CTRL> static __device__ __forceinline__ float shr(float v) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
    }
    static __device__ __forceinline__ float prefix(float v, int lane) {
        v += shr<0x111>(v);
        v += shr<0x112>(v);
        v += shr<0x114>(v);
        v += shr<0x118>(v);
        const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
        const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
        const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47));
        const int row = lane >> 4;
        return v + ((row >= 1 ? r0 : 0.0f) + (row >= 2 ? r1 : 0.0f) + (row >= 3 ? r2 : 0.0f));
    }
    // v of lane l, l the same in every lane
    static __device__ __forceinline__ float lane_value(float v, int l) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
    }
    // v of lane l, l per lane
    static __device__ __forceinline__ float gather(float v, int l) { return __shfl(v, l); }
};
template <> struct Steps<PreciseMath> {
    using real = double;
    static constexpr float kScale = 1.0f;
    static __device__ __forceinline__ float ex(float d) { return expm1_accurate(d) + 1.0f; }
    static __device__ __forceinline__ f32x4_t decay(float d, f32x4_t h) {
        const float f = expm1_accurate(d);
        return f32x4_t{fmaf(f, h[0], h[0]), fmaf(f, h[1], h[1]), fmaf(f, h[2], h[2]), fmaf(f, h[3], h[3])};
    }
    static __device__ __forceinline__ double prefix(double v, int lane) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double u = __shfl_up(v, o);
            if (lane >= o) v += u;
        }
        return v;
    }
    static __device__ __forceinline__ double lane_value(double v, int l) { return __shfl(v, l); }
    static __device__ __forceinline__ double gather(double v, int l) { return __shfl(v, l); }
};

// io rows of four consecutive elements (8 bytes bf16, 16 bytes fp32)
template <typename T> struct Quad;
template <> struct Quad<bf16_t> {
    using raw = u32x2_t;
    static __device__ __forceinline__ raw load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kStream);
    }
    static __device__ __forceinline__ float get(const raw &q, int i) {
        const uint32_t wd = q[i / 2];
        return __uint_as_float(i % 2 ? (wd & 0xffff0000u) : (wd << 16));
    }
    static __device__ __forceinline__ void store(const float (&v)[4], rsrc_t r, uint32_t off) {
        const u32x2_t q = {static_cast<uint32_t>(from_f32<bf16_t>(v[0]).bits) |
                               (static_cast<uint32_t>(from_f32<bf16_t>(v[1]).bits) << 16),
                           static_cast<uint32_t>(from_f32<bf16_t>(v[2]).bits) |
                               (static_cast<uint32_t>(from_f32<bf16_t>(v[3]).bits) << 16)};
        __builtin_amdgcn_raw_buffer_store_b64(q, r, off, 0, kStream);
    }
};
template <> struct Quad<float> {
    using raw = u32x4_t;
    static __device__ __forceinline__ raw load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStream);
    }
    static __device__ __forceinline__ float get(const raw &q, int i) { return __uint_as_float(q[i]); }
    static __device__ __forceinline__ void store(const float (&v)[4], rsrc_t r, uint32_t off) {
        const u32x4_t q = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(q, r, off, 0, kStream);
    }
};

struct SsdParams {
    const void *x, *dt, *z, *B, *C;
    const float *dt_bias, *A, *D, *h0;
    void *y;
    float *last;
    int64_t seqlen, nheads, headdim;
    int softplus;
};

// Vectors of 4, 8 or 16 bytes (buffer loads, LDS stores) and their io elements.
template <int BYTES> struct Vec;
template <> struct Vec<16> {
    using t = u32x4_t;
    template <int CP> static __device__ __forceinline__ t load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
    }
};
template <> struct Vec<8> {
    using t = u32x2_t;
    template <int CP> static __device__ __forceinline__ t load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CP);
    }
};
typedef uint32_t u32x1_t __attribute__((ext_vector_type(1)));
template <> struct Vec<4> {
    using t = u32x1_t;
    template <int CP> static __device__ __forceinline__ t load(rsrc_t r, uint32_t off) {
        u32x1_t v;
        v[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP);
        return v;
    }
};
// element e of a loaded vector: as fp32, and as the LDS operand element
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
    template <typename V> static __device__ __forceinline__ float f32(const V &v, int e) {
        return __uint_as_float(e % 2 ? (v[e / 2] & 0xffff0000u) : (v[e / 2] << 16));
    }
    template <typename V> static __device__ __forceinline__ uint16_t raw(const V &v, int e) {
        return static_cast<uint16_t>(e % 2 ? v[e / 2] >> 16 : v[e / 2] & 0xffffu);
    }
};
template <> struct Elem<float> {
    template <typename V> static __device__ __forceinline__ float f32(const V &v, int e) { return __uint_as_float(v[e]); }
    template <typename V> static __device__ __forceinline__ float raw(const V &v, int e) { return __uint_as_float(v[e]); }
};

// Staging piece size: the bytes that make one piece per thread for a chunk
// of rows of `row_bytes` taken two rows at a time (32 row pairs x row_bytes /
// piece = threads), capped at 16 bytes (then a whole number per thread).
constexpr int piece_bytes(int row_bytes, int threads) {
    return row_bytes * 32 / threads > 16 ? 16 : row_bytes * 32 / threads;
}

template <typename T, int N, int PT, bool WIDE>
__global__ __launch_bounds__((64 * waves_for<PT, WIDE>())) void ssd_chunk_kernel(SsdParams p) {
    using MM = Mma<T>;
    using E = typename MM::E;
    using EL = Elem<T>;
    using Math = typename MathFor<T>::type;
    using ST = Steps<Math>;
    using SR = typename ST::real;
    using QD = Quad<T>;
    constexpr uint32_t es = sizeof(T);
    constexpr int NS = MM::NS;                      // terms of a computed operand
    constexpr int PAD = 16 / sizeof(E);             // 16 bytes of row padding
    constexpr int LN = N + PAD;                     // rows with n contiguous
    constexpr int LQ = kQ + PAD;                    // rows with s contiguous
    constexpr int NPT = PT / 16, NNT = N / 16;
    constexpr int kWaves = waves_for<PT, WIDE>(), kThreads = 64 * kWaves;
    constexpr int NPW = NPT * 4 / kWaves;           // 16-channel blocks per wave (output tiles)
    static_assert(NPW >= 1 && NPW * kWaves == NPT * 4, "waves x tiles");
    constexpr int NSTILE = NNT * NPT;               // 16x16 state tiles
    constexpr int NST = (NSTILE + kWaves - 1) / kWaves;
    constexpr int KB = MM::KB, KPL = MM::KPL;
    // staging pieces: two rows (steps s, s + 1) x PBB bytes of B and C, PXB of
    // x.  B / C piece u (read from L2) covers the step pair u % 32 and element
    // group u / 32, so its transposed LDS writes fall in distinct banks; x
    // piece u (streamed from HBM) covers element group u % (PT / VX) of step
    // pair u / (PT / VX), so a wave reads whole rows.
    constexpr int PBB = piece_bytes(N * es, kThreads), PXB = piece_bytes(PT * es, kThreads);
    constexpr int VB = PBB / es, VX = PXB / es;     // io elements per piece
    constexpr int UBT = (kQ / 2) * (N / VB) / kThreads, UXT = (kQ / 2) * (PT / VX) / kThreads;
    static_assert(UBT >= 1 && UXT >= 1 && (kQ / 2) * (N / VB) == UBT * kThreads &&
                  (kQ / 2) * (PT / VX) == UXT * kThreads, "one or more whole pieces per thread");
    static_assert(N % KB == 0 && kQ % KB == 0, "tile shapes");
    using VBt = typename Vec<PBB>::t;
    using VXt = typename Vec<PXB>::t;

    // one chunk's operands; the state copy alternates between two buffers
    __shared__ __attribute__((aligned(16))) E sC[kQ][LN];       // C[t][n]
    __shared__ __attribute__((aligned(16))) E sB[kQ][LN];       // B[s][n]
    __shared__ __attribute__((aligned(16))) E sBt[N][LQ];       // B[s][n] at [n][s]
    __shared__ __attribute__((aligned(16))) E sX[PT][LQ];       // x[s][p] at [p][s]
    __shared__ __attribute__((aligned(16))) E sXw[NS][PT][LQ];  // w_s x[s][p] at [p][s]
    __shared__ __attribute__((aligned(16))) E sM[NS][kQ][LQ];   // M[t][s]
    __shared__ __attribute__((aligned(16))) E sS[2][NS][PT][LN];// S_in[p][n]
    __shared__ SR sSt[kQ];                          // prefix s_t (scaled units)
    __shared__ __attribute__((aligned(16))) float sDl[kQ];      // Delta_t
    __shared__ __attribute__((aligned(16))) float sU[kQ];       // Delta_s exp(s_e(s) - s_s)
    __shared__ float sR[3][kQ];                     // exp(s_t - s_(16 i + 15))

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, kq = lane >> 4;

    // block -> (b, h, channel tile); consecutive logical blocks (same batch
    // row, so the same B and C) are kept on one XCD when the count allows
    const int64_t H = p.nheads, P = p.headdim, L = p.seqlen;
    const int64_t npb = P / PT;
    const int64_t total = static_cast<int64_t>(gridDim.x);
    int64_t lin = blockIdx.x;
    if (total % 8 == 0) lin = (lin % 8) * (total / 8) + lin / 8;
    const int64_t pt = lin % npb;
    const int64_t h = (lin / npb) % H;
    const int64_t b = lin / (npb * H);
    const int64_t p0 = pt * PT;

    // byte offsets inside one batch row fit in 31 bits (checked by the caller)
    const uint32_t rowX = static_cast<uint32_t>(H * P * es);        // one step of x, z, y
    const uint32_t rowN = static_cast<uint32_t>(N * es);            // one step of B, C
    const uint32_t rowH = static_cast<uint32_t>(H * es);            // one step of dt
    const uint32_t hp0 = static_cast<uint32_t>((h * P + p0) * es);  // this tile inside a step
    const rsrc_t rX = make_rsrc(static_cast<const char *>(p.x) + b * L * H * P * es, static_cast<uint32_t>(L) * rowX);
    const rsrc_t rZ = p.z ? make_rsrc(static_cast<const char *>(p.z) + b * L * H * P * es, static_cast<uint32_t>(L) * rowX)
                          : make_rsrc(p.x, 0u);
    const rsrc_t rY = make_rsrc(static_cast<char *>(p.y) + b * L * H * P * es, static_cast<uint32_t>(L) * rowX);
    const rsrc_t rDT = make_rsrc(static_cast<const char *>(p.dt) + b * L * H * es, static_cast<uint32_t>(L) * rowH);
    const rsrc_t rB = make_rsrc(static_cast<const char *>(p.B) + b * L * N * es, static_cast<uint32_t>(L) * rowN);
    const rsrc_t rC = make_rsrc(static_cast<const char *>(p.C) + b * L * N * es, static_cast<uint32_t>(L) * rowN);

    const float Ah = p.A[h] * ST::kScale;
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
    const float Dh = p.D ? p.D[h] : 0.0f;
    const bool has_z = p.z != nullptr;

    // per-thread staging coordinates and chunk-relative byte offsets
    const int sp = 2 * (tid % 32);                  // step pair of every B / C piece of this thread
    int nB0[UBT], qX0[UXT], sX0[UXT];
    uint32_t oB[UBT], oX[UXT];
#pragma unroll
    for (int i = 0; i < UBT; ++i) {
        nB0[i] = ((tid + i * kThreads) / 32) * VB;
        oB[i] = sp * rowN + nB0[i] * es;
    }
#pragma unroll
    for (int i = 0; i < UXT; ++i) {
        const int u = tid + i * kThreads;
        qX0[i] = (u % (PT / VX)) * VX;
        sX0[i] = 2 * (u / (PT / VX));
        oX[i] = sX0[i] * rowX + hp0 + qX0[i] * es;
    }
    // the output tiles of this wave: steps 16 jw .. + 15, channels 16 (pw0 + c) .. + 15, c < NPW
    const int jw = w % 4, pw0 = (w / 4) * NPW;
    uint32_t oZ[NPW];
#pragma unroll
    for (int c = 0; c < NPW; ++c) oZ[c] = (jw * 16 + l16) * rowX + hp0 + ((pw0 + c) * 16 + kq * 4) * es;
    const uint32_t oDT = lane * rowH + static_cast<uint32_t>(h * es);

    // ---- registers of the chunk being fetched
    VBt rb[UBT][2], rc[UBT][2];
    VXt rx[UXT][2];
    typename Io<T>::raw rdt;
    typename QD::raw rz[NPW], rzn[NPW];

    auto fetch = [&](uint32_t t0) __attribute__((always_inline)) {
        const uint32_t cN = t0 * rowN, cX = t0 * rowX;
#pragma unroll
        for (int i = 0; i < UBT; ++i) {
            rb[i][0] = Vec<PBB>::template load<kCached>(rB, cN + oB[i]);
            rb[i][1] = Vec<PBB>::template load<kCached>(rB, cN + oB[i] + rowN);
            rc[i][0] = Vec<PBB>::template load<kCached>(rC, cN + oB[i]);
            rc[i][1] = Vec<PBB>::template load<kCached>(rC, cN + oB[i] + rowN);
        }
#pragma unroll
        for (int i = 0; i < UXT; ++i) {
            rx[i][0] = Vec<PXB>::template load<kStream>(rX, cX + oX[i]);
            rx[i][1] = Vec<PXB>::template load<kStream>(rX, cX + oX[i] + rowX);
        }
        rdt = Io<T>::template load<kStream>(rDT, t0 * rowH + oDT, 0);
#pragma unroll
        for (int c = 0; c < NPW; ++c) rzn[c] = QD::load(rZ, cX + oZ[c]);
    };

    // ---- initial state: accumulators (fp32) and the operand copy
    f32x4_t acc_s[NST];
#pragma unroll
    for (int r = 0; r < NST; ++r) {
        const int q = w + kWaves * r;
        acc_s[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if (q < NSTILE) {
            const int ni = q / NPT, pi = q % NPT;
            const int n = ni * 16 + kq * 4, pp = pi * 16 + l16;
            if (p.h0) {
                const float *src = p.h0 + (((b * H + h) * P + p0 + pp) * N + n);
                acc_s[r] = *reinterpret_cast<const f32x4_t *>(src);
            }
            const f32x4_t a = acc_s[r];
#pragma unroll
            for (int q2 = 0; q2 < NS; ++q2)
                MM::put4(&sS[0][q2][pp][n], MM::term(a[0], q2), MM::term(a[1], q2), MM::term(a[2], q2),
                         MM::term(a[3], q2));
        }
    }
    for (int i = tid; i < NS * kQ * LQ; i += kThreads) (&sM[0][0][0])[i] = MM::enc(0.0f);

    const int64_t nchunks = (L + kQ - 1) / kQ;
    fetch(0);
    // as many (empty) y stores after the first fetch as every later fetch is
    // followed by, so the staging waits for the fetched data only, not for
    // the previous chunk's stores, on every path into the loop
#pragma unroll
    for (int c = 0; c < NPW; ++c) {
        const float zero4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        QD::store(zero4, rY, kOffNone);
    }

    for (int64_t c = 0; c < nchunks; ++c) {
        const int k = static_cast<int>(c & 1);      // state buffer read by this chunk
        const uint32_t t0 = static_cast<uint32_t>(c * kQ);

        // ---- per-step quantities (lane = step), every wave the same
        const bool valid = static_cast<int64_t>(t0) + lane < L;
        const float v = Io<T>::f32(rdt) + bias;
        const float delta = valid ? (p.softplus ? Math::softplus(v) : v) : 0.0f;
        const SR S = ST::prefix(static_cast<SR>(delta * Ah), lane);
        const SR Send = ST::lane_value(S, 63);
        const float wx = delta * ST::ex(static_cast<float>(Send - S));           // state weight of step t
        const float eS = ST::ex(static_cast<float>(S));                           // decay from the chunk start
        const SR Sblk = ST::gather(S, lane | 15);
        const float u = delta * ST::ex(static_cast<float>(Sblk - S));             // to the end of its 16-block
        const float r0 = ST::ex(static_cast<float>(S - ST::lane_value(S, 15)));   // from the end of block 0
        const float r1 = ST::ex(static_cast<float>(S - ST::lane_value(S, 31)));
        const float r2 = ST::ex(static_cast<float>(S - ST::lane_value(S, 47)));
        float xw0[UXT], xw1[UXT];
#pragma unroll
        for (int i = 0; i < UXT; ++i) {
            xw0[i] = __shfl(wx, sX0[i]);
            xw1[i] = __shfl(wx, sX0[i] + 1);
        }

        // ---- stage the chunk into LDS (every reader of the previous chunk is done)
        __syncthreads();
        if (w == 0) {
            sSt[lane] = S;
            sDl[lane] = delta;
            sU[lane] = u;
            sR[0][lane] = r0;
            sR[1][lane] = r1;
            sR[2][lane] = r2;
        }
#pragma unroll
        for (int i = 0; i < UBT; ++i) {
            const int n0 = nB0[i];
            *reinterpret_cast<VBt *>(&sB[sp][n0]) = rb[i][0];
            *reinterpret_cast<VBt *>(&sB[sp + 1][n0]) = rb[i][1];
            *reinterpret_cast<VBt *>(&sC[sp][n0]) = rc[i][0];
            *reinterpret_cast<VBt *>(&sC[sp + 1][n0]) = rc[i][1];
#pragma unroll
            for (int e = 0; e < VB; ++e) MM::put2(&sBt[n0 + e][sp], EL::raw(rb[i][0], e), EL::raw(rb[i][1], e));
        }
#pragma unroll
        for (int i = 0; i < UXT; ++i) {
            const int q0 = qX0[i], sx = sX0[i];
#pragma unroll
            for (int e = 0; e < VX; ++e) {
                MM::put2(&sX[q0 + e][sx], EL::raw(rx[i][0], e), EL::raw(rx[i][1], e));
                const float x0 = EL::f32(rx[i][0], e) * xw0[i], x1 = EL::f32(rx[i][1], e) * xw1[i];
#pragma unroll
                for (int q2 = 0; q2 < NS; ++q2)
                    MM::put2(&sXw[q2][q0 + e][sx], MM::enc(MM::term(x0, q2)), MM::enc(MM::term(x1, q2)));
            }
        }
#pragma unroll
        for (int c = 0; c < NPW; ++c) rz[c] = rzn[c];
        fetch(t0 + kQ);          // the next chunk (past the end: empty reads)
        __syncthreads();

        // ---- before M is needed: this wave's carried-state readout
        // Y_off^T = S_in C^T (steps 16 jw .., its channel blocks) and its state
        // tiles S^T <- exp(s_Q) S^T + B^T (w x); both read only staged operands
        const int t = jw * 16 + l16;
        f32x4_t acc[NPW];
#pragma unroll
        for (int c = 0; c < NPW; ++c) {
            acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            const E *pb = &sC[t][kq * KPL];
#pragma unroll
            for (int q2 = 0; q2 < NS; ++q2) {
                const E *pa = &sS[k][q2][(pw0 + c) * 16 + l16][kq * KPL];
#pragma unroll
                for (int kk = 0; kk < N / KB; ++kk)
                    acc[c] = MM::mma(MM::load(pa + kk * KB), MM::load(pb + kk * KB), acc[c]);
            }
        }
        {
            const float send = static_cast<float>(Send);
#pragma unroll
            for (int r = 0; r < NST; ++r) {
                const int q = w + kWaves * r;
                if (q < NSTILE) {
                    const int ni = q / NPT, pi = q % NPT;
                    f32x4_t a = ST::decay(send, acc_s[r]);
                    const E *pa = &sBt[ni * 16 + l16][kq * KPL];
#pragma unroll
                    for (int kk = 0; kk < kQ / KB; ++kk) {
                        const typename MM::frag fa = MM::load(pa + kk * KB);
#pragma unroll
                        for (int q2 = 0; q2 < NS; ++q2)
                            a = MM::mma(fa, MM::load(&sXw[q2][pi * 16 + l16][kq * KPL] + kk * KB), a);
                    }
                    acc_s[r] = a;
                    // the copy read by the next chunk (the other buffer: its
                    // last readers finished before this chunk's staging)
#pragma unroll
                    for (int q2 = 0; q2 < NS; ++q2)
                        MM::put4(&sS[k ^ 1][q2][pi * 16 + l16][ni * 16 + kq * 4], MM::term(a[0], q2),
                                 MM::term(a[1], q2), MM::term(a[2], q2), MM::term(a[3], q2));
                }
            }
        }

        // ---- M = (C B^T) masked, times Delta_s exp(s_t - s_s), over the ten
        // 16x16 blocks with s-block i <= t-block j: blocks 0..3 the diagonal
        // (exp per element), blocks 4..9 below it, where the factor splits as
        // u_s r_t^(i) (both at most 1); wave w takes blocks w, w + W, w + 2 W
#pragma unroll
        for (int rr = 0; rr < 3; ++rr) {
            const int qb = w + kWaves * rr;
            if (qb >= 10) break;
            const bool diag = qb < 4;
            const int q = qb - 4;                       // off-diagonal: q = j (j - 1) / 2 + i
            const int j = diag ? qb : 1 + (q >= 1) + (q >= 3);
            const int i = diag ? qb : q - j * (j - 1) / 2;
            f32x4_t g = {0.0f, 0.0f, 0.0f, 0.0f};
            const E *pa = &sB[i * 16 + l16][kq * KPL];
            const E *pb = &sC[j * 16 + l16][kq * KPL];
#pragma unroll
            for (int kk = 0; kk < N / KB; ++kk) g = MM::mma(MM::load(pa + kk * KB), MM::load(pb + kk * KB), g);
            const int tm = j * 16 + l16, s0 = i * 16 + kq * 4;
            float m[4];
            if (diag) {
                const f32x4_t dq = *reinterpret_cast<const f32x4_t *>(&sDl[s0]);
                const SR st = sSt[tm];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    m[e] = s0 + e <= tm ? g[e] * dq[e] * ST::ex(static_cast<float>(st - sSt[s0 + e])) : 0.0f;
            } else {
                const f32x4_t uq = *reinterpret_cast<const f32x4_t *>(&sU[s0]);
                const float rt = sR[i][tm];
#pragma unroll
                for (int e = 0; e < 4; ++e) m[e] = g[e] * uq[e] * rt;
            }
#pragma unroll
            for (int q2 = 0; q2 < NS; ++q2)
                MM::put4(&sM[q2][tm][s0], MM::term(m[0], q2), MM::term(m[1], q2), MM::term(m[2], q2),
                         MM::term(m[3], q2));
        }
        __syncthreads();

        // ---- Y^T += X^T M^T for this wave's tiles, then D skip, gate, store
        {
            const float est = __shfl(eS, t);
            constexpr int kmax = kQ / KB;
            const int nkd = (16 * (jw + 1) + KB - 1) / KB;
            const bool tvalid = static_cast<int64_t>(t0) + t < L;
#pragma unroll
            for (int c = 0; c < NPW; ++c) {
                f32x4_t a = acc[c] * est;
                const E *pa2 = &sX[(pw0 + c) * 16 + l16][kq * KPL];
#pragma unroll
                for (int q2 = 0; q2 < NS; ++q2) {
                    const E *pb2 = &sM[q2][t][kq * KPL];
#pragma unroll
                    for (int kk = 0; kk < kmax; ++kk)
                        if (kk < nkd) a = MM::mma(MM::load(pa2 + kk * KB), MM::load(pb2 + kk * KB), a);
                }
                float yv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int pp = (pw0 + c) * 16 + kq * 4 + e;
                    float o = fmaf(Dh, MM::dec(sX[pp][t]), a[e]);
                    if (has_z) o *= silu(QD::get(rz[c], e));
                    yv[e] = o;
                }
                QD::store(yv, rY, tvalid ? t0 * rowX + oZ[c] : kOffNone);
            }
        }
    }

    if (p.last) {
#pragma unroll
        for (int r = 0; r < NST; ++r) {
            const int q = w + kWaves * r;
            if (q < NSTILE) {
                const int ni = q / NPT, pi = q % NPT;
                float *dst = p.last + (((b * H + h) * P + p0 + pi * 16 + l16) * N + ni * 16 + kq * 4);
                *reinterpret_cast<f32x4_t *>(dst) = acc_s[r];
            }
        }
    }
}

template <typename T, int N, int PT, bool WIDE>
hipError_t launch(const SsdParams &p, int64_t blocks, hipStream_t s) {
    hipLaunchKernelGGL((ssd_chunk_kernel<T, N, PT, WIDE>), dim3(static_cast<unsigned>(blocks)),
                       dim3(64 * waves_for<PT, WIDE>()), 0, s, p);
    return hipGetLastError();
}

// 32-channel tiles when the head size allows; the wide form when the grid
// leaves every CU at most one workgroup
template <typename T, int N>
hipError_t launch_pt(const SsdParams &p, int64_t batch, hipStream_t s) {
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 0;
    if (p.headdim % 32 == 0) {
        const int64_t blocks = batch * p.nheads * (p.headdim / 32);
        return blocks <= cus ? launch<T, N, 32, true>(p, blocks, s) : launch<T, N, 32, false>(p, blocks, s);
    }
    return launch<T, N, 16, false>(p, batch * p.nheads * (p.headdim / 16), s);
}

}  // namespace

bool ssd_supported(int64_t headdim, int64_t dstate, int bf16) {
    if (headdim < 16 || headdim % 16 != 0) return false;
    if (dstate == 32 || dstate == 64) return true;
    return bf16 && dstate == 128;
}

hipError_t launch_ssd_scan(const SsdArgs &a, hipStream_t s) {
    if (a.batch == 0 || a.nheads == 0) return hipSuccess;
    SsdParams p;
    p.x = a.x; p.dt = a.dt; p.z = a.z; p.B = a.B; p.C = a.C;
    p.dt_bias = a.dt_bias; p.A = a.A; p.D = a.D; p.h0 = a.h0;
    p.y = a.y; p.last = a.last_state;
    p.seqlen = a.seqlen; p.nheads = a.nheads; p.headdim = a.headdim;
    p.softplus = a.softplus;
    if (a.bf16) {
        switch (a.dstate) {
        case 32: return launch_pt<bf16_t, 32>(p, a.batch, s);
        case 64: return launch_pt<bf16_t, 64>(p, a.batch, s);
        case 128: return launch_pt<bf16_t, 128>(p, a.batch, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (a.dstate) {
    case 32: return launch_pt<float, 32>(p, a.batch, s);
    case 64: return launch_pt<float, 64>(p, a.batch, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
