// HIP (gfx950) implementation of the COAT FP8-optimizer-state AdamW step.
//
// Method: "COAT: FP8 training, 40% less memory, 1.4x faster"
// (blob.wenxiaobai.com), sections "FP8 optimizer states" and "Solution:
// dynamic range expansion": Adam's two moments are stored per group of G
// elements in FP8, each group with its own scale and its own expansion
// exponent k, chosen on the fly every step so that the expanded group fills
// the FP8 range. FP8 layouts: FP8 guide (maplevalley.com.cn), section
// "format choice"; OCP E4M3FN and E5M2 semantics.
//
// Design (MI355X / CDNA4):
//   * one wavefront owns a tile of 1024 consecutive elements of one tensor;
//     each lane owns 16 consecutive elements, so every stream moves with
//     128-bit loads/stores (fp32 4x16 B, bf16 2x16 B, each FP8 stream 16 B);
//   * a group of G elements spans G/16 lanes of one wave; group statistics
//     are butterfly reductions across those lanes, no LDS round trip;
//   * moments are dequantized, updated and reduced in fp64 (CDNA4 runs fp64
//     FMA at the fp32 rate): the group's k and s are ill-conditioned in its
//     smallest |m'|, usually a near-cancellation of b1*m and (1-b1)*g, so the
//     per-element chain carries 53 bits;
//   * requantization runs in fp32 with the native v_log_f32 / v_exp_f32 and
//     the hardware OCP FP8 converts; an element whose expanded value lies
//     within a relative window of an FP8 rounding midpoint is redone exactly
//     in fp64 with a software encoder, so codes are the exact rounding;
//   * the AdamW update itself (master weights, bf16 copy) runs in fp32;
//   * the multi-tensor kernel walks a descriptor table of a whole parameter
//     list in one launch; tiles never span tensors.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "coat_fp8.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kLaneElems = 16;
constexpr int kTile = kWave * kLaneElems;  // elements per wavefront tile
constexpr int kBlock = 256;                // 4 wavefronts
constexpr int kWavesPerBlock = kBlock / kWave;

// Relative half-width of the window around an FP8 rounding midpoint inside
// which the fp32 fast path defers to the exact fp64 path. The fast path's
// error is a few 1e-6 relative at most (log/exp of arguments up to 32 in
// magnitude); 2^-15 leaves an order of magnitude of margin.
constexpr float kAmbiguity = 0x1p-15f;

// ------------------------------------------------------------------ formats

template <int F>
struct Fmt;

template <>
struct Fmt<COAT_FMT_E4M3> {
    static constexpr int MB = 3;          // mantissa bits
    static constexpr int BIAS = 7;
    static constexpr int EMIN = -6;       // exponent of the smallest normal
    static constexpr int TOP = 0x7E;      // largest finite magnitude code (448)
    static constexpr double FPMAX = 448.0;
    static constexpr float FPMAX_F = 448.0f;
    static constexpr double LOG2_FPMAX = 0x1.19d5d9fd5010bp+3;  // log2(448)
    static constexpr float LOG2_FPMAX_F = 0x1.19d5dap+3f;
    static constexpr double LOG2_RF = 0x1.1ceaecfea8086p+4;     // log2(448 / 2^-9)
    __device__ static bool is_nan(int c) { return c == 0x7F; }
    __device__ static bool is_inf(int) { return false; }
};

template <>
struct Fmt<COAT_FMT_E5M2> {
    static constexpr int MB = 2;
    static constexpr int BIAS = 15;
    static constexpr int EMIN = -14;
    static constexpr int TOP = 0x7B;      // 57344
    static constexpr double FPMAX = 57344.0;
    static constexpr float FPMAX_F = 57344.0f;
    static constexpr double LOG2_FPMAX = 0x1.f9d5d9fd5010bp+3;  // log2(57344)
    static constexpr float LOG2_FPMAX_F = 0x1.f9d5dap+3f;
    static constexpr double LOG2_RF = 0x1.fceaecfea8086p+4;     // log2(57344 / 2^-16)
    __device__ static bool is_nan(int c) { return c > 0x7C; }
    __device__ static bool is_inf(int c) { return c == 0x7C; }
};

// ------------------------------------------------------------------ fp64 math
//
// exp2: u = n + f with n = rint(u), |f| <= 1/2, and 2^f = exp(f ln 2) from its
// Taylor series sum (ln 2)^i f^i / i!. Degree 13 truncates below 2^-57 on
// |f| <= 1/2; the per-element path uses degree 11 (below 2^-47), which keeps
// the dequantized moments far inside what the group statistics need.
// log2: x = m 2^e with m in [sqrt(1/2), sqrt(2)), u = (m-1)/(m+1), and
// ln m = 2 atanh(u) = 2 sum u^(2j+1) / (2j+1); |u| <= 0.1716, so 12 terms
// reach 2^-56. Coefficients are (ln 2)^i / i! and 2 log2(e) / (2j+1) rounded
// to fp64.

__device__ __forceinline__ double exp2_poly11(double f) {
    double p = 0x1.e8cac7351bb25p-32;
    p = __builtin_fma(p, f, 0x1.e4cf5158b8ecap-28);
    p = __builtin_fma(p, f, 0x1.b5253d395e7c4p-24);
    p = __builtin_fma(p, f, 0x1.62c0223a5c824p-20);
    p = __builtin_fma(p, f, 0x1.ffcbfc588b0c7p-17);
    p = __builtin_fma(p, f, 0x1.430912f86c787p-13);
    p = __builtin_fma(p, f, 0x1.5d87fe78a6731p-10);
    p = __builtin_fma(p, f, 0x1.3b2ab6fba4e77p-7);
    p = __builtin_fma(p, f, 0x1.c6b08d704a0c0p-5);
    p = __builtin_fma(p, f, 0x1.ebfbdff82c58fp-3);
    p = __builtin_fma(p, f, 0x1.62e42fefa39efp-1);
    p = __builtin_fma(p, f, 1.0);
    return p;
}

__device__ __forceinline__ double exp2_poly13(double f) {
    double p = 0x1.816193166d0f9p-40;
    p = __builtin_fma(p, f, 0x1.c3bd650fc2986p-36);
    p = __builtin_fma(p, f, 0x1.e8cac7351bb25p-32);
    p = __builtin_fma(p, f, 0x1.e4cf5158b8ecap-28);
    p = __builtin_fma(p, f, 0x1.b5253d395e7c4p-24);
    p = __builtin_fma(p, f, 0x1.62c0223a5c824p-20);
    p = __builtin_fma(p, f, 0x1.ffcbfc588b0c7p-17);
    p = __builtin_fma(p, f, 0x1.430912f86c787p-13);
    p = __builtin_fma(p, f, 0x1.5d87fe78a6731p-10);
    p = __builtin_fma(p, f, 0x1.3b2ab6fba4e77p-7);
    p = __builtin_fma(p, f, 0x1.c6b08d704a0c0p-5);
    p = __builtin_fma(p, f, 0x1.ebfbdff82c58fp-3);
    p = __builtin_fma(p, f, 0x1.62e42fefa39efp-1);
    p = __builtin_fma(p, f, 1.0);
    return p;
}

// v_cvt_i32_f64 clamps out-of-range values to INT_MIN / INT_MAX and maps NaN
// to 0; spelled out so that the compiler cannot treat overflow as undefined.
__device__ __forceinline__ int cvt_i32_sat(double x) {
    int r;
    asm volatile("v_cvt_i32_f64 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// 2^u for any u (NaN -> NaN, huge -> 0 / Inf).
__device__ __forceinline__ double exp2_full(double u) {
    double n = __builtin_rint(u);
    double f = u - n;
    return __builtin_amdgcn_ldexp(exp2_poly13(f), cvt_i32_sat(n));
}

// log2(x) for finite x > 0 (normal or subnormal).
__device__ __forceinline__ double log2_full(double x) {
    int e = __builtin_amdgcn_frexp_exp(x);
    double m = __builtin_amdgcn_frexp_mant(x);  // [0.5, 1)
    if (m < 0x1.6a09e667f3bcdp-1) {             // sqrt(1/2)
        m = m * 2.0;
        e -= 1;
    }
    double u = (m - 1.0) / (m + 1.0);
    double w = u * u;
    double p = 0x1.00ecd7e080215p-3;
    p = __builtin_fma(p, w, 0x1.1964ec6fc9491p-3);
    p = __builtin_fma(p, w, 0x1.3703c1f4d0ffep-3);
    p = __builtin_fma(p, w, 0x1.5b9ac9b743f0dp-3);
    p = __builtin_fma(p, w, 0x1.89f3b1694cffep-3);
    p = __builtin_fma(p, w, 0x1.c68f568d31760p-3);
    p = __builtin_fma(p, w, 0x1.0c9a84994022dp-2);
    p = __builtin_fma(p, w, 0x1.484b13d7c02a9p-2);
    p = __builtin_fma(p, w, 0x1.a61762a7aded9p-2);
    p = __builtin_fma(p, w, 0x1.2776c50ef9bfep-1);
    p = __builtin_fma(p, w, 0x1.ec709dc3a03fdp-1);
    p = __builtin_fma(p, w, 0x1.71547652b82fep+1);
    return __builtin_fma(u, p, (double)e);
}

__device__ __forceinline__ float next_up(float x) {  // x >= 0 finite
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) + 1u);
}
__device__ __forceinline__ float next_down(float x) {  // x > 0 finite
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) - 1u);
}

// ------------------------------------------------------------------ FP8 codec

// Magnitude code of y >= 0 (not NaN): nearest FP8 value, ties to even,
// saturating at the largest finite value. Exact for every fp64 input.
template <int F>
__device__ uint32_t encode_mag_exact(double y) {
    using T = Fmt<F>;
    if (!(y < T::FPMAX)) return T::TOP;
    if (y == 0.0) return 0;
    int e = __builtin_amdgcn_frexp_exp(y) - 1;  // y in [2^e, 2^(e+1))
    int ee = e > T::EMIN ? e : T::EMIN;
    double nq = __builtin_rint(__builtin_amdgcn_ldexp(y, T::MB - ee));  // quanta of 2^(ee-MB)
    int code = ((ee + T::BIAS - 1) << T::MB) + (int)nq;
    return (uint32_t)(code < T::TOP ? code : T::TOP);
}

// Two fp32 values -> two FP8 codes in the low (HI = false) or high half of `old`.
template <int F, bool HI>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b, uint32_t old) {
    if constexpr (F == COAT_FMT_E4M3)
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
    else
        return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

// Exact value of an FP8 code.
template <int F>
__device__ float decode_value(uint32_t code) {
    using T = Fmt<F>;
    int c = code & 0x7F;
    float mag;
    if (T::is_nan(c)) {
        mag = __builtin_nanf("");
    } else if (T::is_inf(c)) {
        mag = __builtin_inff();
    } else {
        int e = c >> T::MB, m = c & ((1 << T::MB) - 1);
        mag = e ? __builtin_amdgcn_ldexpf(1.0f + (float)m / (float)(1 << T::MB), e - T::BIAS)
                : __builtin_amdgcn_ldexpf((float)m, T::EMIN - T::MB);
    }
    return (code & 0x80) ? -mag : mag;
}

// log2(value(c) / fpmax) for magnitude code c, the per-code constant of the
// dequantization x = A 2^(LQ[c] / k). Zero maps to -1e300 and Inf to +1e300
// so that the same arithmetic yields 0 and Inf; NaN codes map to NaN.
template <int F>
__device__ double lq_entry(int c) {
    using T = Fmt<F>;
    if (T::is_nan(c)) return __builtin_nan("");
    if (T::is_inf(c)) return 1e300;
    if (c == 0) return -1e300;
    int e = c >> T::MB, m = c & ((1 << T::MB) - 1);
    double ip, fl;
    if (e == 0) {  // subnormal: m * 2^(EMIN - MB)
        ip = (double)(T::EMIN - T::MB);
        fl = log2_full((double)m);
    } else {       // 2^(e - BIAS) (1 + m / 2^MB)
        ip = (double)(e - T::BIAS);
        fl = log2_full(1.0 + (double)m / (double)(1 << T::MB));
    }
    return (ip - T::LOG2_FPMAX) + fl;
}

// ------------------------------------------------------------------ group state

// Dequantization constants of a stored group: x = A 2^(LQ[q] r) with
// A = (s fpmax)^(1/k) (the group's previous amax) and r = 1/k.
struct OldGroup {
    double A;
    double r;
};

template <int F>
__device__ OldGroup old_group(double s, float k) {
    using T = Fmt<F>;
    OldGroup g;
    g.r = 1.0 / (double)k;
    if (s > 0.0 && s < __builtin_inf()) {
        g.A = exp2_full((log2_full(s) + T::LOG2_FPMAX) * g.r);
    } else {
        g.A = (s == 0.0) ? 0.0 : (s > 0.0 ? s : __builtin_nan(""));  // 0, Inf, NaN propagate
    }
    return g;
}

// Requantization constants of a group from its statistics.
struct NewGroup {
    double s;      // stored scale
    float k;       // stored exponent
    float ia;      // 1 / amax in fp32 (0 for an all-zero group)
    double amax;   // for the exact path
    bool poison;   // non-finite member: every code 0x7F
    bool fast_ok;  // fp32 fast path is valid for every member
};

// k = ln R_fp8 / ln(amax / amin) (= log2 R_fp8 / log2 R), k = 1 for an
// all-zero or near-constant group or without expansion; then the range guard:
// amax^k and amax^k / R_fp8 within [2^-1022, 2^1023].
template <int F>
__device__ NewGroup new_group(double amax, double amin, bool poison, bool expand) {
    using T = Fmt<F>;
    NewGroup g;
    g.poison = poison;
    g.amax = amax;
    g.fast_ok = true;
    if (poison) {
        g.s = __builtin_nan("");
        g.k = 1.0f;
        g.ia = 0.0f;
        return g;
    }
    if (amax == 0.0) {
        g.s = 0.0;
        g.k = 1.0f;
        g.ia = 0.0f;
        return g;
    }
    double L = log2_full(amax);
    float k = 1.0f;
    double R = amax / amin;
    if (expand && R > 1.000001) k = (float)(T::LOG2_RF / log2_full(R));
    double lo = -1022.0 + T::LOG2_RF, hi = 1023.0;
    double kL = (double)k * L;
    if (!(kL >= lo && kL <= hi)) {
        double bound = (L < 0.0) ? lo / L : hi / L;
        float kk = (float)bound;
        if (kk > k) kk = k;
        while (kk > 0.0f && !((double)kk * L >= lo && (double)kk * L <= hi)) kk = next_down(kk);
        while (next_up(kk) <= k && (double)next_up(kk) * L >= lo && (double)next_up(kk) * L <= hi)
            kk = next_up(kk);
        k = kk;
    }
    g.k = k;
    g.s = exp2_full((double)k * L - T::LOG2_FPMAX);
    g.ia = (float)(1.0 / amax);
    // The fp32 path needs every member and 1/amax normal in fp32 and t = |x|/amax
    // at least 2^-100 for nonzero members.
    g.fast_ok = amax <= 0x1p126 && amin >= 0x1p-126 && R <= 0x1p100;
    return g;
}

// Exact code of one element: fpmax (|x| / amax)^k rounded in fp64.
template <int F>
__device__ uint32_t exact_code(double x, const NewGroup& g) {
    using T = Fmt<F>;
    uint32_t sign = __builtin_signbit(x) ? 0x80u : 0u;
    if (g.poison) return 0x7F;
    double t = __builtin_fabs(x) / g.amax;
    if (!(t > 0.0)) return sign;  // zero member or all-zero group
    double y = exp2_full((double)g.k * log2_full(t) + T::LOG2_FPMAX);
    return sign | encode_mag_exact<F>(y);
}

// Fast requantization of 4 elements (fp32 copies xf) into one code word;
// returns the word and sets `amb` to 0x80 in each byte whose code is within the
// ambiguity window of a rounding midpoint.
template <int F>
__device__ __forceinline__ uint32_t fast_codes4(const float* xf, const NewGroup& g, uint32_t& amb) {
    using T = Fmt<F>;
    float lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float t = __builtin_fabsf(xf[i]) * g.ia;
        float l = __builtin_amdgcn_logf(t);
        float z = __builtin_fmaf(g.k, l, T::LOG2_FPMAX_F);
        float y = __builtin_amdgcn_exp2f(z);
        lo[i] = __builtin_copysignf(y * (1.0f - kAmbiguity), xf[i]);
        hi[i] = __builtin_fminf(y * (1.0f + kAmbiguity), T::FPMAX_F);
    }
    uint32_t wl = cvt_pk<F, false>(lo[0], lo[1], 0u);
    wl = cvt_pk<F, true>(lo[2], lo[3], wl);
    uint32_t wh = cvt_pk<F, false>(hi[0], hi[1], 0u);
    wh = cvt_pk<F, true>(hi[2], hi[3], wh);
    uint32_t d = (wl ^ wh) & 0x7F7F7F7Fu;
    amb = (d + 0x7F7F7F7Fu) & 0x80808080u;
    return wl;
}

// ------------------------------------------------------------------ step

struct StepConsts {
    double b1, c1, b2, c2;  // moment coefficients (c = 1 - b), fp64
    float decay;            // 1 - lr wd
    float ssz;              // lr / (1 - b1^t)
    float ib2;              // 1 / sqrt(1 - b2^t)
    float eps;
    int lg2_group;
    int expand_m, expand_v;
};

struct TensorRef {
    float* p;
    uint16_t* w;
    const uint16_t* g;
    uint8_t* mq;
    double* ms;
    float* mk;
    uint8_t* vq;
    double* vs;
    float* vk;
    int64_t n;
};
static_assert(sizeof(TensorRef) == sizeof(coat_tensor), "descriptor layout");

__device__ __forceinline__ double dequant(uint32_t code, const OldGroup& og, const double* lq) {
    double u = lq[code & 0x7F] * og.r;
    double n = __builtin_rint(u);
    double p = exp2_poly11(u - n);
    double x = __builtin_amdgcn_ldexp(p * og.A, cvt_i32_sat(n));
    return (code & 0x80) ? -x : x;
}

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xFFu; }

// Lane-group all-reduce over the G/16 lanes owning one group (butterfly).
__device__ __forceinline__ double group_max(double v, int lanes) {
    for (int d = 1; d < lanes; d <<= 1) v = __builtin_fmax(v, __shfl_xor(v, d, kWave));
    return v;
}
__device__ __forceinline__ double group_min(double v, int lanes) {
    for (int d = 1; d < lanes; d <<= 1) v = __builtin_fmin(v, __shfl_xor(v, d, kWave));
    return v;
}
__device__ __forceinline__ int group_or(int v, int lanes) {
    for (int d = 1; d < lanes; d <<= 1) v |= __shfl_xor(v, d, kWave);
    return v;
}

__device__ __forceinline__ uint32_t select4(int i, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
    return i == 0 ? a0 : (i == 1 ? a1 : (i == 2 ? a2 : a3));
}

// One wavefront tile of the step: elements [tile*1024, tile*1024 + 1024) of t.
template <int FM, int FV>
__device__ void step_tile(const TensorRef& t, int64_t tile, const StepConsts& c,
                          const double* lq_m, const double* lq_v) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
    const int64_t rem = t.n - e0;
    const int nvalid = rem <= 0 ? 0 : (rem >= kLaneElems ? kLaneElems : (int)rem);
    const int lanes_per_group = 1 << (c.lg2_group - 4);
    const int64_t gidx = e0 >> c.lg2_group;

    // ---- loads (zeros past the end contribute nothing to the group statistics)
    float p[16];
    uint32_t gw[8], mq[4], vq[4];
    if (nvalid == kLaneElems) {
        const f32x4* pp = reinterpret_cast<const f32x4*>(t.p + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 v = __builtin_nontemporal_load(pp + i);
            p[4 * i] = v.x; p[4 * i + 1] = v.y; p[4 * i + 2] = v.z; p[4 * i + 3] = v.w;
        }
        const u32x4* gp = reinterpret_cast<const u32x4*>(t.g + e0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            u32x4 v = __builtin_nontemporal_load(gp + i);
            gw[4 * i] = v.x; gw[4 * i + 1] = v.y; gw[4 * i + 2] = v.z; gw[4 * i + 3] = v.w;
        }
        u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t.mq + e0));
        mq[0] = a.x; mq[1] = a.y; mq[2] = a.z; mq[3] = a.w;
        u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t.vq + e0));
        vq[0] = b.x; vq[1] = b.y; vq[2] = b.z; vq[3] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) gw[i] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) { mq[i] = 0u; vq[i] = 0u; }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bool in = i < nvalid;
            p[i] = in ? t.p[e0 + i] : 0.0f;
            gw[i >> 1] |= in ? (uint32_t)t.g[e0 + i] << (16 * (i & 1)) : 0u;
            mq[i >> 2] |= in ? (uint32_t)t.mq[e0 + i] << (8 * (i & 3)) : 0u;
            vq[i >> 2] |= in ? (uint32_t)t.vq[e0 + i] << (8 * (i & 3)) : 0u;
        }
    }

    // ---- stored group state
    double sm = 0.0, sv = 0.0;
    float km = 1.0f, kv = 1.0f;
    if (nvalid > 0) {
        sm = t.ms[gidx]; km = t.mk[gidx];
        sv = t.vs[gidx]; kv = t.vk[gidx];
    }
    const OldGroup om = old_group<FM>(sm, km);
    const OldGroup ov = old_group<FV>(sv, kv);

    // ---- per element: dequantize, moments, statistics, AdamW update
    float xm[16], xv[16];
    double amax_m = 0.0, amin_m = __builtin_inf(), amax_v = 0.0, amin_v = __builtin_inf();
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const double m0 = dequant(byte_of(mq[i >> 2], i & 3), om, lq_m);
        const double v0 = dequant(byte_of(vq[i >> 2], i & 3), ov, lq_v);
        const double g = (double)__builtin_bit_cast(float, ((gw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) << 16);
        const double m1 = __builtin_fma(c.b1, m0, c.c1 * g);
        const double v1 = __builtin_fma(c.b2, v0, c.c2 * (g * g));
        const double am = __builtin_fabs(m1), av = __builtin_fabs(v1);
        bad |= !(am < __builtin_inf()) | !(av < __builtin_inf());
        amax_m = __builtin_fmax(amax_m, am);
        amin_m = __builtin_fmin(amin_m, am == 0.0 ? __builtin_inf() : am);
        amax_v = __builtin_fmax(amax_v, av);
        amin_v = __builtin_fmin(amin_v, av == 0.0 ? __builtin_inf() : av);
        xm[i] = (float)m1;
        xv[i] = (float)v1;
        const float den = __builtin_fmaf(__builtin_amdgcn_sqrtf(xv[i]), c.ib2, c.eps);
        const float upd = xm[i] * __builtin_amdgcn_rcpf(den);
        p[i] = __builtin_fmaf(-c.ssz, upd, p[i] * c.decay);
    }

    // ---- store the new master weights and the bf16 copy
    if (nvalid == kLaneElems) {
        f32x4* pp = reinterpret_cast<f32x4*>(t.p + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_nontemporal_store(f32x4{p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]}, pp + i);
        if (t.w) {
            uint32_t wb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __bf16 lo = (__bf16)p[2 * i], hi = (__bf16)p[2 * i + 1];
                wb[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            u32x4* wp = reinterpret_cast<u32x4*>(t.w + e0);
            __builtin_nontemporal_store(u32x4{wb[0], wb[1], wb[2], wb[3]}, wp);
            __builtin_nontemporal_store(u32x4{wb[4], wb[5], wb[6], wb[7]}, wp + 1);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < nvalid) {
                t.p[e0 + i] = p[i];
                if (t.w) t.w[e0 + i] = __builtin_bit_cast(uint16_t, (__bf16)p[i]);
            }
        }
    }

    // ---- group statistics across the group's lanes
    amax_m = group_max(amax_m, lanes_per_group);
    amin_m = group_min(amin_m, lanes_per_group);
    amax_v = group_max(amax_v, lanes_per_group);
    amin_v = group_min(amin_v, lanes_per_group);
    const bool poison = group_or(bad ? 1 : 0, lanes_per_group) != 0;
    // A non-finite grad poisons both moments' groups (m' and v' both become non-finite).
    const NewGroup nm = new_group<FM>(amax_m, amin_m, poison, c.expand_m);
    const NewGroup nv = new_group<FV>(amax_v, amin_v, poison, c.expand_v);

    // ---- requantize: fast fp32 codes, exact redo of ambiguous elements
    uint32_t cm[4], cv[4], am[4], av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        cm[i] = fast_codes4<FM>(xm + 4 * i, nm, am[i]);
        cv[i] = fast_codes4<FV>(xv + 4 * i, nv, av[i]);
    }
    if (!nm.fast_ok) { am[0] = am[1] = am[2] = am[3] = 0x80808080u; }
    if (!nv.fast_ok) { av[0] = av[1] = av[2] = av[3] = 0x80808080u; }
    if (nvalid < kLaneElems) {  // never redo elements past the end
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t keep = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) keep |= (4 * i + b < nvalid) ? (0x80u << (8 * b)) : 0u;
            am[i] &= keep;
            av[i] &= keep;
        }
    }
    if (nm.poison) { am[0] = am[1] = am[2] = am[3] = 0u; }
    if (nv.poison) { av[0] = av[1] = av[2] = av[3] = 0u; }
    // Pack the 32 flags of this lane (bit 4*i+b: m element 4i+b; bit 16+...: v).
    uint32_t pend = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            pend |= ((am[i] >> (8 * b + 7)) & 1u) << (4 * i + b);
            pend |= ((av[i] >> (8 * b + 7)) & 1u) << (16 + 4 * i + b);
        }
    }
    while (__any(pend != 0u)) {
        if (pend != 0u) {
            const int j = __builtin_ctz(pend);
            pend &= pend - 1u;
            const bool is_v = j >= 16;
            const int e = j & 15, wi = e >> 2, bi = e & 3;
            // Recompute this element's new moment exactly as above.
            const uint32_t codeword = is_v ? select4(wi, vq[0], vq[1], vq[2], vq[3])
                                           : select4(wi, mq[0], mq[1], mq[2], mq[3]);
            const uint32_t gword = (e >> 1) < 4 ? select4(e >> 1, gw[0], gw[1], gw[2], gw[3])
                                                : select4((e >> 1) - 4, gw[4], gw[5], gw[6], gw[7]);
            const double g = (double)__builtin_bit_cast(float, ((gword >> (16 * (e & 1))) & 0xFFFFu) << 16);
            uint32_t code;
            if (is_v) {
                const double v1 = __builtin_fma(c.b2, dequant(byte_of(codeword, bi), ov, lq_v), c.c2 * (g * g));
                code = exact_code<FV>(v1, nv);
            } else {
                const double m1 = __builtin_fma(c.b1, dequant(byte_of(codeword, bi), om, lq_m), c.c1 * g);
                code = exact_code<FM>(m1, nm);
            }
            const uint32_t mask = ~(0xFFu << (8 * bi));
            const uint32_t ins = code << (8 * bi);
            if (is_v) {
                if (wi == 0) cv[0] = (cv[0] & mask) | ins;
                if (wi == 1) cv[1] = (cv[1] & mask) | ins;
                if (wi == 2) cv[2] = (cv[2] & mask) | ins;
                if (wi == 3) cv[3] = (cv[3] & mask) | ins;
            } else {
                if (wi == 0) cm[0] = (cm[0] & mask) | ins;
                if (wi == 1) cm[1] = (cm[1] & mask) | ins;
                if (wi == 2) cm[2] = (cm[2] & mask) | ins;
                if (wi == 3) cm[3] = (cm[3] & mask) | ins;
            }
        }
    }
    if (nm.poison) { cm[0] = cm[1] = cm[2] = cm[3] = 0x7F7F7F7Fu; }
    if (nv.poison) { cv[0] = cv[1] = cv[2] = cv[3] = 0x7F7F7F7Fu; }

    // ---- store codes and group state
    if (nvalid == kLaneElems) {
        __builtin_nontemporal_store(u32x4{cm[0], cm[1], cm[2], cm[3]}, reinterpret_cast<u32x4*>(t.mq + e0));
        __builtin_nontemporal_store(u32x4{cv[0], cv[1], cv[2], cv[3]}, reinterpret_cast<u32x4*>(t.vq + e0));
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < nvalid) {
                t.mq[e0 + i] = (uint8_t)byte_of(cm[i >> 2], i & 3);
                t.vq[e0 + i] = (uint8_t)byte_of(cv[i >> 2], i & 3);
            }
        }
    }
    if (nvalid > 0 && (lane & (lanes_per_group - 1)) == 0) {
        t.ms[gidx] = nm.s; t.mk[gidx] = nm.k;
        t.vs[gidx] = nv.s; t.vk[gidx] = nv.k;
    }
}

template <int FM, int FV>
__device__ __forceinline__ void fill_lq_tables(double* lq_m, double* lq_v) {
    const int i = threadIdx.x;
    if (i < 128) lq_m[i] = lq_entry<FM>(i);
    else if (i < 256) lq_v[i - 128] = lq_entry<FV>(i - 128);
    __syncthreads();
}

__device__ __forceinline__ int64_t wave_id() {
    return (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

template <int FM, int FV>
__global__ __launch_bounds__(kBlock) void step_single_kernel(TensorRef t, StepConsts c) {
    __shared__ double lq[2][128];
    fill_lq_tables<FM, FV>(lq[0], lq[1]);
    const int64_t tiles = (t.n + kTile - 1) / kTile;
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t tile = wave_id(); tile < tiles; tile += nw) step_tile<FM, FV>(t, tile, c, lq[0], lq[1]);
}

// Multi-tensor: descriptors and the tile prefix (count + 1 entries) live in
// device workspace; each wavefront strides over the global tile index space
// and walks the prefix forward to find the tensor of its tile.
template <int FM, int FV>
__global__ __launch_bounds__(kBlock) void step_multi_kernel(const TensorRef* __restrict__ ts,
                                                            const int64_t* __restrict__ tile_begin,
                                                            int count, StepConsts c) {
    __shared__ double lq[2][128];
    fill_lq_tables<FM, FV>(lq[0], lq[1]);
    const int64_t tiles = tile_begin[count];
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    int cur = 0;
    for (int64_t tile = wave_id(); tile < tiles; tile += nw) {
        while (tile >= tile_begin[cur + 1]) ++cur;
        step_tile<FM, FV>(ts[cur], tile - tile_begin[cur], c, lq[0], lq[1]);
    }
}

// ------------------------------------------------------------------ codec kernels

// Quantize fp32 x to (q, s, k): the requantization half of the step.
template <int F>
__global__ __launch_bounds__(kBlock) void quantize_kernel(const float* __restrict__ x, int64_t n,
                                                          int lg2_group, int expand, uint8_t* q,
                                                          double* s, float* k) {
    const int64_t tiles = (n + kTile - 1) / kTile;
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int lane = threadIdx.x & (kWave - 1);
    const int lanes_per_group = 1 << (lg2_group - 4);
    for (int64_t tile = wave_id(); tile < tiles; tile += nw) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
        const int64_t rem = n - e0;
        const int nvalid = rem <= 0 ? 0 : (rem >= kLaneElems ? kLaneElems : (int)rem);
        float xf[16];
        if (nvalid == kLaneElems) {
            const f32x4* xp = reinterpret_cast<const f32x4*>(x + e0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 v = __builtin_nontemporal_load(xp + i);
                xf[4 * i] = v.x; xf[4 * i + 1] = v.y; xf[4 * i + 2] = v.z; xf[4 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) xf[i] = i < nvalid ? x[e0 + i] : 0.0f;
        }
        double amax = 0.0, amin = __builtin_inf();
        bool bad = false;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const double a = __builtin_fabs((double)xf[i]);
            bad |= !(a < __builtin_inf());
            amax = __builtin_fmax(amax, a);
            amin = __builtin_fmin(amin, a == 0.0 ? __builtin_inf() : a);
        }
        amax = group_max(amax, lanes_per_group);
        amin = group_min(amin, lanes_per_group);
        const bool poison = group_or(bad ? 1 : 0, lanes_per_group) != 0;
        const NewGroup ng = new_group<F>(amax, amin, poison, expand);
        uint32_t cw[4], amb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cw[i] = fast_codes4<F>(xf + 4 * i, ng, amb[i]);
        uint32_t pend = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) pend |= ((amb[i] >> (8 * b + 7)) & 1u) << (4 * i + b);
        if (!ng.fast_ok) pend = 0xFFFFu;
        if (nvalid < kLaneElems) pend &= (1u << nvalid) - 1u;
        if (ng.poison) pend = 0;
        while (__any(pend != 0u)) {
            if (pend != 0u) {
                const int e = __builtin_ctz(pend);
                pend &= pend - 1u;
                float xe = xf[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) xe = (e == i) ? xf[i] : xe;
                const uint32_t code = exact_code<F>((double)xe, ng);
                const int wi = e >> 2, bi = e & 3;
                const uint32_t mask = ~(0xFFu << (8 * bi)), ins = code << (8 * bi);
                if (wi == 0) cw[0] = (cw[0] & mask) | ins;
                if (wi == 1) cw[1] = (cw[1] & mask) | ins;
                if (wi == 2) cw[2] = (cw[2] & mask) | ins;
                if (wi == 3) cw[3] = (cw[3] & mask) | ins;
            }
        }
        if (ng.poison) { cw[0] = cw[1] = cw[2] = cw[3] = 0x7F7F7F7Fu; }
        if (nvalid == kLaneElems) {
            __builtin_nontemporal_store(u32x4{cw[0], cw[1], cw[2], cw[3]}, reinterpret_cast<u32x4*>(q + e0));
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i < nvalid) q[e0 + i] = (uint8_t)byte_of(cw[i >> 2], i & 3);
        }
        if (nvalid > 0 && (lane & (lanes_per_group - 1)) == 0) {
            const int64_t gi = e0 >> lg2_group;
            s[gi] = ng.s;
            k[gi] = ng.k;
        }
    }
}

template <int F>
__global__ __launch_bounds__(kBlock) void dequantize_kernel(const uint8_t* __restrict__ q,
                                                            const double* __restrict__ s,
                                                            const float* __restrict__ k, int64_t n,
                                                            int lg2_group, float* __restrict__ x) {
    __shared__ double lq[128];
    if (threadIdx.x < 128) lq[threadIdx.x] = lq_entry<F>(threadIdx.x);
    __syncthreads();
    const int64_t tiles = (n + kTile - 1) / kTile;
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int lane = threadIdx.x & (kWave - 1);
    for (int64_t tile = wave_id(); tile < tiles; tile += nw) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
        const int64_t rem = n - e0;
        const int nvalid = rem <= 0 ? 0 : (rem >= kLaneElems ? kLaneElems : (int)rem);
        if (nvalid == 0) continue;
        const int64_t gi = e0 >> lg2_group;
        const OldGroup og = old_group<F>(s[gi], k[gi]);
        if (nvalid == kLaneElems) {
            u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + e0));
            const uint32_t w[4] = {a.x, a.y, a.z, a.w};
            float out[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) out[i] = (float)dequant(byte_of(w[i >> 2], i & 3), og, lq);
            f32x4* xp = reinterpret_cast<f32x4*>(x + e0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_nontemporal_store(f32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]}, xp + i);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i < nvalid) x[e0 + i] = (float)dequant(q[e0 + i], og, lq);
        }
    }
}

template <int F>
__global__ __launch_bounds__(kBlock) void encode_kernel(const float* __restrict__ y, int64_t n,
                                                        uint8_t* __restrict__ q) {
    using T = Fmt<F>;
    const int64_t nw = (int64_t)gridDim.x * kBlock;
    for (int64_t i4 = (int64_t)blockIdx.x * kBlock + threadIdx.x; 4 * i4 < n; i4 += nw) {
        const int64_t e0 = 4 * i4;
        float v[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) v[b] = (e0 + b < n) ? y[e0 + b] : 0.0f;
        float lo[4], hi[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float a = __builtin_fabsf(v[b]);
            lo[b] = __builtin_copysignf(__builtin_fminf(a * (1.0f - kAmbiguity), T::FPMAX_F), v[b]);
            hi[b] = __builtin_fminf(a * (1.0f + kAmbiguity), T::FPMAX_F);
        }
        uint32_t wl = cvt_pk<F, false>(lo[0], lo[1], 0u);
        wl = cvt_pk<F, true>(lo[2], lo[3], wl);
        uint32_t wh = cvt_pk<F, false>(hi[0], hi[1], 0u);
        wh = cvt_pk<F, true>(hi[2], hi[3], wh);
        uint32_t d = (wl ^ wh) & 0x7F7F7F7Fu;
        d = (d + 0x7F7F7F7Fu) & 0x80808080u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            uint32_t code = byte_of(wl, b);
            const bool nan = v[b] != v[b];
            if (nan) code = 0x7F;
            else if ((d >> (8 * b + 7)) & 1u)
                code = (__builtin_signbit(v[b]) ? 0x80u : 0u) | encode_mag_exact<F>(__builtin_fabs((double)v[b]));
            if (e0 + b < n) q[e0 + b] = (uint8_t)code;
        }
    }
}

template <int F>
__global__ __launch_bounds__(kBlock) void decode_kernel(const uint8_t* __restrict__ q, int64_t n,
                                                        float* __restrict__ y) {
    const int64_t nw = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += nw) y[i] = decode_value<F>(q[i]);
}

// ------------------------------------------------------------------ host side

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int lg2_group_of(int32_t group) {
    if (group < 16 || group > 1024 || (group & (group - 1)) != 0) return -1;
    int l = 0;
    while ((1 << l) < group) ++l;
    return l;
}

bool fmt_ok(int32_t fmt) {
    const int base = fmt & 0xFF;
    return (base == COAT_FMT_E4M3 || base == COAT_FMT_E5M2) && (fmt & ~(0xFF | COAT_FMT_NO_EXPAND)) == 0;
}

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

// Blocks for a grid-stride launch over `waves` wavefront tiles: enough to fill
// every CU `per_cu` times, never more than there is work.
unsigned grid_for(int64_t waves, int per_cu) {
    const int64_t want = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t cap = (int64_t)device_cus() * per_cu;
    int64_t b = want < cap ? want : cap;
    return (unsigned)(b < 1 ? 1 : b);
}

constexpr int kStepBlocksPerCU = 8;

bool finite_f(float x) { return x == x && x - x == 0.0f; }

int make_consts(int32_t group, int32_t fmt_m, int32_t fmt_v, float lr, float b1, float b2, float eps,
                float wd, int64_t step, StepConsts* c) {
    const int lg = lg2_group_of(group);
    if (lg < 0 || !fmt_ok(fmt_m) || !fmt_ok(fmt_v) || step < 1) return COAT_EINVAL;
    if (!finite_f(lr) || !finite_f(b1) || !finite_f(b2) || !finite_f(eps) || !finite_f(wd)) return COAT_EINVAL;
    const double t = (double)step;
    const double bc1 = 1.0 - pow((double)b1, t);
    const double bc2 = 1.0 - pow((double)b2, t);
    if (!(bc1 != 0.0) || !(bc2 > 0.0)) return COAT_EINVAL;
    c->b1 = (double)b1;
    c->c1 = 1.0 - (double)b1;
    c->b2 = (double)b2;
    c->c2 = 1.0 - (double)b2;
    c->decay = (float)(1.0 - (double)lr * (double)wd);
    c->ssz = (float)((double)lr / bc1);
    c->ib2 = (float)(1.0 / sqrt(bc2));
    c->eps = eps;
    c->lg2_group = lg;
    c->expand_m = (fmt_m & COAT_FMT_NO_EXPAND) ? 0 : 1;
    c->expand_v = (fmt_v & COAT_FMT_NO_EXPAND) ? 0 : 1;
    return COAT_OK;
}

int check_tensor(const TensorRef& t) {
    if (t.n < 0) return COAT_EINVAL;
    if (t.n == 0) return COAT_OK;
    if (!t.p || !t.g || !t.mq || !t.ms || !t.mk || !t.vq || !t.vs || !t.vk) return COAT_EINVAL;
    if (!aligned16(t.p) || !aligned16(t.g) || !aligned16(t.mq) || !aligned16(t.vq) ||
        (t.w && !aligned16(t.w)) || !aligned(t.ms, 8) || !aligned(t.vs, 8) || !aligned(t.mk, 4) ||
        !aligned(t.vk, 4))
        return COAT_EALIGN;
    return COAT_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? COAT_OK : COAT_EHIP; }

template <int FM, int FV>
void launch_single(const TensorRef& t, const StepConsts& c, hipStream_t st) {
    const int64_t tiles = (t.n + kTile - 1) / kTile;
    hipLaunchKernelGGL((step_single_kernel<FM, FV>), dim3(grid_for(tiles, kStepBlocksPerCU)), dim3(kBlock),
                       0, st, t, c);
}

template <int FM, int FV>
void launch_multi(const TensorRef* ts, const int64_t* tb, int count, int64_t tiles, const StepConsts& c,
                  hipStream_t st) {
    hipLaunchKernelGGL((step_multi_kernel<FM, FV>), dim3(grid_for(tiles, kStepBlocksPerCU)), dim3(kBlock),
                       0, st, ts, tb, count, c);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

// ====================================================================== C ABI

extern "C" {

int coat_abi_version(void) { return 100; }

const char* coat_strerror(int status) {
    switch (status) {
        case COAT_OK: return "ok";
        case COAT_EINVAL: return "invalid argument";
        case COAT_EALIGN: return "pointer not aligned as required (16 bytes for element arrays)";
        case COAT_EHIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

int coat_fp8_adamw_step(float* params, uint16_t* params_bf16, const uint16_t* grads, uint8_t* m_q,
                        double* m_s, float* m_k, uint8_t* v_q, double* v_s, float* v_k, int64_t n,
                        int32_t group, int32_t fmt_m, int32_t fmt_v, float lr, float beta1,
                        float beta2, float eps, float weight_decay, int64_t step,
                        coat_stream_t stream) {
    StepConsts c;
    int rc = make_consts(group, fmt_m, fmt_v, lr, beta1, beta2, eps, weight_decay, step, &c);
    if (rc) return rc;
    TensorRef t{params, params_bf16, grads, m_q, m_s, m_k, v_q, v_s, v_k, n};
    rc = check_tensor(t);
    if (rc || n == 0) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int fm = fmt_m & 0xFF, fv = fmt_v & 0xFF;
    if (fm == COAT_FMT_E4M3 && fv == COAT_FMT_E4M3) launch_single<COAT_FMT_E4M3, COAT_FMT_E4M3>(t, c, st);
    else if (fm == COAT_FMT_E4M3) launch_single<COAT_FMT_E4M3, COAT_FMT_E5M2>(t, c, st);
    else if (fv == COAT_FMT_E4M3) launch_single<COAT_FMT_E5M2, COAT_FMT_E4M3>(t, c, st);
    else launch_single<COAT_FMT_E5M2, COAT_FMT_E5M2>(t, c, st);
    return launch_status();
}

size_t coat_multi_workspace_bytes(int32_t count) {
    if (count < 0) return 0;
    return align_up(sizeof(TensorRef) * (size_t)count, 256) + align_up(sizeof(int64_t) * ((size_t)count + 1), 256);
}

int coat_multi_plan_init(coat_multi_plan* plan, const coat_tensor* tensors, int32_t count, void* workspace,
                         size_t workspace_bytes, coat_stream_t stream) {
    if (!plan || count < 0 || (count > 0 && !tensors)) return COAT_EINVAL;
    if (!workspace || workspace_bytes < coat_multi_workspace_bytes(count)) return COAT_EINVAL;
    if (!aligned(workspace, 256)) return COAT_EALIGN;
    const size_t desc_bytes = align_up(sizeof(TensorRef) * (size_t)count, 256);
    const size_t total = desc_bytes + sizeof(int64_t) * ((size_t)count + 1);
    std::vector<char> host(total, 0);
    TensorRef* hd = reinterpret_cast<TensorRef*>(host.data());
    int64_t* tb = reinterpret_cast<int64_t*>(host.data() + desc_bytes);
    int64_t tiles = 0, n_total = 0;
    for (int32_t i = 0; i < count; ++i) {
        memcpy(&hd[i], &tensors[i], sizeof(TensorRef));
        const int rc = check_tensor(hd[i]);
        if (rc) return rc;
        tb[i] = tiles;
        tiles += (hd[i].n + kTile - 1) / kTile;
        n_total += hd[i].n;
    }
    tb[count] = tiles;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(workspace, host.data(), total, hipMemcpyHostToDevice, st) != hipSuccess) return COAT_EHIP;
    if (hipStreamSynchronize(st) != hipSuccess) return COAT_EHIP;
    plan->workspace = workspace;
    plan->count = count;
    plan->tiles = tiles;
    plan->n_total = n_total;
    return COAT_OK;
}

int coat_fp8_adamw_step_planned(const coat_multi_plan* plan, int32_t group, int32_t fmt_m, int32_t fmt_v,
                                float lr, float beta1, float beta2, float eps, float weight_decay,
                                int64_t step, coat_stream_t stream) {
    if (!plan || plan->count < 0 || !plan->workspace) return COAT_EINVAL;
    StepConsts c;
    const int rc = make_consts(group, fmt_m, fmt_v, lr, beta1, beta2, eps, weight_decay, step, &c);
    if (rc) return rc;
    if (plan->count == 0 || plan->tiles == 0) return COAT_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const size_t desc_bytes = align_up(sizeof(TensorRef) * (size_t)plan->count, 256);
    const TensorRef* dts = static_cast<const TensorRef*>(plan->workspace);
    const int64_t* dtb = reinterpret_cast<const int64_t*>(static_cast<const char*>(plan->workspace) + desc_bytes);
    const int fm = fmt_m & 0xFF, fv = fmt_v & 0xFF;
    const int count = plan->count;
    const int64_t tiles = plan->tiles;
    if (fm == COAT_FMT_E4M3 && fv == COAT_FMT_E4M3) launch_multi<COAT_FMT_E4M3, COAT_FMT_E4M3>(dts, dtb, count, tiles, c, st);
    else if (fm == COAT_FMT_E4M3) launch_multi<COAT_FMT_E4M3, COAT_FMT_E5M2>(dts, dtb, count, tiles, c, st);
    else if (fv == COAT_FMT_E4M3) launch_multi<COAT_FMT_E5M2, COAT_FMT_E4M3>(dts, dtb, count, tiles, c, st);
    else launch_multi<COAT_FMT_E5M2, COAT_FMT_E5M2>(dts, dtb, count, tiles, c, st);
    return launch_status();
}

int coat_fp8_adamw_step_multi(const coat_tensor* tensors, int32_t count, int32_t group, int32_t fmt_m,
                              int32_t fmt_v, float lr, float beta1, float beta2, float eps,
                              float weight_decay, int64_t step, void* workspace, size_t workspace_bytes,
                              coat_stream_t stream) {
    StepConsts c;
    int rc = make_consts(group, fmt_m, fmt_v, lr, beta1, beta2, eps, weight_decay, step, &c);
    if (rc) return rc;
    coat_multi_plan plan;
    rc = coat_multi_plan_init(&plan, tensors, count, workspace, workspace_bytes, stream);
    if (rc) return rc;
    return coat_fp8_adamw_step_planned(&plan, group, fmt_m, fmt_v, lr, beta1, beta2, eps, weight_decay, step,
                                       stream);
}

int coat_fp8_quantize(const float* x, int64_t n, int32_t group, int32_t fmt, uint8_t* q, double* s,
                      float* k, coat_stream_t stream) {
    const int lg = lg2_group_of(group);
    if (lg < 0 || !fmt_ok(fmt) || n < 0) return COAT_EINVAL;
    if (n == 0) return COAT_OK;
    if (!x || !q || !s || !k) return COAT_EINVAL;
    if (!aligned16(x) || !aligned16(q) || !aligned(s, 8) || !aligned(k, 4)) return COAT_EALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t tiles = (n + kTile - 1) / kTile;
    const int expand = (fmt & COAT_FMT_NO_EXPAND) ? 0 : 1;
    if ((fmt & 0xFF) == COAT_FMT_E4M3)
        hipLaunchKernelGGL(quantize_kernel<COAT_FMT_E4M3>, dim3(grid_for(tiles, 8)), dim3(kBlock), 0, st, x, n, lg, expand, q, s, k);
    else
        hipLaunchKernelGGL(quantize_kernel<COAT_FMT_E5M2>, dim3(grid_for(tiles, 8)), dim3(kBlock), 0, st, x, n, lg, expand, q, s, k);
    return launch_status();
}

int coat_fp8_dequantize(const uint8_t* q, const double* s, const float* k, int64_t n, int32_t group,
                        int32_t fmt, float* x, coat_stream_t stream) {
    const int lg = lg2_group_of(group);
    if (lg < 0 || !fmt_ok(fmt) || n < 0) return COAT_EINVAL;
    if (n == 0) return COAT_OK;
    if (!x || !q || !s || !k) return COAT_EINVAL;
    if (!aligned16(x) || !aligned16(q) || !aligned(s, 8) || !aligned(k, 4)) return COAT_EALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t tiles = (n + kTile - 1) / kTile;
    if ((fmt & 0xFF) == COAT_FMT_E4M3)
        hipLaunchKernelGGL(dequantize_kernel<COAT_FMT_E4M3>, dim3(grid_for(tiles, 8)), dim3(kBlock), 0, st, q, s, k, n, lg, x);
    else
        hipLaunchKernelGGL(dequantize_kernel<COAT_FMT_E5M2>, dim3(grid_for(tiles, 8)), dim3(kBlock), 0, st, q, s, k, n, lg, x);
    return launch_status();
}

int coat_fp8_encode(const float* y, int64_t n, int32_t fmt, uint8_t* q, coat_stream_t stream) {
    if (n < 0 || (fmt != COAT_FMT_E4M3 && fmt != COAT_FMT_E5M2)) return COAT_EINVAL;
    if (n == 0) return COAT_OK;
    if (!y || !q) return COAT_EINVAL;
    if (!aligned(y, 4)) return COAT_EALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t threads = (n + 3) / 4;
    const unsigned grid = grid_for((threads + kWave - 1) / kWave, 16);
    if (fmt == COAT_FMT_E4M3) hipLaunchKernelGGL(encode_kernel<COAT_FMT_E4M3>, dim3(grid), dim3(kBlock), 0, st, y, n, q);
    else hipLaunchKernelGGL(encode_kernel<COAT_FMT_E5M2>, dim3(grid), dim3(kBlock), 0, st, y, n, q);
    return launch_status();
}

int coat_fp8_decode(const uint8_t* q, int64_t n, int32_t fmt, float* y, coat_stream_t stream) {
    if (n < 0 || (fmt != COAT_FMT_E4M3 && fmt != COAT_FMT_E5M2)) return COAT_EINVAL;
    if (n == 0) return COAT_OK;
    if (!y || !q) return COAT_EINVAL;
    if (!aligned(y, 4)) return COAT_EALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const unsigned grid = grid_for((n + kWave - 1) / kWave, 16);
    if (fmt == COAT_FMT_E4M3) hipLaunchKernelGGL(decode_kernel<COAT_FMT_E4M3>, dim3(grid), dim3(kBlock), 0, st, q, n, y);
    else hipLaunchKernelGGL(decode_kernel<COAT_FMT_E5M2>, dim3(grid), dim3(kBlock), 0, st, q, n, y);
    return launch_status();
}

}  // extern "C"
