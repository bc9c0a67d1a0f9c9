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
//     for the per-element work each lane owns 16 consecutive elements (codes
//     and per-group state are read and written that way); a tile wholly
//     inside its tensor moves its master weights, grads and bf16 copy with
//     wave accesses over 1 KB of consecutive bytes, re-laid between the two
//     layouts by a cross-lane swap (grads) and a per-wave LDS area;
//   * a group of G elements spans G/16 lanes of one wave; group statistics
//     are DPP butterfly reductions across those lanes, no LDS round trip;
//   * moments are dequantized, updated and reduced in fp64 (an fp64 FMA
//     issues in about 1.4 times the time of an fp32 one here): the group's k
//     and s are ill-conditioned in its smallest |m'|, usually a
//     near-cancellation of b1*m and (1-b1)*g, so the per-element chain
//     carries 53 bits;
//   * the per-group scalar work (k, s, the dequantization constants) runs
//     once per lane pair: the even lane of a pair does the first moment, the
//     odd lane the second, and the pair swaps results through DPP;
//   * requantization runs in fp32 with the native v_log_f32 / v_exp_f32 and
//     the hardware OCP FP8 converts; an element whose expanded value lies
//     within a relative window of an FP8 rounding midpoint is decided exactly
//     in fp64 by comparing |x| with the group's threshold for that midpoint;
//   * the AdamW update itself (master weights, bf16 copy) runs in fp32;
//   * the multi-tensor kernel walks a descriptor table of a whole parameter
//     list in one launch; tiles never span tensors.
#include <mutex>

#include "coat_common.h"

namespace {

// ------------------------------------------------------------------ fp64 math
//
// exp2: u = n + f with n = rint(u), |f| <= 1/2, and 2^f = exp(f ln 2). The
// polynomial is the degree-10 one interpolating 2^f at the eleven Chebyshev
// nodes of [-1/2, 1/2] (relative error below 2^-51.5), shared by every use but
// the direct path's per-element dequantization below, so that the kernels hold
// few sets of constants (fp64 operands cannot be instruction literals here;
// they occupy registers). The smallest member of a
// group is usually a near-cancellation b1*m + (1-b1)*g whose relative error is
// the dequantization error amplified by |b1*m| / |m'| (1e8 and more in the
// tails of a 13e9-element step), and k and s follow it, so the dequantized
// moments are kept within a few 1e-15.
// The direct path's per-element dequantization splits finer: u = (32 n + j) / 32 + f with
// |f| <= 1/64, 2^u = 2^n 2^(j/32) 2^f, the 32 values 2^(j/32) (correctly
// rounded) from a per-block LDS table and 2^f from the degree-5 polynomial
// interpolating it at the six Chebyshev nodes of [-1/64, 1/64] (widened by
// 2^-12; relative error below 2^-52.6 with its fp64 coefficients). Evaluated
// in fp64 the whole product is within 2^-50.3 of 2^u at worst (2^-51.0 for the
// degree-10 form) for half the polynomial.
// log2: x = m 2^e with m in [sqrt(1/2), sqrt(2)), u = (m-1)/(m+1), and
// ln m = 2 atanh(u) = 2 sum u^(2j+1) / (2j+1); |u| <= 0.1716, so 12 terms
// reach 2^-56. Quotients and reciprocals use the hardware reciprocal estimate
// refined by Newton steps. Coefficients are (ln 2)^i / i! and
// 2 log2(e) / (2j+1) rounded to fp64.

// Coefficients, highest degree first: 2^f on [-1/2, 1/2] (degree 10) and
// 2 log2(e) / (2j+1) for the atanh series of log2 (in w = u^2, 12 terms).
constexpr int kExp2N = 11;
constexpr int kLog2N = 12;
__device__ constexpr double kExp2C[kExp2N] = {
    0x1.e6063f7217bc6p-28, 0x1.b675bca4eeebbp-24, 0x1.62bfd47773353p-20, 0x1.ffcb54062e698p-17,
    0x1.430913096fd9fp-13, 0x1.5d87fe9d7a584p-10, 0x1.3b2ab6fba1ddap-7,  0x1.c6b08d703ce49p-5,
    0x1.ebfbdff82c598p-3,  0x1.62e42fefa3a19p-1,  1.0};
// 2^f on [-1/64, 1/64] (degree 5, highest first) and 2^(j/32), j = 0..31.
constexpr int kExp2SN = 6;
__device__ constexpr double kExp2SC[kExp2SN] = {
    0x1.5d885e7af0753p-10, 0x1.3b2b302e43a47p-7, 0x1.c6b08d7038095p-5, 0x1.ebfbdff7fee04p-3,
    0x1.62e42fefa39efp-1,  1.0};
constexpr int kExp2J = 32;
__device__ constexpr double kExp2JT[kExp2J] = {
    0x1.0000000000000p+0, 0x1.059b0d3158574p+0, 0x1.0b5586cf9890fp+0, 0x1.11301d0125b51p+0,
    0x1.172b83c7d517bp+0, 0x1.1d4873168b9aap+0, 0x1.2387a6e756238p+0, 0x1.29e9df51fdee1p+0,
    0x1.306fe0a31b715p+0, 0x1.371a7373aa9cbp+0, 0x1.3dea64c123422p+0, 0x1.44e086061892dp+0,
    0x1.4bfdad5362a27p+0, 0x1.5342b569d4f82p+0, 0x1.5ab07dd485429p+0, 0x1.6247eb03a5585p+0,
    0x1.6a09e667f3bcdp+0, 0x1.71f75e8ec5f74p+0, 0x1.7a11473eb0187p+0, 0x1.82589994cce13p+0,
    0x1.8ace5422aa0dbp+0, 0x1.93737b0cdc5e5p+0, 0x1.9c49182a3f090p+0, 0x1.a5503b23e255dp+0,
    0x1.ae89f995ad3adp+0, 0x1.b7f76f2fb5e47p+0, 0x1.c199bdd85529cp+0, 0x1.cb720dcef9069p+0,
    0x1.d5818dcfba487p+0, 0x1.dfc97337b9b5fp+0, 0x1.ea4afa2a490dap+0, 0x1.f50765b6e4540p+0};
__device__ constexpr double kLog2C[kLog2N] = {
    0x1.00ecd7e080215p-3, 0x1.1964ec6fc9491p-3, 0x1.3703c1f4d0ffep-3, 0x1.5b9ac9b743f0dp-3,
    0x1.89f3b1694cffep-3, 0x1.c68f568d31760p-3, 0x1.0c9a84994022dp-2, 0x1.484b13d7c02a9p-2,
    0x1.a61762a7aded9p-2, 0x1.2776c50ef9bfep-1, 0x1.ec709dc3a03fdp-1, 0x1.71547652b82fep+1};

// The rare exact paths read the coefficients from an LDS copy (CoefPtr) rather
// than holding them in registers: fp64 constants cannot be instruction literals
// on gfx950, and register copies of them for code that seldom runs would crowd
// out a third wave per SIMD. The per-element and per-group code on the common
// path uses the constants directly.
typedef const __attribute__((address_space(3))) double* CoefPtr;
constexpr int kCoefExp2 = 0;          // offset of the exp2 coefficients
constexpr int kCoefLog2 = kExp2N;     // offset of the log2 coefficients
constexpr int kCoefN = kExp2N + kLog2N;

// a * b + c as the three-address v_fma_f64. With the coefficient (held in a
// register) as the addend, the compiler otherwise picks the accumulating
// v_fmac_f64 and copies the coefficient into the accumulator first, one extra
// move per Horner step.
__device__ __forceinline__ double fma3(double a, double b, double c) {
    double r;
    asm("v_fma_f64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(c));
    return r;
}

__device__ __forceinline__ double exp2_poly10(double f) {
    double p = kExp2C[0];
#pragma unroll
    for (int i = 1; i < kExp2N; ++i) p = fma3(p, f, kExp2C[i]);
    return p;
}
// 2^(d/32 + l) for |d| <= 1/2 and a small l (the low part of the exponent):
// the degree-5 polynomial above in f = d / 32, its coefficients scaled by
// 32^-i (exact) so that d enters unscaled, and its constant term replaced by
// c0 = 1 + l ln 2. That drops l ln 2 (2^f - 1), at most |l| 2^-7 relative:
// 2^-51 for |l| = 2^-44, the low part's size for exponents near 2^8 in
// magnitude, far less for common ones.
__device__ constexpr double kExp2SD[kExp2SN - 1] = {
    kExp2SC[0] * 0x1p-25, kExp2SC[1] * 0x1p-20, kExp2SC[2] * 0x1p-15, kExp2SC[3] * 0x1p-10, kExp2SC[4] * 0x1p-5};
__device__ __forceinline__ double exp2_poly5_32(double d, double c0) {
    double p = kExp2SD[0];
#pragma unroll
    for (int i = 1; i < kExp2SN - 1; ++i) p = fma3(p, d, kExp2SD[i]);
    return __builtin_fma(p, d, c0);
}
__device__ __forceinline__ double exp2_poly10(double f, CoefPtr cf) {
    double p = cf[kCoefExp2];
#pragma unroll
    for (int i = 1; i < kExp2N; ++i) p = __builtin_fma(p, f, cf[kCoefExp2 + i]);
    return p;
}


// v_cvt_i32_f64 clamps out-of-range values to INT_MIN / INT_MAX and maps NaN
// to 0; spelled out so that the compiler cannot treat overflow as undefined.
__device__ __forceinline__ int cvt_i32_sat(double x) {
    int r;
    asm volatile("v_cvt_i32_f64 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// Plain fp64 max / min (v_max_f64, v_min_f64) of values that are never
// signalling NaNs, without the quieting the IEEE mode would otherwise add.
__device__ __forceinline__ double vmax(double a, double b) {
    double r;
    asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ double vmin(double a, double b) {
    double r;
    asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// max(a, |b|) and min(a, |b|) with the absolute value as a source modifier.
__device__ __forceinline__ double vmax_abs(double a, double b) {
    double r;
    asm("v_max_f64 %0, %1, |%2|" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ double vmin_abs(double a, double b) {
    double r;
    asm("v_min_f64 %0, %1, |%2|" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// 2^u for any u (NaN -> NaN, huge -> 0 / Inf).
__device__ __forceinline__ double exp2_full(double u) {
    double n = __builtin_rint(u);
    double f = u - n;
    return __builtin_amdgcn_ldexp(exp2_poly10(f), cvt_i32_sat(n));
}
__device__ __forceinline__ double exp2_full(double u, CoefPtr cf) {
    double n = __builtin_rint(u);
    double f = u - n;
    return __builtin_amdgcn_ldexp(exp2_poly10(f, cf), cvt_i32_sat(n));
}

// 1/b for finite normal b: hardware estimate plus two Newton steps.
__device__ __forceinline__ double rcp_f64(double b) {
    double r = __builtin_amdgcn_rcp(b);
    r = __builtin_fma(__builtin_fma(-b, r, 1.0), r, r);
    r = __builtin_fma(__builtin_fma(-b, r, 1.0), r, r);
    return r;
}

// 1/b to about 2^-48 (one Newton step on the hardware estimate, which is good
// to about 2^-24): enough before a correction step or a rounding to fp32.
__device__ __forceinline__ double rcp_f64_1(double b) {
    const double r = __builtin_amdgcn_rcp(b);
    return __builtin_fma(__builtin_fma(-b, r, 1.0), r, r);
}

// a/b for finite normal b, within an ulp (the final correction step takes the
// quotient from the reciprocal's 2^-48 to full precision).
__device__ __forceinline__ double div_f64(double a, double b) {
    const double r = rcp_f64_1(b);
    const double q = a * r;
    return __builtin_fma(__builtin_fma(-b, q, a), r, q);
}

// log2(x) for finite x > 0 (normal or subnormal); also returns the rounding
// error of the result in `lo` (hi + lo carries about 2^-104 relative of the
// exponent part, within the polynomial's own error). C: coefficient source
// (kLog2C or an LDS copy).
template <typename C>
__device__ __forceinline__ double log2_dd_impl(double x, double& lo, C c) {
    int e = __builtin_amdgcn_frexp_exp(x);
    double m = __builtin_amdgcn_frexp_mant(x);  // [0.5, 1)
    if (m < 0x1.6a09e667f3bcdp-1) {             // sqrt(1/2)
        m = m * 2.0;
        e -= 1;
    }
    const double u = div_f64(m - 1.0, m + 1.0);
    const double w = u * u;
    double p = c[0];
#pragma unroll
    for (int i = 1; i < kLog2N; ++i) p = fma3(p, w, c[i]);
    const double ed = (double)e;
    const double hi = __builtin_fma(u, p, ed);
    lo = __builtin_fma(u, p, ed - hi);  // ed - hi is exact (|u p| <= 1/2)
    return hi;
}
__device__ __forceinline__ double log2_full_dd(double x, double& lo) { return log2_dd_impl(x, lo, kLog2C); }
__device__ __forceinline__ double log2_full_dd(double x, double& lo, CoefPtr cf) {
    return log2_dd_impl(x, lo, cf + kCoefLog2);
}
__device__ __forceinline__ double log2_full(double x) {
    double lo;
    return log2_full_dd(x, lo);
}
__device__ __forceinline__ double log2_full(double x, CoefPtr cf) {
    double lo;
    return log2_full_dd(x, lo, cf);
}

__device__ __forceinline__ float next_up(float x) {  // x >= 0 finite
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) + 1u);
}
__device__ __forceinline__ float next_down(float x) {  // x > 0 finite
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) - 1u);
}

// All-reduce over the `lanes` lanes (a power of two, aligned) owning a group.
// After the first steps the sub-blocks agree, so the mirror permutations pair
// every lane with one of the other half, as an xor would.
__device__ __forceinline__ double group_max(double v, int lanes) {
    for (int d = 1; d < lanes; d <<= 1) v = vmax(v, xlane64(v, d));
    return v;
}
__device__ __forceinline__ double group_min(double v, int lanes) {
    for (int d = 1; d < lanes; d <<= 1) v = vmin(v, xlane64(v, d));
    return v;
}

// Per-block constant tables, one row per moment:
//   lqb[c] = for each of the 256 codes, lq = 32 log2(value(c & 0x7F) / fpmax),
//            the per-code constant of the dequantization |x| = A 2^(lq / 32k)
//            (scaled by 32 for the split of the exponent into 32nds; zero maps
//            to -1e300 and Inf to +1e300 so that the same arithmetic yields 0
//            and Inf, NaN codes to NaN), and b = the moment's decay with the
//            code's sign (the step's first operation on the dequantized value
//            is b x; the codec kernels use b = 1);
//   lqm[c] = log2(midpoint(c, c+1) / fpmax), the per-code constant of the
//            exact requantization threshold.
struct ExpJob {
    double xh, xl;
    int32_t slot;
    int32_t te;  // 1: a TE entry (A = a, times the decay b); 0: a TS entry (and its negative)
};
struct ProdJob {
    uint8_t src, mul, dst, neg;
};
constexpr int kExpJobs = 8;    // per moment: 2 per builder lane
constexpr int kProdJobs = 32;  // per moment: 8 per builder lane
struct TableJobs {
    ExpJob e[kExpJobs];
    ProdJob p[kProdJobs];  // mul: an entry index (a power of 2^r or a TS entry)
};
// One builder lane's share, in the form the builder consumes: two entries
// fm 2^(fa a + r x) written to `slot` and negated to `nslot`, then eight
// products table[src] * table[mul] written to `dst` and negated to `ndst`
// (offsets in bytes; the trash slot where no negative is wanted).
struct LaneJob {
    double xh[2], xl[2], fa[2], fm[2];
    uint32_t slot[2], nslot[2];
    uint32_t src[8], mul[8], dst[8], ndst[8];
};
struct alignas(16) LqEntry {
    double lq;
    double b;
};
// Tables of the direct path and of the codec kernels.
struct DirectTables {
    LqEntry lqb[2][256];
    double lqm[2][128];
    double coef[kCoefN];
    double e32[kExp2J];    // 2^(j/32)
};
// Tables of the table path: lq (unscaled) without the sign and decay (only its rare
// exact paths dequantize code by code), the per-code table offsets and the
// builder lanes' jobs.
struct TabTables {
    double lq[2][128];
    double lqm[2][128];
    double coef[kCoefN];
    uint32_t lut[2][256];  // per-group table offsets of each code (see GroupTable)
    LaneJob lj[8];         // per builder lane (moment * 4 + lane in quad)
};
// Set-up scratch of the table path, in LDS that the waves use later.
struct TabScratch {
    TableJobs jobs[2];     // how the lanes of a group build each moment's table
};

// The coefficient copy, through a pointer the optimizer cannot see through
// (so that per-tile code reloads the coefficients from LDS instead of hoisting
// them into registers across the tile loop).
__device__ __forceinline__ CoefPtr coef_ptr(const double* coef) {
    uint32_t a = (uint32_t)(uintptr_t)(CoefPtr)coef;
    asm volatile("" : "+v"(a));
    return (CoefPtr)(uintptr_t)a;
}

// The dequantization constants of a code, with the sign and decay folded into
// tb (direct path: from the 256-entry table) ...
struct LqSigned {
    static constexpr bool kSplit32 = true;
    const LqEntry* t;
    const double* e32;
    __device__ double get(uint32_t c, double& tb) const {
        const LqEntry e = t[c];
        tb = e.b;
        return e.lq;
    }
};
// ... or with tb formed from the code's sign (table path).
struct LqSplit {
    static constexpr bool kSplit32 = false;
    const double* lq;
    double b;
    __device__ double get(uint32_t c, double& tb) const {
        tb = (c & 0x80u) ? -b : b;
        return lq[c & 0x7Fu];
    }
};

template <int F>
__device__ double lq_entry(int c) {
    using T = Fmt<F>;
    if (T::is_nan(c)) return __builtin_nan("");
    if (T::is_inf(c)) return 1e300;
    if (c == 0) return -1e300;
    const int e = c >> T::MB, m = c & ((1 << T::MB) - 1);
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

template <int F>
__device__ double lqm_entry(int c) {
    using T = Fmt<F>;
    if (c >= T::TOP) return 0.0;
    const double mid = 0.5 * (value_of<F>(c) + value_of<F>(c + 1));
    const int e = __builtin_amdgcn_frexp_exp(mid);
    return ((double)e - T::LOG2_FPMAX) + log2_full(__builtin_amdgcn_frexp_mant(mid));
}

// Per-group dequantization tables (groups of 128 and more, tiles inside the
// tensor). A code's magnitude is 2^(max(e,1) - BIAS - MB) * i with e its
// exponent field and i its integer significand (the mantissa field, plus
// 2^MB when e > 0), so a group's dequantized, decay-scaled moment
// b sign(q) (|q| s)^(1/k) = b 2^(a + r (max(e,1) - BIAS - MB - log2 fpmax)) * sign i^r
// is the product of two table entries: TE[e] (times b) and TS[j],
// j = i + NEG * sign. Layout (entries of one table):
//   E4M3: TE[0..15], NaN at 16 (its NaN code); TS[0..31] at 17..48;
//   E5M2: TE[0..30], Inf at 31 (e = 31); TS[0..15] at 32..47, NaN at 48
//         (its NaN codes);
//   both: the powers (2^r)^0..7 at 49..56, a trash slot at 57.
constexpr int kGroupTableN = 58;
constexpr int kPowBase = 49;
constexpr int kTrash = 57;
struct GroupTable {
    double v[kGroupTableN];
};
template <int F>
constexpr int ts_base() { return F == COAT_FMT_E4M3 ? 17 : 32; }
template <int F>
constexpr int te_special() { return F == COAT_FMT_E4M3 ? 16 : 31; }
constexpr int kE5TsNan = 16;
// k1_tables writes the special exponent entry at index nte (16 and 31)
static_assert(te_special<COAT_FMT_E4M3>() == 16 && te_special<COAT_FMT_E5M2>() == 31, "special TE entries");
template <int F>
__device__ uint32_t lut_entry(int code) {
    using T = Fmt<F>;
    constexpr int NEG = 2 << T::MB;  // sign offset in TS
    const int mag = code & 0x7F, e = mag >> T::MB, m = mag & ((1 << T::MB) - 1);
    int te = e, ts = (e ? (m | (1 << T::MB)) : m) + ((code & 0x80) ? NEG : 0);
    if (T::is_nan(mag)) {
        te = te_special<F>();
        if (F == COAT_FMT_E5M2) ts = kE5TsNan;
    }
    const uint32_t te_off = (uint32_t)(te * 8);
    const uint32_t ts_off = (uint32_t)((ts_base<F>() + ts) * 8);
    return te_off | (ts_off << 16);
}

// The work of building one moment's table, split over four lanes: 8 entries
// evaluated as 2^(A + r x) (x = log2 i for TS[i], A = 0; x = max(e,1) - BIAS
// - MB - log2 fpmax for TE[e], A = a), 2 per lane, then up to 32 products
// table[dst] = table[src] * table[mul], 8 per lane. Entries:
//   E4M3: TS[i], i in {2,3,5,7,11,13}; TE anchors {0,8};
//   E5M2: TS[i], i in {2,3,5,7}; TE anchors {0,8,16,24}.
// Products: TS[2i] = TS[i] 2^r, TS[9] = TS[3]^2, TS[15] = TS[3] TS[5], and
// TE[e + j] = TE[e] 2^(r j) for e >= 1, j < 8 (TE[0] = TE[1], so from the
// anchor 0 the powers start at 0). They read only the evaluated entries and
// the powers, never each other. Unused product slots write a trash entry that
// no code reads.
template <int F>
__device__ void table_jobs(TableJobs& j, int tid) {
    using T = Fmt<F>;
    constexpr bool E4 = F == COAT_FMT_E4M3;
    constexpr int NTS = E4 ? 6 : 4;
    constexpr int TSB = ts_base<F>();
    constexpr int NTE = E4 ? 16 : 31;  // TE entries (E5M2: 31 is the Inf entry)
    if (tid < kExpJobs) {
        ExpJob& e = j.e[tid];
        if (tid < NTS) {
            const int ts[6] = {2, 3, 5, 7, 11, 13};
            const int i = ts[tid];
            e.xh = log2_full_dd((double)i, e.xl);
            e.slot = TSB + i;
            e.te = 0;
        } else {
            const int a = 8 * (tid - NTS);
            const double x = (double)((a > 0 ? a : 1) - T::BIAS - T::MB);
            const double h = x - T::LOG2_FPMAX;
            const double bb = h - x;
            e.xh = h;
            e.xl = ((x - (h - bb)) + (-T::LOG2_FPMAX - bb)) - T::LOG2_FPMAX_LO;
            e.slot = a;
            e.te = 1;
        }
    } else if (tid < kExpJobs + kProdJobs) {
        const int q = tid - kExpJobs;
        ProdJob pj{0, 0, (uint8_t)kTrash, 0};
        // TS products first (src, mul, dst), then the TE chains
        const int ts_src[8] = {2, 3, 2, 5, 3, 7, 3, 3};
        const int ts_mul[8] = {kPowBase + 1, kPowBase + 1, kPowBase + 2, kPowBase + 1, kPowBase + 2, kPowBase + 1,
                               TSB + 3, TSB + 5};
        const int ts_dst[8] = {4, 6, 8, 10, 12, 14, 9, 15};
        const int nts = E4 ? 8 : 2;
        if (q < nts) {
            pj = ProdJob{(uint8_t)(TSB + ts_src[q]), (uint8_t)ts_mul[q], (uint8_t)(TSB + ts_dst[q]), 1};
        } else {
            const int r = q - nts, a = 8 * (r / 7), jj = 1 + r % 7;
            if (a + jj < NTE)
                pj = ProdJob{(uint8_t)a, (uint8_t)(kPowBase + (a == 0 ? jj - 1 : jj)), (uint8_t)(a + jj), 0};
        }
        j.p[q] = pj;
    }
}

// Filled by the block's 256 threads: thread i covers moment i >> 7, code i & 127
// and its negative.
template <int FM, int FV>
__device__ __forceinline__ void fill_direct_tables(DirectTables& ct, double bm, double bv) {
    const int f = threadIdx.x >> 7, c = threadIdx.x & 127;
    const double lq = 32.0 * (f ? lq_entry<FV>(c) : lq_entry<FM>(c));
    const double b = f ? bv : bm;
    ct.lqb[f][c] = LqEntry{lq, b};
    ct.lqb[f][c | 128] = LqEntry{lq, -b};
    ct.lqm[f][c] = f ? lqm_entry<FV>(c) : lqm_entry<FM>(c);
    if (threadIdx.x < kCoefN)
        ct.coef[threadIdx.x] = threadIdx.x < kExp2N ? kExp2C[threadIdx.x] : kLog2C[threadIdx.x - kExp2N];
    if (threadIdx.x < kExp2J) ct.e32[threadIdx.x] = kExp2JT[threadIdx.x];
    __syncthreads();
}

// The same for the table path; `scratch` (LDS the waves use later) holds the
// job lists while the per-lane jobs are derived from them.
template <int FM, int FV>
__device__ __forceinline__ void fill_tab_tables(TabTables& ct, TabScratch& scratch, double bm, double bv) {
    const int f = threadIdx.x >> 7, c = threadIdx.x & 127;
    ct.lq[f][c] = f ? lq_entry<FV>(c) : lq_entry<FM>(c);
    ct.lqm[f][c] = f ? lqm_entry<FV>(c) : lqm_entry<FM>(c);
    if (threadIdx.x < kCoefN)
        ct.coef[threadIdx.x] = threadIdx.x < kExp2N ? kExp2C[threadIdx.x] : kLog2C[threadIdx.x - kExp2N];
    ct.lut[f][c] = f ? lut_entry<FV>(c) : lut_entry<FM>(c);
    ct.lut[f][c | 128] = f ? lut_entry<FV>(c | 128) : lut_entry<FM>(c | 128);
    if (threadIdx.x < 64) table_jobs<FM>(scratch.jobs[0], threadIdx.x);
    else if (threadIdx.x < 128) table_jobs<FV>(scratch.jobs[1], threadIdx.x - 64);
    __syncthreads();
    if (threadIdx.x < 8) {
        const int mu = threadIdx.x >> 2, t = threadIdx.x & 3;
        const bool e4 = (mu ? FV : FM) == COAT_FMT_E4M3;
        const uint32_t NEG = e4 ? 16 : 8;
        const TableJobs& J = scratch.jobs[mu];
        LaneJob& L = ct.lj[threadIdx.x];
        for (int q = 0; q < 2; ++q) {
            const ExpJob& e = J.e[2 * t + q];
            L.xh[q] = e.xh;
            L.xl[q] = e.xl;
            L.fa[q] = e.te ? 1.0 : 0.0;
            L.fm[q] = e.te ? (mu ? bv : bm) : 1.0;
            L.slot[q] = 8u * (uint32_t)e.slot;
            L.nslot[q] = 8u * (e.te ? (uint32_t)kTrash : (uint32_t)e.slot + NEG);
        }
        for (int q = 0; q < 8; ++q) {
            const ProdJob& pj = J.p[8 * t + q];
            L.src[q] = 8u * pj.src;
            L.mul[q] = 8u * pj.mul;
            L.dst[q] = 8u * pj.dst;
            L.ndst[q] = 8u * (pj.neg ? (uint32_t)pj.dst + NEG : (uint32_t)kTrash);
        }
    }
    __syncthreads();
}


// ------------------------------------------------------------------ group state

// Dequantization constants of a stored group: x = 2^(LQ[q] r + a) with
// r = 1/k and a = log2((s fpmax)^(1/k)), the log2 of the group's previous
// amax, carried as a + a_lo (double-double) so that the exponent keeps its
// accuracy for |x| far from 1. A zero scale gives a = -1e300 (every finite
// code decodes to 0) and a NaN scale a = NaN.
struct OldGroup {
    double a;
    double a_lo;
    double r;
    double r_lo;  // rounding error of r = 1/k (used by the per-group tables)
};

__device__ __forceinline__ OldGroup old_group(double s, float k, double log2_fpmax, double log2_fpmax_lo) {
    OldGroup g;
    const double kd = (double)k;
    g.r = rcp_f64(kd);
    g.r_lo = __builtin_fma(-kd, g.r, 1.0) * g.r;
    g.a_lo = 0.0;
    if (s > 0.0 && s < __builtin_inf()) {
        double l_lo;
        const double l = log2_full_dd(s, l_lo);
        // (l + l_lo) + (log2_fpmax + log2_fpmax_lo), two-sum of the leading parts
        const double t = l + log2_fpmax;
        const double bb = t - l;
        const double t_lo = ((l - (t - bb)) + (log2_fpmax - bb)) + (l_lo + log2_fpmax_lo);
        // (t + t_lo) * (r + r_lo), r_lo the rounding error of 1/k
        g.a = t * g.r;
        g.a_lo = __builtin_fma(t, g.r, -g.a) + __builtin_fma(t, g.r_lo, t_lo * g.r);
    } else {
        g.a = (s == 0.0) ? -1e300 : __builtin_nan("");
    }
    return g;
}

// Requantization constants of a group from its statistics.
struct NewGroup {
    double s;      // stored scale
    double amax;   // largest magnitude (exact path)
    double r;      // 1 / k in fp64 (exact path)
    float k;       // stored exponent
    float ia;      // 1 / amax in fp32 (0 for an all-zero group)
    float w;       // the fast path's ambiguity window for this k
    uint32_t flags;
};
constexpr uint32_t kPoison = 1u;  // non-finite member: every code 0x7F
constexpr uint32_t kSlow = 2u;    // fp32 fast path unsafe for this group: exact path for all

// k = ln R_fp8 / ln(amax / amin) (= log2 R_fp8 / log2 R), k = 1 for an
// all-zero or near-constant group or without expansion; then the range guard:
// amax^k and amax^k / R_fp8 within [2^-1022, 2^1023]; s = amax^k / fpmax.
// log2 of x (hi + lo) for finite x > 0. For 0 or a non-finite x (the
// statistics of all-zero and poisoned groups) the result is meaningless and
// unused: new_group overrides everything it feeds for those groups.
__device__ __forceinline__ double log2_stat(double x, double& lo) {
    return log2_full_dd(x, lo);
}

// Whether the correctly rounded fp64 quotient a / b exceeds T = 1 + 1e-6 (the
// fp64 constant), for finite a >= b > 0: the near-constant test of the group's
// ratio, decided without a division. RN(a / b) > T exactly when a / b lies
// above M = T + 2^-53, the midpoint between T and its successor (M b is never
// an fp64 number, as M has 54 significant bits, so no tie arises). With
// d = fma(-T, b, a): a - T b is a multiple of 2^(e_b - 104), so wherever it is
// within 4 h b of zero (h b = 2^-53 b) it has at most 53 significant bits and
// d is exact; farther out, rounding keeps its order against h b. Hence
// a / b > M iff d > h b. Tiny b is scaled by 2^600 first so that the
// difference stays above the fp64 subnormal range; a ratio of two or more
// needs no test.
constexpr double kNearConstant = 1.0 + 1e-6;
__device__ __forceinline__ bool ratio_above_near_constant(double a, double b) {
    if (!(a < 2.0 * b)) return true;
    if (b < 0x1p-960) {
        a = __builtin_amdgcn_ldexp(a, 600);
        b = __builtin_amdgcn_ldexp(b, 600);
    }
    return __builtin_fma(-kNearConstant, b, a) > b * 0x1p-53;
}

// L + L_lo = log2(amax), Lm + Lm_lo = log2(amin) (as from log2_stat); the
// group's log2(amax / amin) is their double-double difference.
__device__ NewGroup new_group(double amax, double amin, double L, double L_lo, double Lm, double Lm_lo,
                              bool poison, bool expand, const FmtRT& F) {
    NewGroup g;
    g.amax = amax;
    // Poisoned and all-zero groups are rare: the common path below runs for
    // every lane (its values for those groups are meaningless: L and Lm are
    // then unusable and 1/amax infinite), the range guard is kept from them,
    // and their fields are overridden in a wave-uniform branch at the end.
    const bool rare = poison || amax == 0.0;
    float k = 1.0f;
    const double d = L - Lm;
    const double log2R = d + (((L - d) - Lm) + (L_lo - Lm_lo));
    if (expand && !rare && ratio_above_near_constant(amax, amin)) k = (float)(F.log2_rf * rcp_f64(log2R));
    const double lo = -1022.0 + F.log2_rf, hi = 1023.0;
    const double kL = (double)k * L;
    if (!rare && !(kL >= lo && kL <= hi)) {
        asm volatile("");  // rare: not to be computed speculatively on the common path
        const double bound = (L < 0.0) ? lo / L : hi / L;
        float kk = (float)bound;
        if (kk > k) kk = k;
        while (kk > 0.0f && !((double)kk * L >= lo && (double)kk * L <= hi)) kk = next_down(kk);
        while (next_up(kk) <= k && (double)next_up(kk) * L >= lo && (double)next_up(kk) * L <= hi)
            kk = next_up(kk);
        k = kk;
    }
    g.k = k;
    g.r = rcp_f64((double)k);
    g.s = exp2_full((double)k * L - F.log2_fpmax);
    // k = 1: s is the plain quotient amax / fpmax, as defined (rare with
    // expansion: near-constant groups)
    if (__builtin_expect(__any(k == 1.0f), 0)) {
        if (k == 1.0f) g.s = amax / F.fpmax;
    }
    g.ia = (float)rcp_f64_1(amax);
    g.w = __builtin_fmaf(kAmbW1, k, F.amb_w0);
    // The fp32 path needs every member and 1/amax normal in fp32 and |x| / amax
    // at least 2^-100 for nonzero members.
    g.flags = (amax <= 0x1p126 && amin >= 0x1p-126 && log2R <= 100.0) ? 0u : kSlow;
    if (__builtin_expect(__any(rare), 0)) {
        if (rare) {
            g.s = poison ? __builtin_nan("") : 0.0;
            g.k = 1.0f;
            g.r = 1.0;
            g.ia = 0.0f;
            g.w = 0.0f;
            g.flags = poison ? kPoison : 0u;
        }
    }
    return g;
}

// Swap the per-group results of a lane pair (lane ^ 1).
__device__ __forceinline__ OldGroup swap_pair(const OldGroup& g) {
    return OldGroup{dpp64<kDppXor1>(g.a), dpp64<kDppXor1>(g.a_lo), dpp64<kDppXor1>(g.r), dpp64<kDppXor1>(g.r_lo)};
}
// The fields the fast requantization reads; amax and r (exact path only) are
// exchanged when that path runs.
__device__ __forceinline__ NewGroup swap_pair(const NewGroup& g) {
    NewGroup o;
    o.s = g.s;  // stored by the computing lane only
    o.amax = 0.0;
    o.r = 0.0;
    o.k = __builtin_bit_cast(float, dpp32<kDppXor1>(__builtin_bit_cast(uint32_t, g.k)));
    o.ia = __builtin_bit_cast(float, dpp32<kDppXor1>(__builtin_bit_cast(uint32_t, g.ia)));
    o.w = __builtin_bit_cast(float, dpp32<kDppXor1>(__builtin_bit_cast(uint32_t, g.w)));
    o.flags = dpp32<kDppXor1>(g.flags);
    return o;
}

// Exact code of one element with magnitude |x| whose fast-path code is `lo`
// (magnitude) and which lies near the midpoint between lo and lo + 1:
// y = fpmax (|x| / amax)^k against that midpoint, ties to the even code. For
// k = 1 the expanded value is formed as fpmax (|x| / amax) with IEEE
// operations; otherwise |x| is compared with amax 2^(log2(mid / fpmax) / k).
__device__ __forceinline__ uint32_t exact_mag(double ax, uint32_t lo, const NewGroup& g, const double* lqm,
                                              double mid, const FmtRT& F, CoefPtr cf) {
    bool up;
    bool tie;
    if (g.k == 1.0f) {
        const double y = F.fpmax * (ax / g.amax);
        up = y > mid;
        tie = y == mid;
    } else {
        const double thr = g.amax * exp2_full(lqm[lo] * g.r, cf);
        up = ax > thr;
        tie = ax == thr;
    }
    if (tie) up = (lo & 1u) != 0;
    return up ? lo + 1 : lo;
}

// Exact code of one element from scratch (groups outside the fp32 path's range
// and the standalone quantizer's slow elements): y = fpmax (|x| / amax)^k in
// fp64, formed as fpmax (|x| / amax) with IEEE operations when k = 1.
template <int F>
__device__ uint32_t exact_code_full(double x, const NewGroup& g, CoefPtr cf) {
    using T = Fmt<F>;
    const uint32_t sign = __builtin_signbit(x) ? 0x80u : 0u;
    if (g.flags & kPoison) return 0x7Fu;
    if (x == 0.0 || g.amax == 0.0) return sign;
    const double t = __builtin_fabs(x) / g.amax;
    const double y = (g.k == 1.0f) ? T::FPMAX * t
                                   : exp2_full((double)g.k * log2_full(t, cf) + T::LOG2_FPMAX, cf);
    return sign | encode_mag_exact<F>(y);
}

// Fast requantization of 4 elements (fp32 copies xf) into one code word;
// `amb` gets 0x80 in each byte whose code is within the ambiguity window of a
// rounding midpoint.
template <int F>
__device__ __forceinline__ uint32_t fast_codes4(const float* xf, const NewGroup& g, uint32_t& amb) {
    using T = Fmt<F>;
    float lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float t = __builtin_fabsf(xf[i]) * g.ia;
        const float l = __builtin_amdgcn_logf(t);
        const float z = __builtin_fmaf(g.k, l, T::LOG2_FPMAX_F);
        const float y = __builtin_amdgcn_exp2f(z);
        lo[i] = __builtin_copysignf(__builtin_fmaf(-y, g.w, y), xf[i]);
        // y <= fpmax (1 + 1e-5) here, far below the overflow midpoint, so no clamp
        hi[i] = __builtin_fmaf(y, g.w, y);
    }
    // The second convert writes the high halves, so the first one's
    // passthrough operand may be any register that dies there.
    uint32_t wl = cvt_pk<F, false>(lo[0], lo[1], __builtin_bit_cast(uint32_t, lo[0]));
    wl = cvt_pk<F, true>(lo[2], lo[3], wl);
    uint32_t wh = cvt_pk<F, false>(hi[0], hi[1], __builtin_bit_cast(uint32_t, hi[0]));
    wh = cvt_pk<F, true>(hi[2], hi[3], wh);
    const uint32_t d = (wl ^ wh) & 0x7F7F7F7Fu;
    amb = (d + 0x7F7F7F7Fu) & 0x80808080u;
    return wl;
}

// ------------------------------------------------------------------ step

static_assert(kTile == kPlanTile, "tile size of the plan tables");

// Dequantize byte i of code word w: returns the magnitude
// 2^(LQ[c] r + a + a_lo) and sets tb to the code's table factor (+/- b), so
// that the signed value times b is tb * magnitude.
// Direct path (every element goes through here): the table holds 32 LQ, so
// U = fma(32 LQ, r, 32 a) = 32 u exactly (scaling by a power of two commutes
// with the rounding); with N = rint(U), U - N is exact (the two are within 1/2
// of each other, or N = 0), 2^u = 2^(N >> 5) 2^((N & 31) / 32) 2^((U - N) / 32).
// A NaN u gives N = 0 and a NaN result; a huge |u| saturates N, and the power
// of two then flushes to 0 or Inf. Table path (only its rare exact branches
// come here): 2^u = 2^rint(u) 2^(u - rint(u)) with the degree-10 polynomial.
template <typename L>
__device__ __forceinline__ double dequant_mag(uint32_t w, int i, const OldGroup& og, const L& src, double& tb) {
    const double lq = src.get((w >> (8 * i)) & 0xFFu, tb);
    if constexpr (L::kSplit32) {
        const double u32 = __builtin_fma(lq, og.r, og.a * 32.0);
        const double n32 = __builtin_rint(u32);
        const int ni = cvt_i32_sat(n32);
        const double c0 = __builtin_fma(og.a_lo, 0x1.62e42fefa39efp-1, 1.0);
        return __builtin_amdgcn_ldexp(src.e32[ni & 31] * exp2_poly5_32(u32 - n32, c0), ni >> 5);
    } else {
        const double u = __builtin_fma(lq, og.r, og.a);
        const double n = __builtin_rint(u);
        return __builtin_amdgcn_ldexp(exp2_poly10((u - n) + og.a_lo), cvt_i32_sat(n));
    }
}


// Groups stored with k = 1 (near-constant or all-zero groups, and every group
// without expansion): the dequantized magnitude is the plain product |q| s
// and the new moment b x + c g takes the definition's two roundings,
// RN(RN(b x) + RN(c g)), so that such groups carry the defining arithmetic
// exactly from step to step. Such a group's OldGroup has r = 1 exactly
// (k1_mark); where the rare paths read it back, its a_lo holds s instead of
// the low part of a (k1_group: the exact k = 1 formula needs s, the general
// one is not used for it there). The code's value comes from the hardware OCP
// convert, exact in fp32 (a NaN code gives NaN, the E5M2 Inf code Inf; times
// s: Inf, or NaN for s = 0).
template <int F>
__device__ __forceinline__ double code_value(uint32_t w, int i) {
    const int b = (int)(w >> (8 * i));
    if constexpr (F == COAT_FMT_E4M3)
        return (double)__builtin_amdgcn_cvt_f32_fp8(b, 0);
    else
        return (double)__builtin_amdgcn_cvt_f32_bf8(b, 0);
}
// Byte i of code word w: RN(RN(b x) + cg), x = sign(q) RN(|q| s).
template <int F>
__device__ __forceinline__ double k1_moment(uint32_t w, int i, double s, double b, double cg) {
    const double x = code_value<F>(w, i) * s;
    const double bx = b * x;
    return bx + cg;
}
__device__ __forceinline__ OldGroup k1_mark(OldGroup g, float k) {
    if (k == 1.0f) g.r = 1.0;
    return g;
}
__device__ __forceinline__ OldGroup k1_group(OldGroup g, double s, float k) {
    if (k == 1.0f) {
        g.r = 1.0;
        g.a_lo = s;
    }
    return g;
}
__device__ __forceinline__ bool is_k1(const OldGroup& g) { return g.r == 1.0; }

__device__ __forceinline__ uint32_t select4(int i, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
    return i == 0 ? a0 : (i == 1 ? a1 : (i == 2 ? a2 : a3));
}

__device__ __forceinline__ double bf16_to_f64(uint32_t word, int half) {
    return (double)__builtin_bit_cast(float, half ? (word & 0xFFFF0000u) : (word << 16));
}

// Re-layout area of one wave for whole tiles. The global streams of a tile
// are read and written 16 bytes per lane with consecutive lanes on
// consecutive 16 bytes (a wave instruction covers 1 KB); measured on the
// 13B list, the step's access pattern moves about 5 % faster that way than
// with each lane reading and writing its own 16 elements (64 bytes of master
// weights, 32 of grads and of the bf16 copy), which is the layout the
// per-element work needs (a lane's elements lie in one group). So the grads
// arrive 8 per lane per half tile, the master weights 4 per lane per quarter
// tile, and the grads, the update term and the bf16 copy are re-laid between
// the two layouts here: 256 chunks of 16 bytes, with one chunk of padding
// after every 16 so that each of the lane patterns used hits 16 distinct
// bank groups.
constexpr int kXferChunks = 256 + 16;
struct alignas(16) Xfer {
    uint32_t w[kXferChunks * 4];
};
// byte offset of 16-byte chunk c of the tile's data
__device__ __forceinline__ uint32_t xfer_off(uint32_t c) { return (c + (c >> 4)) * 16u; }
// xfer_off(a + 16 j) = xfer_off(a) + 272 j; and for a group of four chunks
// 4m .. 4m + 3 (never split by the padding) xfer_off(4m + q) = xfer_off(4m) + 16 q:
// the per-lane part once, the rest as instruction offsets.
constexpr uint32_t kXferRow = 17 * 16;
// The lane's index, formed where it is used (two mbcnt instructions) and
// opaque to the optimizer: offsets derived from it are then computed in each
// tile rather than hoisted out of the tile loop into registers (spilled).
__device__ __forceinline__ int lane_opaque() {
    uint32_t l = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(l));
    return (int)l;
}

// Per-wave LDS area after the element pass: what the rare exact paths need,
// so that no registers are held for it through the requantization. Whole
// tiles re-lay through x; their rare paths read the codes and grads again
// from global memory (both unchanged until the tile's codes are stored).
// Tiles that end inside their tensor park codes and grads here instead.
struct ParkDirect {
    union {
        struct {
            uint32_t gw[8][kWave];
            uint32_t mq[4][kWave];
            uint32_t vq[4][kWave];
        } in;
        Xfer x;
    };
    uint16_t wide[kWave];  // per lane: elements whose final master weight is in x (rare)
    double og[6][kWave];   // m: a, a_lo, r; v: a, a_lo, r
};
struct ParkTab {
    Xfer x;
    uint16_t wide[kWave];
    double s[kWave];      // the stored scale and exponent as loaded (the lane's moment, TileIn s0,
    float k[kWave];       // k0), from which the rare paths recompute the group constants
};

// Exact decision for the elements whose fast code is flagged in `amb` (one
// moment): the element's new moment is recomputed in fp64 exactly as in the
// main pass (its old code word old_word(w) and grad word grad_word(w), og the
// moment's dequantization constants), then rounded with the fp64 threshold (or from scratch for
// groups outside the fp32 path's range). Loops until no lane has a flagged
// element.
template <int F, typename OW, typename GW, typename L>
__device__ __forceinline__ void redo_ambiguous(uint32_t (&amb)[4], uint32_t (&codes)[4], OW old_word, GW grad_word,
                                               const OldGroup& og, const NewGroup& ng, const L& lq, const double* lqm,
                                               const FmtRT& F_, double b, double cb, bool square, CoefPtr cf) {
    while (__any((amb[0] | amb[1] | amb[2] | amb[3]) != 0u)) {
        if ((amb[0] | amb[1] | amb[2] | amb[3]) != 0u) {
            const int wi = amb[0] ? 0 : (amb[1] ? 1 : (amb[2] ? 2 : 3));
            const uint32_t aw = select4(wi, amb[0], amb[1], amb[2], amb[3]);
            const int bi = __builtin_ctz(aw) >> 3;
            const int e = 4 * wi + bi;
            const uint32_t oldw = old_word(wi);
            const double g = bf16_to_f64(grad_word(e >> 1), e & 1);
            double tb;
            const double mag = dequant_mag(oldw >> (8 * bi), 0, og, lq, tb);
            const double cgx = square ? (cb * g) * g : cb * g;
            const double x = is_k1(og) ? k1_moment<F>(oldw, bi, og.a_lo, b, cgx) : __builtin_fma(tb, mag, cgx);
            const uint32_t fastw = select4(wi, codes[0], codes[1], codes[2], codes[3]);
            const uint32_t lo = byte_of(fastw, bi) & 0x7Fu;
            uint32_t code;
            if (ng.flags & kSlow) {
                code = exact_code_full<F>(x, ng, cf);
            } else {
                const double mid = 0.5 * (value_of<F>(lo) + value_of<F>(lo + 1));
                code = (__builtin_signbit(x) ? 0x80u : 0u) | exact_mag(__builtin_fabs(x), lo, ng, lqm, mid, F_, cf);
            }
            const uint32_t mask = ~(0xFFu << (8 * bi)), ins = code << (8 * bi);
            const uint32_t clear = ~(0x80u << (8 * bi));
            if (wi == 0) { codes[0] = (codes[0] & mask) | ins; amb[0] &= clear; }
            if (wi == 1) { codes[1] = (codes[1] & mask) | ins; amb[1] &= clear; }
            if (wi == 2) { codes[2] = (codes[2] & mask) | ins; amb[2] &= clear; }
            if (wi == 3) { codes[3] = (codes[3] & mask) | ins; amb[3] &= clear; }
        }
    }
}

// A wave-uniform copy of a pointer, held in scalar registers (so that a
// per-lane choice between two such pointers needs no vector load).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// One tile's inputs in registers. Tiles that end inside their tensor: the
// lane's own 16 elements of every stream. Whole tiles (load_full_tile): the
// codes of the lane's own 16 elements and the stored state of its group, the
// grads 8 per lane per half tile (elements 512 h + 8 lane + j, re-laid before
// use) and the master weights 4 per lane per quarter tile (elements
// 256 i + 4 lane + j, p[4 i + j]).
struct TileIn {
    float p[16];
    uint32_t gw[8], mq[4], vq[4];
    double s0, s1;  // stored scales: the lane's moment (pair split) or m and v
    float k0, k1;
};

// Synchronous loads of one tile for the general path (any group size, tiles
// that end inside the tensor). Zeros past the end contribute nothing to the
// group statistics. With the per-group work split over a lane pair, each lane
// loads the stored state of one moment (even lane m, odd lane v) of its group,
// also lanes past the end of the tensor, which take part in the pair's work.
__device__ __forceinline__ void load_tile(const TensorRef& t, int64_t tile, int lg2_group, TileIn& in) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
    const int64_t rem = t.n - e0;
    const int nvalid = rem <= 0 ? 0 : (rem >= kLaneElems ? kLaneElems : (int)rem);
    const int64_t gidx = e0 >> lg2_group;
    const gfloat* P = gp(t.p);
    const gu16* Gr = gp(t.g);
    const gu8* MQ = gp(t.mq);
    const gu8* VQ = gp(t.vq);
    if (nvalid == kLaneElems) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 v = reinterpret_cast<const gf32x4*>(P + e0)[i];
            in.p[4 * i] = v.x; in.p[4 * i + 1] = v.y; in.p[4 * i + 2] = v.z; in.p[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4 v = reinterpret_cast<const gu32x4*>(Gr + e0)[i];
            in.gw[4 * i] = v.x; in.gw[4 * i + 1] = v.y; in.gw[4 * i + 2] = v.z; in.gw[4 * i + 3] = v.w;
        }
        const u32x4 a = *reinterpret_cast<const gu32x4*>(MQ + e0);
        in.mq[0] = a.x; in.mq[1] = a.y; in.mq[2] = a.z; in.mq[3] = a.w;
        const u32x4 b = *reinterpret_cast<const gu32x4*>(VQ + e0);
        in.vq[0] = b.x; in.vq[1] = b.y; in.vq[2] = b.z; in.vq[3] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) in.gw[i] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) { in.mq[i] = 0u; in.vq[i] = 0u; }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bool inb = i < nvalid;
            in.p[i] = inb ? P[e0 + i] : 0.0f;
            in.gw[i >> 1] |= inb ? (uint32_t)Gr[e0 + i] << (16 * (i & 1)) : 0u;
            in.mq[i >> 2] |= inb ? (uint32_t)MQ[e0 + i] << (8 * (i & 3)) : 0u;
            in.vq[i >> 2] |= inb ? (uint32_t)VQ[e0 + i] << (8 * (i & 3)) : 0u;
        }
    }
    in.s0 = 0.0; in.s1 = 0.0; in.k0 = 1.0f; in.k1 = 1.0f;
    if (lg2_group >= 5) {
        if ((gidx << lg2_group) < t.n) {
            const bool odd = (lane & 1) != 0;
            in.s0 = odd ? gp(t.vs)[gidx] : gp(t.ms)[gidx];
            in.k0 = odd ? gp(t.vk)[gidx] : gp(t.mk)[gidx];
        }
    } else if (nvalid > 0) {
        in.s0 = gp(t.ms)[gidx]; in.k0 = gp(t.mk)[gidx];
        in.s1 = gp(t.vs)[gidx]; in.k1 = gp(t.vk)[gidx];
    }
}

// Loads of a tile that lies wholly inside its tensor, for group sizes whose
// per-group work is split over lane pairs (even lane m, odd lane v).
// Issued in the order the tile consumes them (vmcnt retires in order): the
// stored scales first (the group constants and tables need only them), then
// the codes, grads and master weights, all before any use.
// QUAD (table path): lanes 4..7 of each 8 load the second moment's scale and
// exponent, lanes 0..3 the first's (the moment whose table the lane builds);
// otherwise odd lanes the second's and even lanes the first's.
template <bool QUAD = false>
__device__ __forceinline__ void load_full_tile(const TensorRef& t, int64_t tile, int lg2_group, TileIn& in) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
    const int64_t gidx = e0 >> lg2_group;
    const bool odd = ((QUAD ? lane >> 2 : lane) & 1) != 0;
    in.s0 = gp(odd ? uniform_ptr(t.vs) : uniform_ptr(t.ms))[gidx];
    in.k0 = gp(odd ? uniform_ptr(t.vk) : uniform_ptr(t.mk))[gidx];
    in.s1 = 0.0;
    in.k1 = 1.0f;
    const u32x4 a = *reinterpret_cast<const gu32x4*>(gp(t.mq) + e0);
    in.mq[0] = a.x; in.mq[1] = a.y; in.mq[2] = a.z; in.mq[3] = a.w;
    const u32x4 b = *reinterpret_cast<const gu32x4*>(gp(t.vq) + e0);
    in.vq[0] = b.x; in.vq[1] = b.y; in.vq[2] = b.z; in.vq[3] = b.w;
    // Grads 8 per lane per half tile, master weights 4 per lane per quarter
    // tile, each wave load covering 1 KB (re-laid in step_tile). A grads load
    // h puts chunk c = 64 h + 2 (lane mod 32) + lane / 32 (elements 8c ..
    // 8c + 7) in the lane, so that one swap of the two halves' words between
    // lanes l and l + 32 leaves each lane its own 16 elements.
    const gu16* Gl = gp(t.g) + tile * kTile + (uint32_t)(16 * (lane & 31) + 8 * (lane >> 5));
    const gfloat* Pl = gp(t.p) + tile * kTile + (uint32_t)(4 * lane);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const u32x4 v = *reinterpret_cast<const gu32x4*>(Gl + 512 * h);
        in.gw[4 * h] = v.x; in.gw[4 * h + 1] = v.y; in.gw[4 * h + 2] = v.z; in.gw[4 * h + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 v = *reinterpret_cast<const gf32x4*>(Pl + 256 * i);
        in.p[4 * i] = v.x; in.p[4 * i + 1] = v.y; in.p[4 * i + 2] = v.z; in.p[4 * i + 3] = v.w;
    }
    // every load is issued before any use of what they return
    asm volatile("" : "+v"(in.s0), "+v"(in.k0) :: "memory");
}

// Per-wave LDS of the table path: the group tables during the element pass,
// then the park area; of the direct path: the park area.
union WaveLdsTab {
    GroupTable tbl[16];
    ParkTab pk;
    TabScratch setup;  // wave 0's, during the block's set-up only
};
struct WaveLdsDirect {
    ParkDirect pk;
};
template <bool TAB>
struct StepLds;
template <>
struct StepLds<true> {
    using Tables = TabTables;
    using Wave = WaveLdsTab;
};
template <>
struct StepLds<false> {
    using Tables = DirectTables;
    using Wave = WaveLdsDirect;
};

// 2^(h + l) for a double-double exponent with |l| small.
__device__ __forceinline__ double exp2_dd(double h, double l) {
    const double n = __builtin_rint(h);
    return __builtin_amdgcn_ldexp(exp2_poly10((h - n) + l), cvt_i32_sat(n));
}

// (A + r x) in double-double for x = xh + xl and r = rh + rl, A = ah + al.
__device__ __forceinline__ void fma_dd(double ah, double al, double rh, double rl, double xh, double xl,
                                       double& h, double& l) {
    const double p = rh * xh;
    const double pe = __builtin_fma(rh, xh, -p) + __builtin_fma(rh, xl, rl * xh);
    h = ah + p;
    const double bb = h - ah;
    l = ((ah - (h - bb)) + (p - bb)) + (al + pe);
}

// Builds the group tables of this tile (groups of 8 lanes or more): lanes
// 0..3 of each group build the first moment's table, lanes 4..7 the second's,
// each taking its LaneJob. Every entry is a correctly rounded 2^(A + r x)
// with a double-double exponent, or a product of such values with at most
// five roundings (TE[15] = TE[8] (2^r)^7, (2^r)^7 = (2^r)^4 (2^r)^3).
template <int FM, int FV>
__device__ __forceinline__ void build_tables(WaveLdsTab& wl, const TabTables& ct, const OldGroup& og, int lpg) {
    // opaque, so that the lane's job parameters are derived in each tile
    // instead of being hoisted out of the tile loop into registers
    int lane = threadIdx.x & (kWave - 1);
    asm volatile("" : "+v"(lane));
    const int l = lane & (lpg - 1);
    if (l >= 8) return;
    const int mu = l >> 2, t = l & 3;
    const bool e4 = (mu ? FV : FM) == COAT_FMT_E4M3;
    const int tsb = e4 ? ts_base<COAT_FMT_E4M3>() : ts_base<COAT_FMT_E5M2>();
    char* gb = reinterpret_cast<char*>(&wl.tbl[(lane / lpg) * 2 + mu]);
    auto at = [&](uint32_t off) -> double& { return *reinterpret_cast<double*>(gb + off); };
    const double a = og.a, a_lo = og.a_lo, r = og.r, r_lo = og.r_lo;
    const LaneJob& J = ct.lj[l];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        double h, lo;
        fma_dd(J.fa[q] * a, J.fa[q] * a_lo, r, r_lo, J.xh[q], J.xl[q], h, lo);
        const double v = J.fm[q] * exp2_dd(h, lo);
        at(J.slot[q]) = v;
        at(J.nslot[q]) = -v;
    }
    asm volatile("" ::: "memory");
    if (t == 0) {
        const double P = at(8u * (tsb + 2));
        const double P2 = P * P, P3 = P2 * P, P4 = P2 * P2;
        at(8u * kPowBase) = 1.0;
        at(8u * (kPowBase + 1)) = P;
        at(8u * (kPowBase + 2)) = P2;
        at(8u * (kPowBase + 3)) = P3;
        at(8u * (kPowBase + 4)) = P4;
        at(8u * (kPowBase + 5)) = P4 * P;
        at(8u * (kPowBase + 6)) = P4 * P2;
        at(8u * (kPowBase + 7)) = P4 * P3;
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const double v = at(J.src[q]) * at(J.mul[q]);
        at(J.dst[q]) = v;
        at(J.ndst[q]) = -v;
    }
    if (t == 3) {
        const int NEG = e4 ? 16 : 8;
        double* g = reinterpret_cast<double*>(gb);
        // The constant entries, from high words materialized here (opaque to
        // the optimizer): held across the tile loop instead, these constants
        // took eight registers.
        uint32_t h_nz = 0x80000000u, h_one = 0x3FF00000u, h_mone = 0xBFF00000u, h_nan = 0x7FF80000u,
                 h_inf = 0x7FF00000u;
        asm volatile("" : "+v"(h_nz), "+v"(h_one), "+v"(h_mone), "+v"(h_nan), "+v"(h_inf));
        auto hi_only = [](uint32_t h) { return __builtin_bit_cast(double, (uint64_t)h << 32); };
        g[tsb] = 0.0;
        g[tsb + NEG] = hi_only(h_nz);
        g[tsb + 1] = hi_only(h_one);
        g[tsb + 1 + NEG] = hi_only(h_mone);
        if (e4) {
            g[te_special<COAT_FMT_E4M3>()] = hi_only(h_nan);
        } else {
            g[te_special<COAT_FMT_E5M2>()] = hi_only(h_inf);
            g[tsb + kE5TsNan] = hi_only(h_nan);
        }
    }
    asm volatile("" ::: "memory");
}

// The tables of a moment stored with k = 1, built by the same builder lanes
// (after build_tables, or alone in a wave whose groups all have k = 1):
// TE[e] = 2^(max(e,1) - BIAS - MB) exactly and TS[+-i] = +-RN(b RN(i s)), so
// that a code's TE TS, an exact product, is RN(b RN(|q| s)) and the element
// pass's fma(TE, TS, c g) forms RN(RN(b x) + RN(c g)), the definition's two
// roundings (see k1_moment). The special entries are written here as well
// (E4M3: the NaN exponent entry; E5M2: the Inf exponent entry and the NaN
// significand entry), since a wave that builds only these tables reuses LDS
// that held other data: NaN codes must decode to NaN and Inf codes to Inf.
template <int FM, int FV>
__device__ __forceinline__ void k1_tables(WaveLdsTab& wl, int lpg, double s, float k, double b1, double b2) {
    const int lane = threadIdx.x & (kWave - 1);
    const int l = lane & (lpg - 1);
    if (l >= 8 || k != 1.0f) return;
    const int mu = l >> 2, t = l & 3;
    const bool e4 = (mu ? FV : FM) == COAT_FMT_E4M3;
    const int bias = e4 ? Fmt<COAT_FMT_E4M3>::BIAS : Fmt<COAT_FMT_E5M2>::BIAS;
    const int mb = e4 ? Fmt<COAT_FMT_E4M3>::MB : Fmt<COAT_FMT_E5M2>::MB;
    const int nte = e4 ? 16 : 31;       // TE entries below the special one
    const int nts = 2 << mb;            // significands 0 .. 2^(MB+1) - 1; NEG = nts
    const int tsb = e4 ? ts_base<COAT_FMT_E4M3>() : ts_base<COAT_FMT_E5M2>();
    const double b = mu ? b2 : b1;
    double* g = reinterpret_cast<double*>(&wl.tbl[(lane / lpg) * 2 + mu]);
    for (int e = t; e < nte; e += 4) g[e] = __builtin_amdgcn_ldexp(1.0, (e > 0 ? e : 1) - bias - mb);
    for (int i = t; i < nts; i += 4) {
        const double v = b * ((double)i * s);
        g[tsb + i] = v;
        g[tsb + i + nts] = -v;
    }
    if (t == 3) {
        // te_special(F) is nte in both formats
        g[nte] = e4 ? __builtin_nan("") : __builtin_inf();
        if (!e4) g[tsb + kE5TsNan] = __builtin_nan("");
    }
    asm volatile("" ::: "memory");
}

// The same out of line, for kernels in which k = 1 groups are rare (a call
// keeps its registers off the tile loop).
template <int FM, int FV>
__device__ __attribute__((noinline)) void k1_tables_cold(WaveLdsTab& wl, int lpg, double s, float k, double b1,
                                                         double b2) {
    k1_tables<FM, FV>(wl, lpg, s, k, b1, b2);
}

// The group-table offsets (TE, TS) of byte i of code word w, packed low / high.
__device__ __forceinline__ uint32_t code_offsets(uint32_t w, int i, const uint32_t* lut) {
    return lut[(w >> (8 * i)) & 0xFFu];
}
// The group's two table entries for a code with table offsets e; their
// product is b sign(q) (|q| s)^(1/k).
struct EntryPair {
    double te, ts;
};
__device__ __forceinline__ EntryPair table_entries(uint32_t e, const GroupTable& g) {
    const char* base = reinterpret_cast<const char*>(&g);
    return EntryPair{*reinterpret_cast<const double*>(base + (e & 0xFFFFu)),
                     *reinterpret_cast<const double*>(base + (e >> 16))};
}

// One wavefront tile of the step: elements [tile*1024, tile*1024 + 1024) of t,
// inputs in `in`. FULL: every element lies in the tensor and the group work is
// split over lane pairs (group >= 32), so no lane needs a bounds check.
// LG: log2 of the group size when fixed at compile time (0: c.lg2_group), so
// that the lane-group reductions unroll into straight DPP sequences.
__device__ __forceinline__ LqSigned lq_source(const DirectTables& ct, int f, double) {
    return LqSigned{ct.lqb[f], ct.e32};
}
__device__ __forceinline__ LqSplit lq_source(const TabTables& ct, int f, double b) { return LqSplit{ct.lq[f], b}; }

// The dequantization constants of both moments from the park area (rare
// paths, after the element pass). Table path: each lane parked the stored
// scale and exponent of moment (lane >> 2) & 1, lane i and lane 7 - i of each
// 8 the two; direct path: both moments' constants.
template <int FM, int FV, bool TAB, typename PK>
__device__ __forceinline__ void parked_old_groups(const PK& pk, OldGroup& gm, OldGroup& gv) {
    const int lane = threadIdx.x & (kWave - 1);
    if constexpr (TAB) {
        const FmtRT fm = fmt_rt<FM>(), fv = fmt_rt<FV>();
        const bool q_odd = ((lane >> 2) & 1) != 0;
        const OldGroup mine = k1_group(old_group(pk.s[lane], pk.k[lane], q_odd ? fv.log2_fpmax : fm.log2_fpmax,
                                                 q_odd ? fv.log2_fpmax_lo : fm.log2_fpmax_lo),
                                       pk.s[lane], pk.k[lane]);
        const OldGroup other{xlane64(mine.a, 4), xlane64(mine.a_lo, 4), xlane64(mine.r, 4), xlane64(mine.r_lo, 4)};
        gm = q_odd ? other : mine;
        gv = q_odd ? mine : other;
    } else {
        gm = OldGroup{pk.og[0][lane], pk.og[1][lane], pk.og[2][lane], 0.0};
        gv = OldGroup{pk.og[3][lane], pk.og[4][lane], pk.og[5][lane], 0.0};
    }
}

// The rare exact statistics of a tile (some lane of the wave has a zero or a
// non-finite new moment): zeros excluded from the minimum, non-finite moments
// flagged, each element recomputed in fp64 from its code and grad words
// (code_word(second, w), grad_word(w)). Moments finite in fp64 but beyond the
// fp32 range (a bf16 grad of about 1e20 or more, or a huge stored state) leave
// the fp32 update without a usable value: it is redone in fp64 from the
// master weight as loaded (p0(i), before the tile's master weights are
// stored), one element per lane at a time, and handed to on_wide(i, p').
struct RareStats {
    double amax_m, amin_m, amax_v, amin_v;
    uint32_t bad;       // bit 0: a first moment of the lane is not finite, bit 1: a second moment
    uint32_t redone;    // the lane's elements whose update was redone in fp64
    uint32_t any_wide;  // some lane of the wave redid one
};
template <int FM, int FV, typename LQ, typename CW, typename GW, typename P0, typename OW>
__device__ __forceinline__ RareStats rare_stats(const OldGroup& pm, const OldGroup& pv, const LQ& lq_m,
                                                const LQ& lq_v, const StepConsts& c, int nvalid, CW code_word,
                                                GW grad_word, P0 p0, OW on_wide) {
    RareStats r{0.0, __builtin_inf(), 0.0, __builtin_inf(), 0u, 0u, 0u};
    uint32_t wide = 0u;
    // not unrolled: one element's code and grad words at a time
#pragma unroll 1
    for (int i = 0; i < 16; ++i) {
        const uint32_t wm = code_word(false, i >> 2);
        const uint32_t wv = code_word(true, i >> 2);
        const double g = bf16_to_f64(grad_word(i >> 1), i & 1);
        double tbm, tbv;
        const double m0 = dequant_mag(wm >> (8 * (i & 3)), 0, pm, lq_m, tbm);
        const double v0 = dequant_mag(wv >> (8 * (i & 3)), 0, pv, lq_v, tbv);
        const double m1 = is_k1(pm) ? k1_moment<FM>(wm, i & 3, pm.a_lo, c.b1, c.c1 * g)
                                    : __builtin_fma(tbm, m0, c.c1 * g);
        const double v1 = is_k1(pv) ? k1_moment<FV>(wv, i & 3, pv.a_lo, c.b2, (c.c2 * g) * g)
                                    : __builtin_fma(tbv, v0, (c.c2 * g) * g);
        const double am = __builtin_fabs(m1), av = __builtin_fabs(v1);
        const bool fin_m = am < __builtin_inf(), fin_v = av < __builtin_inf();
        r.bad |= (fin_m ? 0u : 1u) | (fin_v ? 0u : 2u);
        r.amax_m = vmax(r.amax_m, am);
        r.amin_m = vmin(r.amin_m, am == 0.0 ? __builtin_inf() : am);
        r.amax_v = vmax(r.amax_v, av);
        r.amin_v = vmin(r.amin_v, av == 0.0 ? __builtin_inf() : av);
        const bool beyond = !(__builtin_fabsf((float)m1) <= 0x1.fffffep+127f) ||
                            !(__builtin_fabsf((float)v1) <= 0x1.fffffep+127f);
        wide |= (beyond && fin_m && fin_v && i < nvalid) ? 1u << i : 0u;
    }
    r.any_wide = __any(wide != 0u) ? 1u : 0u;
    while (__any(wide != 0u)) {
        if (wide != 0u) {
            const int i = __builtin_ctz(wide);
            wide &= wide - 1u;
            r.redone |= 1u << i;
            const double g = bf16_to_f64(grad_word(i >> 1), i & 1);
            double tbm, tbv;
            const uint32_t wm = code_word(false, i >> 2), wv = code_word(true, i >> 2);
            const double m0 = dequant_mag(wm >> (8 * (i & 3)), 0, pm, lq_m, tbm);
            const double v0 = dequant_mag(wv >> (8 * (i & 3)), 0, pv, lq_v, tbv);
            const double m1 = is_k1(pm) ? k1_moment<FM>(wm, i & 3, pm.a_lo, c.b1, c.c1 * g)
                                        : __builtin_fma(tbm, m0, c.c1 * g);
            const double v1 = is_k1(pv) ? k1_moment<FV>(wv, i & 3, pv.a_lo, c.b2, (c.c2 * g) * g)
                                        : __builtin_fma(tbv, v0, (c.c2 * g) * g);
            const double den = __builtin_sqrt(v1) * (double)c.ib2 + (double)c.eps;
            on_wide(i, (float)((double)p0(i) * (double)c.decay - (double)c.ssz * (m1 / den)));
        }
    }
    return r;
}

template <int FM, int FV, bool FULL, bool TAB, int LG, bool K1 = false>
__device__ __forceinline__ void step_tile(const TensorRef& t, int64_t tile, const StepConsts& c,
                                          const typename StepLds<TAB>::Tables& ct,
                                          typename StepLds<TAB>::Wave& wl, TileIn& in) {
    static_assert(!TAB || FULL, "tables only for whole tiles");
    auto& pk = wl.pk;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
    const int64_t rem = t.n - e0;
    const int nvalid = FULL ? kLaneElems : (rem <= 0 ? 0 : (rem >= kLaneElems ? kLaneElems : (int)rem));
    const int lg = LG ? LG : c.lg2_group;
    const int lpg = 1 << (lg - 4);  // lanes per group
    const int64_t gidx = e0 >> lg;
    // The lane's group holds elements (possibly not in this lane): its state is
    // stored even by lanes past the end, which take part in the pair's work.
    const bool gvalid = FULL || (gidx << lg) < t.n;
    const bool pair = FULL || lpg >= 2;      // per-group work split over a lane pair
    // Opaque to the optimizer, so that the per-lane choices between the two
    // formats' constants are made in each tile rather than held in registers
    // (spilled) across the tile loop.
    int odd_bit = lane & 1;
    asm volatile("" : "+v"(odd_bit));
    const bool odd = odd_bit != 0;
    const CoefPtr cf = coef_ptr(ct.coef);
    const FmtRT fm = fmt_rt<FM>(), fv = fmt_rt<FV>();

    gfloat* P = gp(t.p);
    gu8* MQ = gp(t.mq);
    gu8* VQ = gp(t.vq);
    float (&p)[16] = in.p;
    uint32_t (&gw)[8] = in.gw;
    const uint32_t (&mq)[4] = in.mq;
    const uint32_t (&vq)[4] = in.vq;
    // whole tiles: the wave's re-layout area
    unsigned char* X = reinterpret_cast<unsigned char*>(&wl.pk.x);

    // ---- stored group state -> dequantization constants (all lanes must be
    // active: the pair split exchanges results between lanes)
    auto groups_of = [&](double s0, float k0, double s1, float k1, OldGroup& gm, OldGroup& gv) {
        if (pair) {
            const OldGroup mine = k1_mark(old_group(s0, k0, odd ? fv.log2_fpmax : fm.log2_fpmax,
                                                    odd ? fv.log2_fpmax_lo : fm.log2_fpmax_lo),
                                          k0);
            const OldGroup other = swap_pair(mine);
            gm = odd ? other : mine;
            gv = odd ? mine : other;
        } else {
            gm = k1_mark(old_group(s0, k0, fm.log2_fpmax, fm.log2_fpmax_lo), k0);
            gv = k1_mark(old_group(s1, k1, fv.log2_fpmax, fv.log2_fpmax_lo), k1);
        }
    };
    // Table path: a lane holds the state of moment (lane >> 2) & 1, the one
    // whose table it builds; lane i and lane 7 - i of each 8 hold the two.
    const bool q_odd = ((lane >> 2) & 1) != 0;
    auto own_group = [&](double s0, float k0) {
        return old_group(s0, k0, q_odd ? fv.log2_fpmax : fm.log2_fpmax, q_odd ? fv.log2_fpmax_lo : fm.log2_fpmax_lo);
    };
    // the same from the parked state (rare paths, after the element pass)
    auto parked_groups = [&](OldGroup& gm, OldGroup& gv) { parked_old_groups<FM, FV, TAB>(pk, gm, gv); };
    OldGroup om, ov;
    // Direct path: the dequantization constants are parked at once (the rare
    // paths read them back after the element pass); a group stored with k = 1
    // parks its s in place of a_lo (k1_group), from where the exact k = 1
    // element pass also reads it.
    bool k1_wave = false;  // some group of the wave stored with k = 1
    if constexpr (!TAB) {
        groups_of(in.s0, in.k0, in.s1, in.k1, om, ov);
        pk.og[0][lane] = om.a; pk.og[1][lane] = om.a_lo; pk.og[2][lane] = om.r;
        pk.og[3][lane] = ov.a; pk.og[4][lane] = ov.a_lo; pk.og[5][lane] = ov.r;
        k1_wave = __any(is_k1(om) || is_k1(ov));
        if (__builtin_expect(k1_wave, 0)) {
            double sm = in.s0, sv = in.s1;
            if (pair) {
                const double other = dpp64<kDppXor1>(in.s0);
                sm = odd ? other : in.s0;
                sv = odd ? in.s0 : other;
            }
            if (is_k1(om)) pk.og[1][lane] = sm;
            if (is_k1(ov)) pk.og[4][lane] = sv;
        }
    }
    // Whole tiles: the grads as loaded hold chunks 2 l and 2 l + 1 of the
    // lane's half of the tile (l = lane mod 32) split between lanes l and
    // l + 32 (lane l: its own even chunk and, in the second half's words, lane
    // l + 32's even chunk; lane l + 32 the odd ones); one swap of lane l's
    // second words with lane l + 32's first words (v_permlane32_swap) gives
    // each lane its own 16 elements in order. Done just before the element pass.
    auto own_grads = [&]() {
        if constexpr (FULL) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const auto r = __builtin_amdgcn_permlane32_swap(gw[k], gw[4 + k], false, false);
                gw[k] = r[0];
                gw[4 + k] = r[1];
            }
        }
    };

    // ---- per element: dequantize, moments, statistics, AdamW update
    const auto lq_m = lq_source(ct, 0, c.b1);
    const auto lq_v = lq_source(ct, 1, c.b2);
    float xm[16], xv[16];
    double amax_m = 0.0, amin_m = __builtin_inf(), amax_v = 0.0, amin_v = __builtin_inf();
    bool k1_mixed = false;  // wave-uniform: see the direct element pass
    // sum of xm * xv: not finite if any moment is infinite or NaN (or beyond fp32)
    float fin = 0.0f;
    // upd(i, cg, cg2, m1, v1): the new moments of element i from c1 g and c2 g^2
    auto element_pass = [&](auto upd_moments) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const double g = bf16_to_f64(gw[i >> 1], i & 1);
            double m1, v1;
            upd_moments(i, c.c1 * g, (c.c2 * g) * g, m1, v1);
            amax_m = vmax_abs(amax_m, m1);
            amin_m = vmin_abs(amin_m, m1);
            amax_v = vmax_abs(amax_v, v1);
            amin_v = vmin_abs(amin_v, v1);
            xm[i] = (float)m1;
            xv[i] = (float)v1;
            fin = __builtin_fmaf(xm[i], xv[i], fin);
        }
        // the master weights last: their loads were issued last
        if constexpr (FULL) {
            // whole tiles: the update term m / (sqrt(v) / (1 - b2^t)^(1/2) + eps)
            // of the lane's elements into the re-layout area (chunks 4 lane + q),
            // applied to the master weights in their layout after the rare paths
            asm volatile("" ::: "memory");  // after the last table read (the area overlaps the tables)
            const uint32_t ob = xfer_off(4 * lane_opaque());
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float u[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 4 * q + j;
                    const float den = __builtin_fmaf(__builtin_amdgcn_sqrtf(xv[i]), c.ib2, c.eps);
                    u[j] = xm[i] * __builtin_amdgcn_rcpf(den);
                }
                *reinterpret_cast<f32x4*>(X + ob + 16 * q) = f32x4{u[0], u[1], u[2], u[3]};
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float den = __builtin_fmaf(__builtin_amdgcn_sqrtf(xv[i]), c.ib2, c.eps);
                const float upd = xm[i] * __builtin_amdgcn_rcpf(den);
                p[i] = __builtin_fmaf(-c.ssz, upd, p[i] * c.decay);
            }
        }
    };
    if constexpr (TAB) {
        // groups of 128 and more: per-group tables
        // K1 (launches without expansion, where every group is stored with
        // k = 1 after the first step): a wave whose groups all have k = 1
        // builds only the exact k = 1 tables
        if (K1 && __all(in.k0 == 1.0f)) {
            k1_tables<FM, FV>(wl, lpg, in.s0, in.k0, c.b1, c.b2);
        } else {
            build_tables<FM, FV>(wl, ct, own_group(in.s0, in.k0), lpg);
            if (__builtin_expect(__any(in.k0 == 1.0f), 0)) {
                if constexpr (K1) k1_tables<FM, FV>(wl, lpg, in.s0, in.k0, c.b1, c.b2);
                else k1_tables_cold<FM, FV>(wl, lpg, in.s0, in.k0, c.b1, c.b2);
            }
        }
        const GroupTable& tm = wl.tbl[(lane / lpg) * 2];
        const GroupTable& tv = wl.tbl[(lane / lpg) * 2 + 1];
        // Software-pipelined: element i's group-table reads are issued before
        // the code-table reads of element i + 1, so that waiting for the former
        // leaves the latter in flight and the two dependent LDS round trips of a
        // lookup overlap (the pass is otherwise bound by LDS latency; about
        // 1.5 % off the step on the 13B list).
        uint32_t em = code_offsets(mq[0], 0, ct.lut[0]), ev = code_offsets(vq[0], 0, ct.lut[1]);
        own_grads();
        element_pass([&](int i, double cg, double cg2, double& m1, double& v1) {
            const EntryPair xm_ = table_entries(em, tm), xv_ = table_entries(ev, tv);
            if (i + 1 < kLaneElems) {
                em = code_offsets(mq[(i + 1) >> 2], (i + 1) & 3, ct.lut[0]);
                ev = code_offsets(vq[(i + 1) >> 2], (i + 1) & 3, ct.lut[1]);
            }
            m1 = __builtin_fma(xm_.te, xm_.ts, cg);
            v1 = __builtin_fma(xv_.te, xv_.ts, cg2);
        });
        asm volatile("" ::: "memory");  // the park area reuses the tables' LDS
    } else {
        own_grads();
        if (!K1 || __builtin_expect(!k1_wave, 1) || !__all(is_k1(om) && is_k1(ov))) {
            // (a wave with k = 1 groups takes this pass, then the exact
            // statistics path below, which treats the k = 1 groups exactly;
            // K1 kernels have a pass of their own for waves of k = 1 groups)
            element_pass([&](int i, double cg, double cg2, double& m1, double& v1) {
                double tbm, tbv;
                const double m0 = dequant_mag(mq[i >> 2], i & 3, om, lq_m, tbm);
                const double v0 = dequant_mag(vq[i >> 2], i & 3, ov, lq_v, tbv);
                m1 = __builtin_fma(tbm, m0, cg);
                v1 = __builtin_fma(tbv, v0, cg2);
            });
            k1_mixed = k1_wave;
        } else {
            // every group of the wave stored with k = 1 (e.g. no expansion)
            const double sm = pk.og[1][lane], sv = pk.og[4][lane];
            element_pass([&](int i, double cg, double cg2, double& m1, double& v1) {
                m1 = k1_moment<FM>(mq[i >> 2], i & 3, sm, c.b1, cg);
                v1 = k1_moment<FV>(vq[i >> 2], i & 3, sv, c.b2, cg2);
            });
        }
    }
    // A zero moment (the minimum is over nonzero members) or a non-finite one:
    // the statistics are redone exactly.
    const bool special = amin_m == 0.0 || amin_v == 0.0 || !(__builtin_fabsf(fin) <= 0x1.fffffep+127f) || k1_mixed;
    // ---- park what only the exact paths (statistics with zeros, requantization) need
    if constexpr (!FULL) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pk.in.gw[i][lane] = gw[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) { pk.in.mq[i][lane] = mq[i]; pk.in.vq[i][lane] = vq[i]; }
    }
    if constexpr (TAB) {
        pk.s[lane] = in.s0;
        pk.k[lane] = in.k0;
    }
    // later reads of the park area must come from LDS, not from registers
    asm volatile("" ::: "memory");
    // The rare paths' codes and grads: whole tiles read them again from global
    // memory (unchanged until this tile's codes are stored), others from the park area.
    // (tile base, uniform, plus a 32-bit lane offset: one address register)
    auto code_word = [&](bool second, int w) -> uint32_t {
        if constexpr (FULL) {
            const gu8* base = (second ? VQ : MQ) + tile * kTile;
            return *reinterpret_cast<const gu32*>(base + (uint32_t)(16 * lane + 4 * w));
        } else {
            return second ? pk.in.vq[w][lane] : pk.in.mq[w][lane];
        }
    };
    auto grad_word = [&](int w) -> uint32_t {
        if constexpr (FULL) {
            const gu16* base = gp(t.g) + tile * kTile;
            return *reinterpret_cast<const gu32*>(base + (uint32_t)(16 * lane + 2 * w));
        } else {
            return pk.in.gw[w][lane];
        }
    };

    // bit 0: a first moment of the lane is not finite, bit 1: a second moment
    uint32_t bad = 0u;
    // whole tiles: some lane's update was redone in fp64 (its final master
    // weights are in the re-layout area, flagged in pk.wide)
    bool any_wide = false;
    if (__builtin_expect(__any(special), 0)) {
        RareStats r;
        OldGroup pm, pv;
        parked_groups(pm, pv);
        if constexpr (FULL) {
            r = rare_stats<FM, FV>(pm, pv, lq_m, lq_v, c, nvalid, code_word, grad_word,
                           [&](int i) { return (P + tile * kTile)[(uint32_t)(16 * lane + i)]; },
                           [&](int i, float pc) {
                               *reinterpret_cast<float*>(X + xfer_off(4 * lane_opaque() + (i >> 2)) + 4 * (i & 3)) = pc;
                           });
            if (r.any_wide) pk.wide[lane] = (uint16_t)r.redone;
        } else {
            r = rare_stats<FM, FV>(pm, pv, lq_m, lq_v, c, nvalid, code_word, grad_word,
                           [&](int i) { return P[e0 + i]; },
                           [&](int i, float pc) {
#pragma unroll
                               for (int j = 0; j < 16; ++j) p[j] = (j == i) ? pc : p[j];
                           });
        }
        amax_m = r.amax_m; amin_m = r.amin_m; amax_v = r.amax_v; amin_v = r.amin_v;
        bad = r.bad;
        any_wide = r.any_wide != 0u;
    }

    // ---- store the new master weights and the bf16 copy
    if constexpr (FULL) {
        // The update term to the master weights' layout (chunk 64 i + lane:
        // elements 256 i + 4 lane + j), applied there; redone elements take
        // their final value from the same slot.
        const int xl = lane_opaque();
        float pn[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 u = *reinterpret_cast<const f32x4*>(X + xfer_off(xl) + 4 * kXferRow * i);
            const float uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) pn[4 * i + j] = __builtin_fmaf(-c.ssz, uu[j], p[4 * i + j] * c.decay);
            if (__builtin_expect(any_wide, 0)) {
                // element 256 i + 4 lane + j lies in lane 16 i + lane / 4, at its index 4 (lane & 3) + j
                const uint32_t fl = (pk.wide[16 * i + (xl >> 2)] >> (4 * (xl & 3))) & 0xFu;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if ((fl >> j) & 1u) pn[4 * i + j] = uu[j];
            }
        }
        gfloat* Pl = P + tile * kTile + (uint32_t)(4 * xl);  // then constant offsets
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<gf32x4*>(Pl + 256 * i) = f32x4{pn[4 * i], pn[4 * i + 1], pn[4 * i + 2], pn[4 * i + 3]};
        if (t.w) {
            // bf16 pairs (one packed RNE convert each) to the grads' layout:
            // elements 256 i + 4 lane .. + 3 are bytes 512 i + 8 lane .. + 7 of
            // the copy, read back 16 bytes per lane (elements 512 h + 8 lane ..)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{pn[4 * i], pn[4 * i + 1]}, bf16x2));
                const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{pn[4 * i + 2], pn[4 * i + 3]}, bf16x2));
                *reinterpret_cast<u32x2*>(X + xfer_off(xl >> 1) + 8 * (xl & 1) + 2 * kXferRow * i) = u32x2{lo, hi};
            }
            gu16* Wl = gp(t.w) + tile * kTile + (uint32_t)(8 * xl);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<gu32x4*>(Wl + 512 * h) =
                    *reinterpret_cast<const u32x4*>(X + xfer_off(xl) + 4 * kXferRow * h);
        }
    } else if (nvalid == kLaneElems) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            reinterpret_cast<gf32x4*>(P + e0)[i] = f32x4{p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]};
        if (t.w) {
            // one packed RNE convert per pair (v_cvt_pk_bf16_f32)
            uint32_t wb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wb[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2 * i], p[2 * i + 1]}, bf16x2));
            gu32x4* wp = reinterpret_cast<gu32x4*>(gp(t.w) + e0);
            wp[0] = u32x4{wb[0], wb[1], wb[2], wb[3]};
            wp[1] = u32x4{wb[4], wb[5], wb[6], wb[7]};
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < nvalid) {
                P[e0 + i] = p[i];
                if (t.w) gp(t.w)[e0 + i] = __builtin_bit_cast(uint16_t, (__bf16)p[i]);
            }
        }
    }

    // ---- group statistics across the group's lanes
    amax_m = group_max(amax_m, lpg);
    amin_m = group_min(amin_m, lpg);
    amax_v = group_max(amax_v, lpg);
    amin_v = group_min(amin_v, lpg);
    // Each moment's group is poisoned by its own non-finite members (a NaN or
    // Inf grad makes both moments non-finite; a poisoned stored state only its own).
    const uint32_t bad_group = group_or(bad, lpg);
    const bool poison_m = (bad_group & 1u) != 0u, poison_v = (bad_group & 2u) != 0u;

    // ---- requantization constants (the lane pair splits the two moments)
    NewGroup nm, nv;
    double own_amax = 0.0, own_r = 0.0;  // pair split: this lane's moment's exact-path fields
    if (pair) {
        const double amax_x = odd ? amax_v : amax_m, amin_x = odd ? amin_v : amin_m;
        double L, L_lo, Lm, Lm_lo;
        if (lpg >= 4) {
            // lane quad: lanes 0, 1 take log2 of the m and v maxima, lanes 2, 3
            // of the minima, and partners (lane ^ 2) swap them
            const bool hiq = (lane & 2) != 0;
            double xl_lo;
            const double xl = log2_stat(hiq ? amin_x : amax_x, xl_lo);
            const double yl = dpp64<kDppXor2>(xl), yl_lo = dpp64<kDppXor2>(xl_lo);
            L = hiq ? yl : xl;
            L_lo = hiq ? yl_lo : xl_lo;
            Lm = hiq ? xl : yl;
            Lm_lo = hiq ? xl_lo : yl_lo;
        } else {
            L = log2_stat(amax_x, L_lo);
            Lm = log2_stat(amin_x, Lm_lo);
        }
        const NewGroup mine = new_group(amax_x, amin_x, L, L_lo, Lm, Lm_lo, odd ? poison_v : poison_m,
                                        odd ? c.expand_v : c.expand_m, odd ? fv : fm);
        const NewGroup other = swap_pair(mine);
        nm = odd ? other : mine;
        nv = odd ? mine : other;
        own_amax = mine.amax;
        own_r = mine.r;
        if (gvalid && (lane & (lpg - 1)) < 2) {
            double* sp = odd ? uniform_ptr(t.vs) : uniform_ptr(t.ms);
            float* kp = odd ? uniform_ptr(t.vk) : uniform_ptr(t.mk);
            gp(sp)[gidx] = mine.s;
            gp(kp)[gidx] = mine.k;
        }
    } else {
        double a_lo, b_lo, c_lo, d_lo;
        const double la = log2_stat(amax_m, a_lo), lb = log2_stat(amin_m, b_lo);
        const double lc = log2_stat(amax_v, c_lo), ld = log2_stat(amin_v, d_lo);
        nm = new_group(amax_m, amin_m, la, a_lo, lb, b_lo, poison_m, c.expand_m, fm);
        nv = new_group(amax_v, amin_v, lc, c_lo, ld, d_lo, poison_v, c.expand_v, fv);
        if (nvalid > 0) {
            gp(t.ms)[gidx] = nm.s; gp(t.mk)[gidx] = nm.k;
            gp(t.vs)[gidx] = nv.s; gp(t.vk)[gidx] = nv.k;
        }
    }

    // ---- requantize: fast fp32 codes, exact decision near midpoints
    uint32_t cm[4], cv[4], am[4], av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        cm[i] = fast_codes4<FM>(xm + 4 * i, nm, am[i]);
        cv[i] = fast_codes4<FV>(xv + 4 * i, nv, av[i]);
    }
    // Groups outside the fp32 path's range (every element decided exactly) or
    // poisoned (no element decided; every code NaN) are rare: their flags are
    // applied in a wave-uniform branch, so that a tile without them spends no
    // selects on them.
    const bool flagged = (nm.flags | nv.flags) != 0u;
    const bool any_flagged = __builtin_expect(__any(flagged), 0);
    if (any_flagged) {
        if (nm.flags & kSlow) { am[0] = am[1] = am[2] = am[3] = 0x80808080u; }
        if (nv.flags & kSlow) { av[0] = av[1] = av[2] = av[3] = 0x80808080u; }
    }
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
    if (any_flagged) {
        if (nm.flags & kPoison) { am[0] = am[1] = am[2] = am[3] = 0u; }
        if (nv.flags & kPoison) { av[0] = av[1] = av[2] = av[3] = 0u; }
    }
    if (__any((am[0] | am[1] | am[2] | am[3] | av[0] | av[1] | av[2] | av[3]) != 0u)) {
        if (pair) {  // the other moment's exact-path fields, from the partner lane
            const double oa = dpp64<kDppXor1>(own_amax), orr = dpp64<kDppXor1>(own_r);
            nm.amax = odd ? oa : own_amax;
            nm.r = odd ? orr : own_r;
            nv.amax = odd ? own_amax : oa;
            nv.r = odd ? own_r : orr;
        }
        OldGroup pm, pv;
        parked_groups(pm, pv);
        redo_ambiguous<FM>(am, cm, [&](int w) { return code_word(false, w); }, grad_word, pm, nm, lq_m, ct.lqm[0],
                           fm, c.b1, c.c1, false, cf);
        redo_ambiguous<FV>(av, cv, [&](int w) { return code_word(true, w); }, grad_word, pv, nv, lq_v, ct.lqm[1],
                           fv, c.b2, c.c2, true, cf);
    }
    if (any_flagged) {
        if (nm.flags & kPoison) { cm[0] = cm[1] = cm[2] = cm[3] = 0x7F7F7F7Fu; }
        if (nv.flags & kPoison) { cv[0] = cv[1] = cv[2] = cv[3] = 0x7F7F7F7Fu; }
    }

    // ---- store codes
    if (nvalid == kLaneElems) {
        *reinterpret_cast<gu32x4*>(MQ + e0) = u32x4{cm[0], cm[1], cm[2], cm[3]};
        *reinterpret_cast<gu32x4*>(VQ + e0) = u32x4{cv[0], cv[1], cv[2], cv[3]};
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < nvalid) {
                MQ[e0 + i] = (uint8_t)byte_of(cm[i >> 2], i & 3);
                VQ[e0 + i] = (uint8_t)byte_of(cv[i >> 2], i & 3);
            }
        }
    }
}


// Which tiles a step kernel launch covers.
constexpr int kPhaseFull = 1;     // tiles wholly inside their tensor
constexpr int kPhasePartial = 2;  // last tiles that end inside their tensor
// A step over one tensor. TAB (groups of 128 and more): the whole tiles with
// per-group tables, and nothing else; otherwise the tiles of `phases` on the
// direct path (group 16: every tile on the general path).
template <int FM, int FV, bool TAB, bool K1>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(TAB ? 4 : 3, TAB ? 4 : 3))) void step_single_kernel(
    TensorRef t, StepConsts c, int phases) {
    __shared__ typename StepLds<TAB>::Tables ct;
    __shared__ typename StepLds<TAB>::Wave wls[kWavesPerBlock];
    auto& wl = wls[threadIdx.x / kWave];
    if constexpr (TAB) fill_tab_tables<FM, FV>(ct, wls[0].setup, c.b1, c.b2);
    else fill_direct_tables<FM, FV>(ct, c.b1, c.b2);
    const int64_t full = t.n / kTile;
    const int64_t tiles = (t.n + kTile - 1) / kTile;
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    int64_t first = 0, last = 0;
    if (c.lg2_group >= 5) {
        if (phases & kPhaseFull) {
            for (int64_t tile = wave_id(); tile < full; tile += nw) {
                TileIn in;
                load_full_tile<TAB>(t, tile, c.lg2_group, in);
                step_tile<FM, FV, true, TAB, 0, K1>(t, tile, c, ct, wl, in);
            }
        }
        first = full;
        if (phases & kPhasePartial) last = tiles;
    } else {
        last = tiles;
    }
    if constexpr (!TAB) {
        // general path: the partial tile (every tile for group 16)
        for (int64_t tile = first + wave_id(); tile < last; tile += nw) {
            TileIn in;
            load_tile(t, tile, c.lg2_group, in);
            step_tile<FM, FV, false, false, 0, K1>(t, tile, c, ct, wl, in);
        }
    }
}

// The whole tiles of a multi-tensor launch. Each block takes one contiguous
// run of the global tile index space, its waves interleaved so that a block
// streams adjacent tiles together, and reads a tensor's descriptor once per
// run segment rather than once per tile (the descriptor table is too large
// for the scalar cache, and each of its reads sits on the path to the tile's
// loads). f(t, tile) gets the tensor and the tile's index within it.
template <typename F>
__device__ __forceinline__ void block_full_tiles(const TensorRef* __restrict__ ts, const int64_t* __restrict__ fb,
                                                 int count, int64_t full, F&& f) {
    const int64_t per = (full + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < full ? b0 + per : full;
    int64_t tile = b0 + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (tile >= b1) return;
    // the tensor holding `tile`: fb[lo] <= tile < fb[hi], fb[0] = 0, fb[count] = full
    int lo = 0, hi = count;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (fb[mid] <= tile) lo = mid;
        else hi = mid;
    }
    int cur = lo;
    while (tile < b1) {
        const int64_t tb = fb[cur], te = fb[cur + 1];
        if (tile >= te) {  // tile < full keeps cur + 1 <= count
            ++cur;
            continue;
        }
        const TensorRef t = ts[cur];
        const int64_t stop = te < b1 ? te : b1;
        for (; tile < stop; tile += kWavesPerBlock) f(t, tile - tb);
    }
}

// Multi-tensor: descriptors, the prefix of full tiles per tensor (count + 1
// entries) and the list of tensors with a partial last tile live in device
// workspace. The whole tiles are split into one contiguous run per block
// (block_full_tiles); then the partial tiles take the general path, one per
// wavefront. Phases and TAB as for the single kernel. Both the table and the
// direct variants run at four waves per SIMD (the direct one spills a few
// registers outside its tile loop, and its LDS still fits four blocks per
// CU): on the 13B list at G = 32 that is about 1 % faster than three waves.
template <int FM, int FV, bool TAB, int LG, bool K1>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void step_multi_kernel(
    const TensorRef* __restrict__ ts, const int64_t* __restrict__ full_begin, const int32_t* __restrict__ partial,
    int count, int n_partial, StepConsts c, int phases) {
    __shared__ typename StepLds<TAB>::Tables ct;
    __shared__ typename StepLds<TAB>::Wave wls[kWavesPerBlock];
    auto& wl = wls[threadIdx.x / kWave];
    if constexpr (TAB) fill_tab_tables<FM, FV>(ct, wls[0].setup, c.b1, c.b2);
    else fill_direct_tables<FM, FV>(ct, c.b1, c.b2);
    const int lg = LG ? LG : c.lg2_group;
    const int64_t full = full_begin[count];
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    if (phases & kPhaseFull) {
        if (lg >= 5) {
            block_full_tiles(ts, full_begin, count, full, [&](const TensorRef& t, int64_t tile) {
                TileIn in;
                load_full_tile<TAB>(t, tile, lg, in);
                step_tile<FM, FV, true, TAB, LG, K1>(t, tile, c, ct, wl, in);
            });
        } else if constexpr (!TAB) {
            block_full_tiles(ts, full_begin, count, full, [&](const TensorRef& t, int64_t tile) {
                TileIn in;
                load_tile(t, tile, lg, in);
                step_tile<FM, FV, false, false, LG, K1>(t, tile, c, ct, wl, in);
            });
        }
    }
    if constexpr (!TAB) {
        if (phases & kPhasePartial) {
            for (int64_t i = wave_id(); i < n_partial; i += nw) {
                const TensorRef& t = ts[partial[i]];
                const int64_t tile = t.n / kTile;
                TileIn in;
                load_tile(t, tile, lg, in);
                step_tile<FM, FV, false, false, LG, K1>(t, tile, c, ct, wl, in);
            }
        }
    }
}

// ------------------------------------------------------------------ codec kernels

// Quantize fp32 x to (q, s, k): the requantization half of the step.
template <int F>
__global__ __launch_bounds__(kBlock) void quantize_kernel(const float* __restrict__ x, int64_t n,
                                                          int lg2_group, int expand, uint8_t* q,
                                                          double* s, float* k) {
    __shared__ DirectTables ct;
    __shared__ Xfer xfs[kWavesPerBlock];
    fill_direct_tables<F, F>(ct, 1.0, 1.0);
    unsigned char* XA = reinterpret_cast<unsigned char*>(&xfs[threadIdx.x / kWave]);
    const int64_t tiles = (n + kTile - 1) / kTile;
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int lane = threadIdx.x & (kWave - 1);
    const int lpg = 1 << (lg2_group - 4);
    const FmtRT fr = fmt_rt<F>();
    const gfloat* X = gp(x);
    gu8* Q = gp(q);
    for (int64_t tile = wave_id(); tile < tiles; tile += nw) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
        const int64_t rem = n - e0;
        const int nvalid = rem <= 0 ? 0 : (rem >= kLaneElems ? kLaneElems : (int)rem);
        float xf[16];
        if ((tile + 1) * kTile <= n) {
            // a whole tile: loaded 4 elements per lane per quarter tile (each
            // wave load 1 KB), re-laid through LDS to the lane's own 16
            const int xl = lane_opaque();
            const gfloat* Xl = X + tile * kTile + (uint32_t)(4 * xl);
            const uint32_t ib = xfer_off(xl);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4*>(XA + ib + 4 * kXferRow * i) = *reinterpret_cast<const gf32x4*>(Xl + 256 * i);
            const uint32_t ob = xfer_off(4 * lane_opaque());
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(XA + ob + 16 * i);
                xf[4 * i] = v.x; xf[4 * i + 1] = v.y; xf[4 * i + 2] = v.z; xf[4 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) xf[i] = i < nvalid ? X[e0 + i] : 0.0f;
        }
        double amax = 0.0, amin = __builtin_inf();
        bool bad = false;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const double a = __builtin_fabs((double)xf[i]);
            bad |= !(a < __builtin_inf());
            amax = vmax(amax, a);
            amin = vmin(amin, a == 0.0 ? __builtin_inf() : a);
        }
        amax = group_max(amax, lpg);
        amin = group_min(amin, lpg);
        const bool poison = group_or(bad ? 1u : 0u, lpg) != 0u;
        double la_lo, lb_lo;
        const CoefPtr cf = coef_ptr(ct.coef);
        const double la = log2_stat(amax, la_lo), lb = log2_stat(amin, lb_lo);
        const NewGroup ng = new_group(amax, amin, la, la_lo, lb, lb_lo, poison, expand, fr);
        uint32_t cw[4], amb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cw[i] = fast_codes4<F>(xf + 4 * i, ng, amb[i]);
        if (ng.flags & kSlow) { amb[0] = amb[1] = amb[2] = amb[3] = 0x80808080u; }
        if (nvalid < kLaneElems) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t keep = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) keep |= (4 * i + b < nvalid) ? (0x80u << (8 * b)) : 0u;
                amb[i] &= keep;
            }
        }
        if (ng.flags & kPoison) { amb[0] = amb[1] = amb[2] = amb[3] = 0u; }
        while (__any((amb[0] | amb[1] | amb[2] | amb[3]) != 0u)) {
            if ((amb[0] | amb[1] | amb[2] | amb[3]) != 0u) {
                const int wi = amb[0] ? 0 : (amb[1] ? 1 : (amb[2] ? 2 : 3));
                const uint32_t aw = select4(wi, amb[0], amb[1], amb[2], amb[3]);
                const int bi = __builtin_ctz(aw) >> 3;
                const int e = 4 * wi + bi;
                float xe = xf[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) xe = (e == i) ? xf[i] : xe;
                const double xd = (double)xe;
                const uint32_t lo = byte_of(select4(wi, cw[0], cw[1], cw[2], cw[3]), bi) & 0x7Fu;
                const double mid = 0.5 * (value_of<F>(lo) + value_of<F>(lo + 1));
                const uint32_t code = (ng.flags & kSlow)
                                          ? exact_code_full<F>(xd, ng, cf)
                                          : ((__builtin_signbit(xd) ? 0x80u : 0u) |
                                             exact_mag(__builtin_fabs(xd), lo, ng, ct.lqm[0], mid, fr, cf));
                const uint32_t mask = ~(0xFFu << (8 * bi)), ins = code << (8 * bi);
                const uint32_t clear = ~(0x80u << (8 * bi));
                if (wi == 0) { cw[0] = (cw[0] & mask) | ins; amb[0] &= clear; }
                if (wi == 1) { cw[1] = (cw[1] & mask) | ins; amb[1] &= clear; }
                if (wi == 2) { cw[2] = (cw[2] & mask) | ins; amb[2] &= clear; }
                if (wi == 3) { cw[3] = (cw[3] & mask) | ins; amb[3] &= clear; }
            }
        }
        if (ng.flags & kPoison) { cw[0] = cw[1] = cw[2] = cw[3] = 0x7F7F7F7Fu; }
        if (nvalid == kLaneElems) {
            *reinterpret_cast<gu32x4*>(Q + e0) = u32x4{cw[0], cw[1], cw[2], cw[3]};
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i < nvalid) Q[e0 + i] = (uint8_t)byte_of(cw[i >> 2], i & 3);
        }
        if (nvalid > 0 && (lane & (lpg - 1)) == 0) {
            const int64_t gi = e0 >> lg2_group;
            gp(s)[gi] = ng.s;
            gp(k)[gi] = ng.k;
        }
    }
}

// 2^f on [-1/2, 1/2] to a relative error below 2^-28.5: the degree-6
// polynomial interpolating 2^f at the seven Chebyshev nodes of the interval,
// highest degree first. Used where the result is rounded to fp32 (the state
// dequantizer), so that the rounded value is within one fp32 ulp.
constexpr int kExp2ShortN = 7;
__device__ constexpr double kExp2ShortC[kExp2ShortN] = {
    0x1.443fffc87faa0p-13, 0x1.5f48c04f4eff9p-10, 0x1.3b2a1b7152d23p-7, 0x1.c6aecc669b99bp-5,
    0x1.ebfbe045f4d57p-3,  0x1.62e430d034700p-1,  1.0};

// Byte i of code word w dequantized and rounded to fp32:
// sign(q) 2^(LQ[q] r + a + a_lo) (LQ of the magnitude from lq[128], the sign
// from the code's sign bit, so that a zero keeps it and a NaN stays NaN).
__device__ __forceinline__ float dequant_f32(uint32_t w, int i, const OldGroup& og, const double* lq) {
    const uint32_t c = (w >> (8 * i)) & 0xFFu;
    const double u = __builtin_fma(lq[c & 0x7Fu], og.r, og.a);
    const double n = __builtin_rint(u);
    const double f = (u - n) + og.a_lo;
    double p = kExp2ShortC[0];
#pragma unroll
    for (int j = 1; j < kExp2ShortN; ++j) p = fma3(p, f, kExp2ShortC[j]);
    const float mag = (float)__builtin_amdgcn_ldexp(p, cvt_i32_sat(n));
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, mag) | ((c & 0x80u) << 24));
}

template <int F>
__global__ __launch_bounds__(kBlock) void dequantize_kernel(const uint8_t* __restrict__ q,
                                                            const double* __restrict__ s,
                                                            const float* __restrict__ k, int64_t n,
                                                            int lg2_group, float* __restrict__ x) {
    __shared__ double lq[128];
    __shared__ Xfer xfs[kWavesPerBlock];
    if (threadIdx.x < 128) lq[threadIdx.x] = lq_entry<F>((int)threadIdx.x);
    __syncthreads();
    unsigned char* XA = reinterpret_cast<unsigned char*>(&xfs[threadIdx.x / kWave]);
    const int64_t tiles = (n + kTile - 1) / kTile;
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int lane = threadIdx.x & (kWave - 1);
    const gu8* Q = gp(q);
    gfloat* X = gp(x);
    for (int64_t tile = wave_id(); tile < tiles; tile += nw) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
        const int64_t rem = n - e0;
        const int nvalid = rem <= 0 ? 0 : (rem >= kLaneElems ? kLaneElems : (int)rem);
        if (nvalid == 0) continue;
        const int64_t gi = e0 >> lg2_group;
        const double sg = gp(s)[gi];
        const float kg = gp(k)[gi];
        const OldGroup og = old_group(sg, kg, Fmt<F>::LOG2_FPMAX, Fmt<F>::LOG2_FPMAX_LO);
        // k = 1: the plain product |q| s, rounded to fp32 (as the definition)
        const bool k1 = kg == 1.0f;
        auto k1_value = [&](uint32_t w, int i) { return (float)(code_value<F>(w, i) * sg); };
        if ((tile + 1) * kTile <= n) {
            // a whole tile: the lane's 16 values re-laid through LDS and stored
            // 4 per lane per quarter tile (each wave store 1 KB)
            const u32x4 a = *reinterpret_cast<const gu32x4*>(Q + e0);
            const uint32_t w[4] = {a.x, a.y, a.z, a.w};
            float out[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) out[i] = dequant_f32(w[i >> 2], i & 3, og, lq);
            if (__builtin_expect(__any(k1), 0)) {
                if (k1) {
#pragma unroll 1
                    for (int i = 0; i < 16; ++i) out[i] = k1_value(w[i >> 2], i & 3);
                }
            }
            const uint32_t ob = xfer_off(4 * lane_opaque());
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4*>(XA + ob + 16 * i) = f32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
            const int xl = lane_opaque();
            gfloat* Xl = X + tile * kTile + (uint32_t)(4 * xl);
            const uint32_t ib = xfer_off(xl);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<gf32x4*>(Xl + 256 * i) = *reinterpret_cast<const f32x4*>(XA + ib + 4 * kXferRow * i);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i < nvalid) X[e0 + i] = k1 ? k1_value(Q[e0 + i], 0) : dequant_f32(Q[e0 + i], 0, og, lq);
        }
    }
}

template <int F>
__global__ __launch_bounds__(kBlock) void encode_kernel(const float* __restrict__ y, int64_t n,
                                                        uint8_t* __restrict__ q) {
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
            lo[b] = __builtin_copysignf(__builtin_fminf(a * (1.0f - kAmbiguity), Fmt<F>::FPMAX_F), v[b]);
            hi[b] = __builtin_fminf(a * (1.0f + kAmbiguity), Fmt<F>::FPMAX_F);
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

// Many more blocks than fit on a CU at once (3 or 4 here): blocks are handed to CUs
// as earlier ones finish, which evens out the load across CUs and XCDs (some
// run several per cent slower than others: with exactly one resident round of
// blocks the 13B step takes 10 % longer); beyond a few hundred per CU each
// block's table set-up starts to cost more than the finer balance gains.
constexpr int kStepBlocksPerCU = 256;
// Small launches would otherwise give each wave a single tile, so that each
// block's table set-up (paid once per block) weighs as much as a third of its
// tiles' work: there every wave gets at least this many tiles, as long as
// that still leaves four blocks per CU (else one tile per wave). On the
// GPT-2-small list (121 k tiles) 4 or 6 take 13 % off the step, 2 and 8 a
// little less, 16 and 32 half as much (coarser balance across the CUs).
constexpr int kStepMinTilesPerWave = 4;
inline unsigned step_grid(int64_t waves) {
    const unsigned most = grid_for(waves, kStepBlocksPerCU);
    const int64_t per_block = (int64_t)kWavesPerBlock * kStepMinTilesPerWave;
    const int64_t thin = (waves + per_block - 1) / per_block;
    const unsigned fill = grid_for(waves, 4);
    const int64_t least = thin > (int64_t)fill ? thin : (int64_t)fill;
    return (int64_t)most < least ? most : (unsigned)least;
}

// Groups of 128 and more: the whole tiles run in the table kernel, then a
// direct-path launch covers any partial tiles. Otherwise one direct-path launch.
template <int FM, int FV, bool K1>
void launch_single_k1(const TensorRef& t, const StepConsts& c, hipStream_t st) {
    const int64_t tiles = (t.n + kTile - 1) / kTile, full = t.n / kTile;
    if (c.lg2_group >= 7) {
        if (full > 0)
            hipLaunchKernelGGL((step_single_kernel<FM, FV, true, K1>), dim3(step_grid(full)),
                               dim3(kBlock), 0, st, t, c, kPhaseFull);
        if (tiles > full)
            hipLaunchKernelGGL((step_single_kernel<FM, FV, false, K1>), dim3(1), dim3(kBlock), 0, st, t, c,
                               kPhasePartial);
        return;
    }
    hipLaunchKernelGGL((step_single_kernel<FM, FV, false, K1>), dim3(step_grid(tiles)),
                       dim3(kBlock), 0, st, t, c, kPhaseFull | kPhasePartial);
}
// Without expansion for either moment every group is stored with k = 1 after
// the first step: the K1 kernels, which treat whole waves of such groups on
// a path of their own.
template <int FM, int FV>
void launch_single(const TensorRef& t, const StepConsts& c, hipStream_t st) {
    if (!c.expand_m && !c.expand_v) launch_single_k1<FM, FV, true>(t, c, st);
    else launch_single_k1<FM, FV, false>(t, c, st);
}

// The multi-tensor kernels are specialized on the group size (groups of
// 128 .. 1024 in the table kernel, 16 .. 64 in the direct one); partial tiles
// of groups of 128 and more take the direct kernel with the size at run time.
template <int FM, int FV, bool TAB, int LG>
void launch_multi_lg(const TensorRef* ts, const int64_t* fb, const int32_t* partial, int count, int n_partial,
                     int64_t waves, const StepConsts& c, int phases, hipStream_t st) {
    // K1 kernels for launches without expansion (see launch_single)
    if (!c.expand_m && !c.expand_v)
        hipLaunchKernelGGL((step_multi_kernel<FM, FV, TAB, LG, true>), dim3(step_grid(waves)),
                           dim3(kBlock), 0, st, ts, fb, partial, count, n_partial, c, phases);
    else
        hipLaunchKernelGGL((step_multi_kernel<FM, FV, TAB, LG, false>), dim3(step_grid(waves)),
                           dim3(kBlock), 0, st, ts, fb, partial, count, n_partial, c, phases);
}

template <int FM, int FV>
void launch_multi(const TensorRef* ts, const int64_t* fb, const int32_t* partial, int count, int n_partial,
                  int64_t tiles, int64_t full, const StepConsts& c, hipStream_t st) {
    const int both = kPhaseFull | kPhasePartial;
    switch (c.lg2_group) {
        case 4: launch_multi_lg<FM, FV, false, 4>(ts, fb, partial, count, n_partial, tiles, c, both, st); return;
        case 5: launch_multi_lg<FM, FV, false, 5>(ts, fb, partial, count, n_partial, tiles, c, both, st); return;
        case 6: launch_multi_lg<FM, FV, false, 6>(ts, fb, partial, count, n_partial, tiles, c, both, st); return;
        default: break;
    }
    if (full > 0) {
        switch (c.lg2_group) {
            case 7: launch_multi_lg<FM, FV, true, 7>(ts, fb, partial, count, n_partial, full, c, kPhaseFull, st); break;
            case 8: launch_multi_lg<FM, FV, true, 8>(ts, fb, partial, count, n_partial, full, c, kPhaseFull, st); break;
            case 9: launch_multi_lg<FM, FV, true, 9>(ts, fb, partial, count, n_partial, full, c, kPhaseFull, st); break;
            default: launch_multi_lg<FM, FV, true, 10>(ts, fb, partial, count, n_partial, full, c, kPhaseFull, st); break;
        }
    }
    if (n_partial > 0)
        launch_multi_lg<FM, FV, false, 0>(ts, fb, partial, count, n_partial, n_partial, c, kPhasePartial, st);
}

}  // namespace

// ------------------------------------------------------------------ static plan tables

// The plan tables of coat_fp8_adamw_step_multi_static: the same layout as a
// plan workspace (descriptors, full-tile prefix, partial-tile list, each
// section 256-byte aligned), sized for COAT_STATIC_MAX_TENSORS tensors. Each
// GPU the library runs on holds its own copy until the process ends. In host
// code the name is only a stand-in: kernels get the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kStaticLayout.total];

namespace {

// Plan tables reach device memory (the static array, or a caller's
// workspace) through kernel arguments (captured at launch, so the host side
// needs no staging memory and no synchronization).
__global__ __launch_bounds__(64) void arg_copy_kernel(ArgChunk chunk, uint32_t bytes, unsigned char* dst) {
    for (uint32_t i = threadIdx.x * 16u; i < bytes; i += 64u * 16u)
        *reinterpret_cast<u32x4*>(dst + i) = *reinterpret_cast<const u32x4*>(chunk.data + i);
}

// ChunkWriter's sink for device memory at `base`: one copy launch per chunk.
struct LaunchSink {
    unsigned char* base;
    hipStream_t st;
    bool operator()(const ArgChunk& chunk, uint32_t bytes, size_t offset) {
        hipLaunchKernelGGL(arg_copy_kernel, dim3(1), dim3(64), 0, st, chunk, bytes, base + offset);
        return hipGetLastError() == hipSuccess;
    }
};

// The device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int static_tables(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return COAT_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return COAT_EHIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return COAT_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

int coat_abi_version(void) { return 102; }

const char* coat_strerror(int status) {
    switch (status) {
        case COAT_OK: return "ok";
        case COAT_EINVAL: return "invalid argument";
        case COAT_EALIGN: return "pointer not aligned as required (16 bytes for element arrays)";
        case COAT_EHIP: return "HIP runtime error at launch";
        case COAT_ERANGE: return "more tensors than the library's static plan table holds (COAT_STATIC_MAX_TENSORS)";
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

// Workspace layout: plan_layout (descriptors, the full-tile prefix, the
// indices of tensors with a partial last tile, each section 256-byte aligned).
size_t coat_multi_workspace_bytes(int32_t count) {
    if (count < 0) return 0;
    return plan_layout((size_t)count).total;
}

int coat_multi_plan_init(coat_multi_plan* plan, const coat_tensor* tensors, int32_t count, void* workspace,
                         size_t workspace_bytes, coat_stream_t stream) {
    if (!plan || count < 0 || (count > 0 && !tensors)) return COAT_EINVAL;
    if (!workspace || workspace_bytes < coat_multi_workspace_bytes(count)) return COAT_EINVAL;
    if (!aligned(workspace, 256)) return COAT_EALIGN;
    PlanSummary sum;
    const int rc = scan_tensors(tensors, count, &sum);
    if (rc) return rc;
    // the tables travel in the arguments of small copy launches on `stream`:
    // no host staging buffer, no wait
    LaunchSink sink{static_cast<unsigned char*>(workspace), reinterpret_cast<hipStream_t>(stream)};
    if (!write_plan_tables(tensors, count, plan_layout((size_t)count), sink)) return COAT_EHIP;
    plan->workspace = workspace;
    plan->count = count;
    plan->tiles = sum.tiles;
    plan->n_total = sum.n_total;
    plan->n_partial = sum.n_partial;
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
    const PlanLayout L = plan_layout((size_t)plan->count);
    const char* ws = static_cast<const char*>(plan->workspace);
    const TensorRef* dts = reinterpret_cast<const TensorRef*>(ws + L.desc);
    const int64_t* dfb = reinterpret_cast<const int64_t*>(ws + L.fb);
    const int32_t* dpt = reinterpret_cast<const int32_t*>(ws + L.partial);
    const int fm = fmt_m & 0xFF, fv = fmt_v & 0xFF;
    const int count = plan->count, np = plan->n_partial;
    const int64_t tiles = plan->tiles, full = plan->tiles - plan->n_partial;
    if (fm == COAT_FMT_E4M3 && fv == COAT_FMT_E4M3) launch_multi<COAT_FMT_E4M3, COAT_FMT_E4M3>(dts, dfb, dpt, count, np, tiles, full, c, st);
    else if (fm == COAT_FMT_E4M3) launch_multi<COAT_FMT_E4M3, COAT_FMT_E5M2>(dts, dfb, dpt, count, np, tiles, full, c, st);
    else if (fv == COAT_FMT_E4M3) launch_multi<COAT_FMT_E5M2, COAT_FMT_E4M3>(dts, dfb, dpt, count, np, tiles, full, c, st);
    else launch_multi<COAT_FMT_E5M2, COAT_FMT_E5M2>(dts, dfb, dpt, count, np, tiles, full, c, st);
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

int coat_fp8_adamw_step_multi_static(const coat_tensor* tensors, int32_t count, int32_t group, int32_t fmt_m,
                                     int32_t fmt_v, float lr, float beta1, float beta2, float eps,
                                     float weight_decay, int64_t step, coat_stream_t stream) {
    if (count < 0 || (count > 0 && !tensors)) return COAT_EINVAL;
    if (count > COAT_STATIC_MAX_TENSORS) return COAT_ERANGE;
    StepConsts c;
    int rc = make_consts(group, fmt_m, fmt_v, lr, beta1, beta2, eps, weight_decay, step, &c);
    if (rc) return rc;
    PlanSummary sum;
    rc = scan_tensors(tensors, count, &sum);
    if (rc) return rc;
    if (sum.tiles == 0) return COAT_OK;
    void* base = nullptr;
    rc = static_tables(&base);
    if (rc) return rc;
    unsigned char* ws = static_cast<unsigned char*>(base);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // every byte the step reads is written here first; nothing needs clearing
    LaunchSink sink{ws, st};
    if (!write_plan_tables(tensors, count, kStaticLayout, sink)) return COAT_EHIP;
    const TensorRef* dts = reinterpret_cast<const TensorRef*>(ws + kStaticLayout.desc);
    const int64_t* dfb = reinterpret_cast<const int64_t*>(ws + kStaticLayout.fb);
    const int32_t* dpt = reinterpret_cast<const int32_t*>(ws + kStaticLayout.partial);
    const int n_partial = sum.n_partial;
    const int64_t tiles = sum.tiles, full = sum.full;
    const int fm = fmt_m & 0xFF, fv = fmt_v & 0xFF;
    if (fm == COAT_FMT_E4M3 && fv == COAT_FMT_E4M3) launch_multi<COAT_FMT_E4M3, COAT_FMT_E4M3>(dts, dfb, dpt, count, n_partial, tiles, full, c, st);
    else if (fm == COAT_FMT_E4M3) launch_multi<COAT_FMT_E4M3, COAT_FMT_E5M2>(dts, dfb, dpt, count, n_partial, tiles, full, c, st);
    else if (fv == COAT_FMT_E4M3) launch_multi<COAT_FMT_E5M2, COAT_FMT_E4M3>(dts, dfb, dpt, count, n_partial, tiles, full, c, st);
    else launch_multi<COAT_FMT_E5M2, COAT_FMT_E5M2>(dts, dfb, dpt, count, n_partial, tiles, full, c, st);
    return launch_status();
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
