// Definitions shared by the HIP sources of the library: vector and address
// space types, the tiling constants, the FP8 formats (OCP E4M3FN and E5M2; bit
// layouts per the FP8 guide on maplevalley.com.cn, section "format choice"),
// cross-lane moves, the exact FP8 encode and decode, and the launch helpers
// (argument checks and plan tables are in coat_host.h).
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "coat_fp8.h"
#include "coat_host.h"

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) uint16_t gu16;
typedef __attribute__((address_space(1))) uint32_t gu32;
typedef __attribute__((address_space(1))) uint8_t gu8;
typedef __attribute__((address_space(1))) double gf64;
typedef __attribute__((address_space(1))) f32x4 gf32x4;
typedef __attribute__((address_space(1))) u32x4 gu32x4;

constexpr int kWave = 64;
constexpr int kLaneElems = 16;
constexpr int kTile = kWave * kLaneElems;  // elements per wavefront tile
constexpr int kBlock = 256;                // 4 wavefronts
constexpr int kWavesPerBlock = kBlock / kWave;

// Relative half-width of the window around an FP8 rounding midpoint inside
// which a converted value is decided exactly (plain encoding, no transcendentals).
constexpr float kAmbiguity = 0x1p-15f;

// Window of the requantization fast path, per group: w = W0 + W1 k relative.
// The fast path forms y = 2^(k log2(|x| / amax) + log2 fpmax) in fp32. Its
// error: |x| / amax carries three fp32 roundings (<= 3 * 2^-24 relative, k
// times that in y); v_log_f32 is accurate to about an ulp of its result, whose
// magnitude times k stays below log2 R_fp8 (17.8 for E4M3, 31.8 for E5M2), so
// k times that error stays below log2(R_fp8) * 2^-23; the fma adds half an
// ulp of |z| <= 16; v_exp_f32 about an ulp. In total below ln 2 * (2^-23
// log2 R_fp8 + 2^-20 + k * 2.6e-7) + 1.2e-7, i.e. 2.2e-6 + 1.8e-7 k (E4M3)
// and 3.4e-6 + 1.8e-7 k (E5M2); measured maxima on gfx950 over 1.6e7 samples
// per k sit at 55-70 % of that. W0 and W1 take twice the bound.
constexpr float kAmbW1 = 3.6e-7f;

template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gp(T* p) {
    return (__attribute__((address_space(1))) T*)p;
}

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
    static constexpr double LOG2_FPMAX_LO = 0x1.b332ac903a414p-52;  // its rounding error
    static constexpr float LOG2_FPMAX_F = 0x1.19d5dap+3f;
    static constexpr float AMB_W0 = 4.4e-6f;  // fast-path window, see kAmbW1
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
    static constexpr double LOG2_FPMAX_LO = 0x1.b332ac903a414p-52;  // its rounding error
    static constexpr float LOG2_FPMAX_F = 0x1.f9d5dap+3f;
    static constexpr float AMB_W0 = 6.8e-6f;  // fast-path window, see kAmbW1
    static constexpr double LOG2_RF = 0x1.fceaecfea8086p+4;     // log2(57344 / 2^-16)
    __device__ static bool is_nan(int c) { return c > 0x7C; }
    __device__ static bool is_inf(int c) { return c == 0x7C; }
};

// Per-lane format constants, for code that serves both moments at once.
struct FmtRT {
    double fpmax, log2_fpmax, log2_fpmax_lo, log2_rf;
    float fpmax_f, log2_fpmax_f, amb_w0;
};
template <int F>
__device__ __forceinline__ FmtRT fmt_rt() {
    using T = Fmt<F>;
    return FmtRT{T::FPMAX, T::LOG2_FPMAX, T::LOG2_FPMAX_LO, T::LOG2_RF, T::FPMAX_F, T::LOG2_FPMAX_F, T::AMB_W0};
}

// ------------------------------------------------------------------ cross-lane

// Value of lane (lane ^ 1), (lane ^ 2), ... via DPP within a row of 16.
// Every pattern used here reads a valid lane of the same row with all rows
// and banks enabled, so no lane keeps its old value: the move has no "old"
// operand (an update_dpp with old = 0 costs a v_mov per move to set it).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp32<CTRL>((uint32_t)b), hi = dpp32<CTRL>((uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within 16

__device__ __forceinline__ double xlane64(double v, int d) {
    switch (d) {
        case 1: return dpp64<kDppXor1>(v);
        case 2: return dpp64<kDppXor2>(v);
        case 4: return dpp64<kDppHalfMirror>(v);
        case 8: return dpp64<kDppMirror>(v);
        default: return __shfl_xor(v, d, kWave);
    }
}
__device__ __forceinline__ uint32_t xlane32(uint32_t v, int d) {
    switch (d) {
        case 1: return dpp32<kDppXor1>(v);
        case 2: return dpp32<kDppXor2>(v);
        case 4: return dpp32<kDppHalfMirror>(v);
        case 8: return dpp32<kDppMirror>(v);
        default: return (uint32_t)__shfl_xor((int)v, d, kWave);
    }
}

// OR over the `lanes` lanes (a power of two, aligned) owning a group.
__device__ __forceinline__ uint32_t group_or(uint32_t v, int lanes) {
    for (int d = 1; d < lanes; d <<= 1) v |= xlane32(v, d);
    return v;
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

// Exact value of a magnitude code (finite codes only).
template <int F>
__device__ double value_of(int c) {
    using T = Fmt<F>;
    const int e = c >> T::MB, m = c & ((1 << T::MB) - 1);
    return e ? __builtin_amdgcn_ldexp(1.0 + (double)m / (double)(1 << T::MB), e - T::BIAS)
             : __builtin_amdgcn_ldexp((double)m, T::EMIN - T::MB);
}

// Exact value of an FP8 code.
template <int F>
__device__ float decode_value(uint32_t code) {
    using T = Fmt<F>;
    const int c = code & 0x7F;
    float mag;
    if (T::is_nan(c)) mag = __builtin_nanf("");
    else if (T::is_inf(c)) mag = __builtin_inff();
    else mag = (float)value_of<F>(c);
    return (code & 0x80) ? -mag : mag;
}

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xFFu; }

__device__ __forceinline__ int64_t wave_id() {
    return (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

// ------------------------------------------------------------------ host side

inline int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

// Blocks for a grid-stride launch over `waves` wavefront tiles: enough to fill
// every CU `per_cu` times, never more than there is work.
inline unsigned grid_for(int64_t waves, int per_cu) {
    const int64_t want = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t cap = (int64_t)device_cus() * per_cu;
    int64_t b = want < cap ? want : cap;
    return (unsigned)(b < 1 ? 1 : b);
}

inline int launch_status() { return hipGetLastError() == hipSuccess ? COAT_OK : COAT_EHIP; }

}  // namespace
