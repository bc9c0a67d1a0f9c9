// HIP (gfx950) FP8 activation codec: bf16 values to E4M3 / E5M2 codes with
// one fp32 scale per tensor or per group of G consecutive values, and back.
#include "coat_common.h"

namespace {

// ------------------------------------------------------------------ activation codec
//
// Article, section "Solution: mixed-granularity FP8 precision flow": layer
// inputs are kept in FP8 for the backward pass, with a quantization
// granularity that differs between layers. Plain absmax scaling of bf16
// values with one fp32 scale per tensor or per group of G consecutive values:
// s = RN32(amax / fpmax), code = encode(RN32(x / s)) (the sign alone when
// s = 0), value = RN_bf16(RN32(decode(code) s)); a tensor or group holding a
// NaN or Inf gets s = NaN and every code 0x7F.
//
// RN32(x / s) without a division per value: x has at most 8 significant bits
// and s at most 24, so a quotient that is not an fp32 number lies at least
// 2^-49 (relative) from every midpoint between fp32 neighbours (the distance
// is a nonzero multiple of 2^(e-24) / s's integer significand in the binade
// [2^e, 2^(e+1)), likewise in the subnormal range), while x * RN64(1 / s),
// rounded to fp64, is within 2^-52 of it. Rounding that product to fp32 thus
// gives RN32(x / s) exactly; the hardware converts round it to the FP8 grid,
// nearest with ties to even, after a clamp to the largest finite magnitude.

// bf16 magnitude bits of 16 values (two 16-byte words per 8 values) -> max.
__device__ __forceinline__ uint32_t bf16_absmax_bits(const uint32_t (&w)[8]) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t a = w[i] & 0x7FFF7FFFu;
        const uint32_t lo = a & 0xFFFFu, hi = a >> 16;
        m = m > lo ? m : lo;
        m = m > hi ? m : hi;
    }
    return m;
}

__device__ __forceinline__ uint32_t group_umax(uint32_t v, int lanes) {
    for (int d = 1; d < lanes; d <<= 1) {
        const uint32_t o = xlane32(v, d);
        v = v > o ? v : o;
    }
    return v;
}

// Codes of the 16 bf16 values in w (value i in half i & 1 of word i >> 1) for
// a group with magnitude bits `amax_bits`; returns the four code words.
template <int F>
__device__ __forceinline__ void act_codes16(const uint32_t (&w)[8], uint32_t amax_bits, uint32_t (&out)[4]) {
    using T = Fmt<F>;
    if (amax_bits >= 0x7F80u) {  // Inf or NaN in the group
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = 0x7F7F7F7Fu;
        return;
    }
    const float amax = __builtin_bit_cast(float, amax_bits << 16);
    const float sc = (float)((double)amax / T::FPMAX);
    if (sc == 0.0f) {  // all zero: the sign alone
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t c = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int j = 4 * i + b;
                c |= ((w[j >> 1] >> (16 * (j & 1) + 15)) & 1u) << (8 * b + 7);
            }
            out[i] = c;
        }
        return;
    }
    const double r = 1.0 / (double)sc;  // RN64(1 / s); fp64 holds it for a subnormal s too
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float y[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int j = 4 * i + b;
            const float x = __builtin_bit_cast(float, (j & 1) ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16));
            const float q = (float)((double)x * r);  // RN32(x / s)
            y[b] = __builtin_fminf(__builtin_fmaxf(q, -T::FPMAX_F), T::FPMAX_F);
        }
        uint32_t c = cvt_pk<F, false>(y[0], y[1], 0u);
        out[i] = cvt_pk<F, true>(y[2], y[3], c);
    }
}

// Loads the lane's 16 bf16 values of a tile (zeros past n).
__device__ __forceinline__ void act_load16(const uint16_t* x, int64_t n, int64_t e0, uint32_t (&w)[8]) {
    if (e0 + kLaneElems <= n) {
        const gu32x4* p = reinterpret_cast<const gu32x4*>(gp(x) + e0);
        const u32x4 a = p[0], b = p[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (e0 + i < n) w[i >> 1] |= (uint32_t)gp(x)[e0 + i] << (16 * (i & 1));
    }
}

__device__ __forceinline__ void act_store16(uint8_t* q, int64_t n, int64_t e0, const uint32_t (&c)[4]) {
    if (e0 + kLaneElems <= n) {
        *reinterpret_cast<gu32x4*>(gp(q) + e0) = u32x4{c[0], c[1], c[2], c[3]};
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (e0 + i < n) gp(q)[e0 + i] = (uint8_t)byte_of(c[i >> 2], i & 3);
    }
}

// Per group of G = 2^lg2_group (16 .. 1024): a group spans G / 16 lanes.
template <int F>
__global__ __launch_bounds__(kBlock) void act_quantize_group_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                    int lg2_group, uint8_t* __restrict__ q,
                                                                    float* __restrict__ s) {
    const int64_t tiles = (n + kTile - 1) / kTile;
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int lane = threadIdx.x & (kWave - 1);
    const int lpg = 1 << (lg2_group - 4);
    auto code = [&](int64_t e0, const uint32_t (&w)[8]) {
        const uint32_t am = group_umax(bf16_absmax_bits(w), lpg);
        uint32_t c[4];
        act_codes16<F>(w, am, c);
        act_store16(q, n, e0, c);
        if ((lane & (lpg - 1)) == 0 && e0 < n) {
            const float amax = __builtin_bit_cast(float, am << 16);
            gp(s)[e0 >> lg2_group] = am >= 0x7F80u ? __builtin_nanf("") : (float)((double)amax / Fmt<F>::FPMAX);
        }
    };
    // two tiles per iteration: both tiles' loads are in flight together
    int64_t tile = wave_id();
    for (; tile + nw < tiles; tile += 2 * nw) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems, e1 = e0 + nw * kTile;
        uint32_t w0[8], w1[8];
        act_load16(x, n, e0, w0);
        act_load16(x, n, e1, w1);
        code(e0, w0);
        code(e1, w1);
    }
    if (tile < tiles) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
        uint32_t w[8];
        act_load16(x, n, e0, w);
        code(e0, w);
    }
}

// Per tensor: acc[0] = 0, then the magnitude bits' maximum, then the codes,
// then acc[0] = the scale (acc is the caller's scale word).
__global__ void act_zero_kernel(uint32_t* acc) {
    if (threadIdx.x == 0) gp(acc)[0] = 0u;
}

// One atomic per block (atomics on one word serialize); four tiles per
// iteration keep more loads in flight per wavefront.
__global__ __launch_bounds__(kBlock) void act_absmax_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                            uint32_t* acc) {
    __shared__ uint32_t wmax[kWavesPerBlock];
    const int64_t tiles = (n + kTile - 1) / kTile;
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t off = (int64_t)lane * kLaneElems;
    uint32_t m = 0;
    int64_t tile = wave_id();
    for (; tile + 3 * nw < tiles; tile += 4 * nw) {
        uint32_t w0[8], w1[8], w2[8], w3[8];
        act_load16(x, n, tile * kTile + off, w0);
        act_load16(x, n, (tile + nw) * kTile + off, w1);
        act_load16(x, n, (tile + 2 * nw) * kTile + off, w2);
        act_load16(x, n, (tile + 3 * nw) * kTile + off, w3);
        const uint32_t a = bf16_absmax_bits(w0), b = bf16_absmax_bits(w1);
        const uint32_t c = bf16_absmax_bits(w2), d = bf16_absmax_bits(w3);
        const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
        const uint32_t v = ab > cd ? ab : cd;
        m = m > v ? m : v;
    }
    for (; tile < tiles; tile += nw) {
        uint32_t w[8];
        act_load16(x, n, tile * kTile + off, w);
        const uint32_t v = bf16_absmax_bits(w);
        m = m > v ? m : v;
    }
    m = group_umax(m, kWave);
    if (lane == 0) wmax[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t bm = 0;
        for (int i = 0; i < kWavesPerBlock; ++i) bm = bm > wmax[i] ? bm : wmax[i];
        atomicMax(acc, bm);
    }
}

template <int F>
__global__ __launch_bounds__(kBlock) void act_quantize_tensor_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                     const uint32_t* acc, uint8_t* __restrict__ q) {
    const int64_t tiles = (n + kTile - 1) / kTile;
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t am = __builtin_amdgcn_readfirstlane(gp(acc)[0]);
    auto code = [&](int64_t e0, const uint32_t (&w)[8]) {
        uint32_t c[4];
        act_codes16<F>(w, am, c);
        act_store16(q, n, e0, c);
    };
    // two tiles per iteration: both tiles' loads are in flight together
    int64_t tile = wave_id();
    for (; tile + nw < tiles; tile += 2 * nw) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems, e1 = e0 + nw * kTile;
        uint32_t w0[8], w1[8];
        act_load16(x, n, e0, w0);
        act_load16(x, n, e1, w1);
        code(e0, w0);
        code(e1, w1);
    }
    if (tile < tiles) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
        uint32_t w[8];
        act_load16(x, n, e0, w);
        code(e0, w);
    }
}

template <int F>
__global__ void act_finalize_kernel(uint32_t* acc) {
    if (threadIdx.x == 0) {
        const uint32_t am = gp(acc)[0];
        const float amax = __builtin_bit_cast(float, am << 16);
        const float sc = am >= 0x7F80u ? __builtin_nanf("") : (float)((double)amax / Fmt<F>::FPMAX);
        gp(acc)[0] = __builtin_bit_cast(uint32_t, sc);
    }
}

// Codes and scales back to bf16: RN_bf16(decode(code) * s) with the fp32
// product. lg2_group < 0: one scale for the tensor.
// Exact value of byte B of a code word, by the hardware OCP converts.
template <int F, int B>
__device__ __forceinline__ float fp8_byte_value(uint32_t w) {
    if constexpr (F == COAT_FMT_E4M3)
        return __builtin_amdgcn_cvt_f32_fp8((int)w, B);
    else
        return __builtin_amdgcn_cvt_f32_bf8((int)w, B);
}

template <int F>
__global__ __launch_bounds__(kBlock) void act_dequantize_kernel(const uint8_t* __restrict__ q,
                                                                const float* __restrict__ s, int64_t n,
                                                                int lg2_group, uint16_t* __restrict__ x) {
    const int64_t tiles = (n + kTile - 1) / kTile;
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int lane = threadIdx.x & (kWave - 1);
    auto load = [&](int64_t e0, uint32_t (&c)[4]) {
        if (e0 + kLaneElems <= n) {
            const u32x4 v = *reinterpret_cast<const gu32x4*>(gp(q) + e0);
            c[0] = v.x; c[1] = v.y; c[2] = v.z; c[3] = v.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) c[i] = 0u;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (e0 + i < n) c[i >> 2] |= (uint32_t)gp(q)[e0 + i] << (8 * (i & 3));
        }
    };
    auto decode = [&](int64_t e0, const uint32_t (&c)[4]) {
        if (e0 >= n) return;
        const float sc = gp(s)[lg2_group < 0 ? 0 : (e0 >> lg2_group)];
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v0 = fp8_byte_value<F, 0>(c[i]) * sc, v1 = fp8_byte_value<F, 1>(c[i]) * sc;
            const float v2 = fp8_byte_value<F, 2>(c[i]) * sc, v3 = fp8_byte_value<F, 3>(c[i]) * sc;
            o[2 * i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v0) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v1) << 16);
            o[2 * i + 1] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v2) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v3) << 16);
        }
        if (e0 + kLaneElems <= n) {
            gu32x4* p = reinterpret_cast<gu32x4*>(gp(x) + e0);
            p[0] = u32x4{o[0], o[1], o[2], o[3]};
            p[1] = u32x4{o[4], o[5], o[6], o[7]};
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (e0 + i < n) gp(x)[e0 + i] = (uint16_t)(o[i >> 1] >> (16 * (i & 1)));
        }
    };
    // two tiles per iteration: both tiles' loads are in flight together
    int64_t tile = wave_id();
    for (; tile + nw < tiles; tile += 2 * nw) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems, e1 = e0 + nw * kTile;
        uint32_t c0[4], c1[4];
        load(e0, c0);
        load(e1, c1);
        decode(e0, c0);
        decode(e1, c1);
    }
    if (tile < tiles) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
        uint32_t c[4];
        load(e0, c);
        decode(e0, c);
    }
}

}  // namespace

// ====================================================================== C ABI

// Blocks per CU of the coding passes (capped by the work). These kernels are
// short (about 0.1 ms on a 16384 x 13824 matrix): with many more blocks than
// fit at once each wavefront codes one or two tile pairs and the launch ends
// evenly across CUs; on that matrix 128 per CU took 11-21 % off the group
// quantizer and the dequantizer against 16 (256 and more: no further gain).
// The per-tensor maximum pass is insensitive to this (1 to 16 per CU within
// 2 %) and keeps 2.
constexpr int kActBlocksPerCU = 128;
constexpr int kActMaxBlocksPerCU = 2;

extern "C" {

int coat_fp8_act_quantize(const uint16_t* x, int64_t n, int32_t group, int32_t fmt, uint8_t* q, float* scale,
                          coat_stream_t stream) {
    const int lg = group == 0 ? 0 : lg2_group_of(group);
    if (n < 0 || lg < 0 || (fmt != COAT_FMT_E4M3 && fmt != COAT_FMT_E5M2)) return COAT_EINVAL;
    if (n == 0) return COAT_OK;
    if (!x || !q || !scale) return COAT_EINVAL;
    if (!aligned16(x) || !aligned16(q) || !aligned(scale, 4)) return COAT_EALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t tiles = (n + kTile - 1) / kTile;
    const unsigned grid = grid_for(tiles, kActBlocksPerCU);
    const bool e4 = fmt == COAT_FMT_E4M3;
    if (group != 0) {
        if (e4) hipLaunchKernelGGL(act_quantize_group_kernel<COAT_FMT_E4M3>, dim3(grid), dim3(kBlock), 0, st, x, n, lg, q, scale);
        else hipLaunchKernelGGL(act_quantize_group_kernel<COAT_FMT_E5M2>, dim3(grid), dim3(kBlock), 0, st, x, n, lg, q, scale);
        return launch_status();
    }
    uint32_t* acc = reinterpret_cast<uint32_t*>(scale);
    hipLaunchKernelGGL(act_zero_kernel, dim3(1), dim3(kWave), 0, st, acc);
    hipLaunchKernelGGL(act_absmax_kernel, dim3(grid_for(tiles, kActMaxBlocksPerCU)), dim3(kBlock), 0, st, x, n, acc);
    if (e4) {
        hipLaunchKernelGGL(act_quantize_tensor_kernel<COAT_FMT_E4M3>, dim3(grid), dim3(kBlock), 0, st, x, n,
                           (const uint32_t*)acc, q);
        hipLaunchKernelGGL(act_finalize_kernel<COAT_FMT_E4M3>, dim3(1), dim3(kWave), 0, st, acc);
    } else {
        hipLaunchKernelGGL(act_quantize_tensor_kernel<COAT_FMT_E5M2>, dim3(grid), dim3(kBlock), 0, st, x, n,
                           (const uint32_t*)acc, q);
        hipLaunchKernelGGL(act_finalize_kernel<COAT_FMT_E5M2>, dim3(1), dim3(kWave), 0, st, acc);
    }
    return launch_status();
}

int coat_fp8_act_dequantize(const uint8_t* q, const float* scale, int64_t n, int32_t group, int32_t fmt,
                            uint16_t* x, coat_stream_t stream) {
    const int lg = group == 0 ? 0 : lg2_group_of(group);
    if (n < 0 || lg < 0 || (fmt != COAT_FMT_E4M3 && fmt != COAT_FMT_E5M2)) return COAT_EINVAL;
    if (n == 0) return COAT_OK;
    if (!x || !q || !scale) return COAT_EINVAL;
    if (!aligned16(x) || !aligned16(q) || !aligned(scale, 4)) return COAT_EALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const unsigned grid = grid_for((n + kTile - 1) / kTile, kActBlocksPerCU);
    const int lgs = group == 0 ? -1 : lg;
    if (fmt == COAT_FMT_E4M3)
        hipLaunchKernelGGL(act_dequantize_kernel<COAT_FMT_E4M3>, dim3(grid), dim3(kBlock), 0, st, q, scale, n, lgs, x);
    else
        hipLaunchKernelGGL(act_dequantize_kernel<COAT_FMT_E5M2>, dim3(grid), dim3(kBlock), 0, st, q, scale, n, lgs, x);
    return launch_status();
}

}  // extern "C"
