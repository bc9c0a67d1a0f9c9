// Bandwidth instrument for bench.py --ceiling (not part of the step library).
//
// Moves exactly the bytes of one FP8-state AdamW step over a flat parameter
// buffer, in one of the step kernel's access patterns, and computes nothing:
// one 64-lane wavefront per tile of 1024 consecutive elements, 128-bit loads
// of the fp32 master weights (64 B per lane), the bf16 grads (32 B) and the
// two code arrays (16 B each), and per group of G elements an fp64 scale and
// an fp32 exponent for each moment (read by the lanes that read them in the
// step); then 128-bit stores of the master weights, a bf16 copy and the
// codes, and the per-group scale and exponent. Layout 0 gives each lane 16
// consecutive elements of every stream (the step's pattern for a tile that
// ends inside its tensor); layout 1 is the step's pattern for a whole tile:
// codes and per-group state as in layout 0, but each wave access of the
// master weights, grads and bf16 copy covering 1 KB of consecutive bytes
// (master weights 4 per lane per quarter tile, grads and bf16 copy 8 per lane
// per half tile). Every stored master weight, code, scale and exponent is the
// one loaded, so the state is left as it was; the bf16 copy holds the high
// halves of master weights of the same tile (their order within the tile is
// not the step's, which re-lays them through LDS). The grid is the step's:
// one contiguous run of tiles per block, the block's four wavefronts taking
// its tiles in turn, 256 blocks per CU.
//
// Its time is the memory-only floor of the step's access pattern: what the
// step would take if its arithmetic were free.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWave = 64, kLaneElems = 16, kTile = kWave * kLaneElems, kBlock = 256, kWaves = kBlock / kWave;

template <int LAYOUT>
__global__ __launch_bounds__(kBlock) void pattern_kernel(float* __restrict__ p, uint16_t* __restrict__ w,
                                                         const uint16_t* __restrict__ g, uint8_t* __restrict__ mq,
                                                         uint8_t* __restrict__ vq, double* __restrict__ ms,
                                                         float* __restrict__ mk, double* __restrict__ vs,
                                                         float* __restrict__ vk, int64_t tiles, int lg2_group) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t per = (tiles + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < tiles ? b0 + per : tiles;
    const int lpg = 1 << (lg2_group - 4);
    const bool odd = ((lane >> 2) & 1) != 0;  // the step's lane roles: lanes 4..7 of 8 hold the second moment
    for (int64_t tile = b0 + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); tile < b1; tile += kWaves) {
        const int64_t e0 = tile * kTile + (int64_t)lane * kLaneElems;
        const int64_t gi = e0 >> lg2_group;
        const double s = odd ? vs[gi] : ms[gi];
        const float k = odd ? vk[gi] : mk[gi];
        const u32x4 a = *reinterpret_cast<const u32x4*>(mq + e0);
        const u32x4 b = *reinterpret_cast<const u32x4*>(vq + e0);
        // layout 0: elements e0 .. e0 + 15 of each stream; layout 1: master
        // weights at 256 i + 4 lane, grads and bf16 copy at 512 h + 8 lane
        const int64_t t0 = tile * kTile;
        const uint16_t* gl = LAYOUT ? g + t0 + 8 * lane : g + e0;
        float* pl = LAYOUT ? p + t0 + 4 * lane : p + e0;
        uint16_t* wl = LAYOUT ? w + t0 + 8 * lane : w + e0;
        const int gstep = LAYOUT ? 512 : 8, pstep = LAYOUT ? 256 : 4;
        const u32x4 g0 = *reinterpret_cast<const u32x4*>(gl);
        const u32x4 g1 = *reinterpret_cast<const u32x4*>(gl + gstep);
        f32x4 pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = *reinterpret_cast<const f32x4*>(pl + pstep * i);
        // opaque to the optimizer, so that storing back what was loaded is not
        // dropped as a store of an unchanged value
        u32x4 a_ = a, b_ = b;
        double s_ = s;
        float k_ = k;
        asm volatile("" : "+v"(pv[0]), "+v"(pv[1]), "+v"(pv[2]), "+v"(pv[3]), "+v"(a_), "+v"(b_), "+v"(s_), "+v"(k_));
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(pl + pstep * i) = pv[i];
        u32x4 hi[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const f32x4 x = pv[2 * i], y = pv[2 * i + 1];
            auto h = [](float lo_, float hi_) {
                return (__builtin_bit_cast(uint32_t, lo_) >> 16) | (__builtin_bit_cast(uint32_t, hi_) & 0xFFFF0000u);
            };
            hi[i] = u32x4{h(x.x, x.y), h(x.z, x.w), h(y.x, y.y), h(y.z, y.w)};
        }
        *reinterpret_cast<u32x4*>(wl) = hi[0];
        *reinterpret_cast<u32x4*>(wl + gstep) = hi[1];
        *reinterpret_cast<u32x4*>(mq + e0) = a_;
        *reinterpret_cast<u32x4*>(vq + e0) = b_;
        // the grads are only read: an empty asm that takes them keeps their loads
        asm volatile("" ::"v"(g0.x), "v"(g0.y), "v"(g0.z), "v"(g0.w), "v"(g1.x), "v"(g1.y), "v"(g1.z), "v"(g1.w));
        if ((lane & (lpg - 1)) == 0 || (lane & (lpg - 1)) == 4) {
            if (odd) {
                vs[gi] = s_;
                vk[gi] = k_;
            } else {
                ms[gi] = s_;
                mk[gi] = k_;
            }
        }
    }
}

// Plain streams for scale: each block takes one contiguous run of 16-byte
// words, each lane four words per iteration (all loads before the stores).
constexpr int kUnroll = 4;
__device__ __forceinline__ void run_of(int64_t n16, int64_t& b0, int64_t& b1) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    b0 = (int64_t)blockIdx.x * per;
    b1 = b0 + per < n16 ? b0 + per : n16;
}

__global__ __launch_bounds__(kBlock) void copy_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ b, int64_t n16) {
    int64_t b0, b1;
    run_of(n16, b0, b1);
    for (int64_t i = b0 + threadIdx.x; i < b1; i += (int64_t)kBlock * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kBlock;
            v[u] = j < b1 ? a[j] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kBlock;
            if (j < b1) b[j] = v[u];
        }
    }
}

__global__ __launch_bounds__(kBlock) void read_kernel(const u32x4* __restrict__ a, int64_t n16, uint32_t* out) {
    int64_t b0, b1;
    run_of(n16, b0, b1);
    uint32_t acc = 0;
    for (int64_t i = b0 + threadIdx.x; i < b1; i += (int64_t)kBlock * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kBlock;
            v[u] = j < b1 ? a[j] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) out[0] = acc;  // keeps the loads; almost never taken
}

__global__ __launch_bounds__(kBlock) void write_kernel(u32x4* __restrict__ b, int64_t n16) {
    int64_t b0, b1;
    run_of(n16, b0, b1);
    for (int64_t i = b0 + threadIdx.x; i < b1; i += (int64_t)kBlock * kUnroll) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kBlock;
            if (j < b1) b[j] = u32x4{(uint32_t)j, 0u, 0u, 0u};
        }
    }
}

unsigned plain_blocks() {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return (unsigned)(cus * 64);
}

}  // namespace

extern "C" {

// Plain streams over n16 16-byte words on `stream`, 64 blocks per CU: copy a
// to b, read a (out: a 4-byte device word written only in a case that does
// not arise), write b. Return 0, or -1 / -3 as below.
int ceiling_copy_pass(const void* a, void* b, int64_t n16, hipStream_t stream) {
    if (n16 <= 0) return -1;
    hipLaunchKernelGGL(copy_kernel, dim3(plain_blocks()), dim3(kBlock), 0, stream, (const u32x4*)a, (u32x4*)b, n16);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
int ceiling_read_pass(const void* a, int64_t n16, uint32_t* out, hipStream_t stream) {
    if (n16 <= 0 || !out) return -1;
    hipLaunchKernelGGL(read_kernel, dim3(plain_blocks()), dim3(kBlock), 0, stream, (const u32x4*)a, n16, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
int ceiling_write_pass(void* b, int64_t n16, hipStream_t stream) {
    if (n16 <= 0) return -1;
    hipLaunchKernelGGL(write_kernel, dim3(plain_blocks()), dim3(kBlock), 0, stream, (u32x4*)b, n16);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}


// One pass over n elements (a multiple of 1024) with groups of 2^lg2_group
// (128 .. 1024), in access pattern `layout` (0 or 1, as above), on `stream`;
// blocks = 256 per CU, each reserving `lds_bytes` of LDS (the step's
// per-block LDS gives the step's residency: four blocks per CU; 0 lets the
// probe fill the CU). Returns 0, or -1 for a bad argument, -3 if the launch
// failed.
int ceiling_pattern_pass(float* p, uint16_t* w, const uint16_t* g, uint8_t* mq, uint8_t* vq, double* ms,
                         float* mk, double* vs, float* vk, int64_t n, int lg2_group, int layout, int lds_bytes,
                         hipStream_t stream) {
    if (n <= 0 || n % kTile || lg2_group < 7 || lg2_group > 10 || lds_bytes < 0 || lds_bytes > 65536 ||
        (layout != 0 && layout != 1))
        return -1;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t tiles = n / kTile;
    int64_t blocks = (int64_t)cus * 256;
    const int64_t need = (tiles + kWaves - 1) / kWaves;
    if (blocks > need) blocks = need;
    if (layout == 0)
        hipLaunchKernelGGL(pattern_kernel<0>, dim3((unsigned)blocks), dim3(kBlock), (unsigned)lds_bytes, stream, p, w,
                           g, mq, vq, ms, mk, vs, vk, tiles, lg2_group);
    else
        hipLaunchKernelGGL(pattern_kernel<1>, dim3((unsigned)blocks), dim3(kBlock), (unsigned)lds_bytes, stream, p, w,
                           g, mq, vq, ms, mk, vs, vk, tiles, lg2_group);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
