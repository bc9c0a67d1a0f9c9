// Host-side logic of the step library that touches no GPU: argument checks,
// the step's constants, and the multi-tensor plan tables with their chunked
// copy into device memory (a caller's workspace or the library's static
// array). Plain C++
// with no HIP dependency, so that the same code builds into a host-only
// driver that runs under AddressSanitizer and UndefinedBehaviorSanitizer on
// the CPU.
//
// The step it prepares is the AdamW update of COAT's FP8 optimizer states
// (page "FP8训练新范式：减少40%显存占用，训练速度提高1.4倍", sections
// FP8优化器状态 and 动态范围扩展): moment coefficients and bias corrections
// here, per-element work in the kernels.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "coat_fp8.h"

namespace {

constexpr int64_t kPlanTile = 1024;  // elements per wavefront tile (the kernels' kTile)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline int lg2_group_of(int32_t group) {
    if (group < 16 || group > 1024 || (group & (group - 1)) != 0) return -1;
    int l = 0;
    while ((1 << l) < group) ++l;
    return l;
}

inline bool fmt_ok(int32_t fmt) {
    const int base = fmt & 0xFF;
    return (base == COAT_FMT_E4M3 || base == COAT_FMT_E5M2) && (fmt & ~(0xFF | COAT_FMT_NO_EXPAND)) == 0;
}

inline bool finite_f(float x) { return x == x && x - x == 0.0f; }

// The step's constants, passed to the kernels by value.
struct StepConsts {
    double b1, c1, b2, c2;  // moment coefficients (c = 1 - b), fp64
    float decay;            // 1 - lr wd
    float ssz;              // lr / (1 - b1^t)
    float ib2;              // 1 / sqrt(1 - b2^t)
    float eps;
    int lg2_group;
    int expand_m, expand_v;
};

// One tensor's arrays, in the order and layout of coat_tensor.
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

// Bias corrections in fp64 on the host; the per-element coefficients the
// kernels read. COAT_EINVAL for a group size or format the kernels do not
// take, step < 1, a non-finite hyperparameter, or a bias correction of zero.
inline int make_consts(int32_t group, int32_t fmt_m, int32_t fmt_v, float lr, float b1, float b2, float eps,
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

// COAT_EINVAL for n < 0 or a missing array of a non-empty tensor, COAT_EALIGN
// for an element array off 16 bytes or a scale / exponent array off its type.
inline int check_tensor(const TensorRef& t) {
    if (t.n < 0) return COAT_EINVAL;
    if (t.n == 0) return COAT_OK;
    if (!t.p || !t.g || !t.mq || !t.ms || !t.mk || !t.vq || !t.vs || !t.vk) return COAT_EINVAL;
    if (!aligned16(t.p) || !aligned16(t.g) || !aligned16(t.mq) || !aligned16(t.vq) ||
        (t.w && !aligned16(t.w)) || !aligned(t.ms, 8) || !aligned(t.vs, 8) || !aligned(t.mk, 4) ||
        !aligned(t.vk, 4))
        return COAT_EALIGN;
    return COAT_OK;
}

constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Plan tables of a multi-tensor step: the descriptors, the prefix of whole
// tiles per tensor (count + 1 int64, first 0, last the total) and the indices
// of the tensors whose last tile is partial (int32), each section 256-byte
// aligned.
struct PlanLayout {
    size_t desc, fb, partial;  // section offsets in bytes
    size_t total;
};
constexpr PlanLayout plan_layout(size_t count) {
    return PlanLayout{0, align_up(sizeof(TensorRef) * count, 256),
                      align_up(sizeof(TensorRef) * count, 256) + align_up(sizeof(int64_t) * (count + 1), 256),
                      align_up(sizeof(TensorRef) * count, 256) + align_up(sizeof(int64_t) * (count + 1), 256) +
                          align_up(sizeof(int32_t) * count, 256)};
}

// Totals over a tensor list.
struct PlanSummary {
    int64_t tiles;      // all tiles, whole and partial
    int64_t full;       // whole tiles
    int64_t n_total;    // elements
    int32_t n_partial;  // tensors whose last tile is partial
};

// Checks every descriptor (check_tensor) and sums the list.
inline int scan_tensors(const coat_tensor* tensors, int32_t count, PlanSummary* s) {
    *s = PlanSummary{0, 0, 0, 0};
    for (int32_t i = 0; i < count; ++i) {
        TensorRef t;
        memcpy(&t, &tensors[i], sizeof(TensorRef));
        const int rc = check_tensor(t);
        if (rc) return rc;
        s->full += t.n / kPlanTile;
        s->tiles += (t.n + kPlanTile - 1) / kPlanTile;
        s->n_total += t.n;
        if (t.n % kPlanTile) ++s->n_partial;
    }
    return COAT_OK;
}

// The static plan tables (coat_fp8_adamw_step_multi_static): the same sections
// sized for COAT_STATIC_MAX_TENSORS tensors.
constexpr PlanLayout kStaticLayout = plan_layout((size_t)COAT_STATIC_MAX_TENSORS);

// The tables reach device memory (a caller's workspace or the library's
// static array) through kernel arguments, 3 KB per copy.
constexpr uint32_t kArgChunkBytes = 3072;
struct alignas(16) ArgChunk {
    unsigned char data[kArgChunkBytes];
};

// Packs consecutive bytes of one table section into argument chunks and hands
// each full chunk to `sink(chunk, bytes, offset)`, offset being the chunk's
// byte offset in the table image; sections are 16-byte aligned and padded, so
// a chunk is rounded up to 16 bytes (its tail zeroed). The sink returns false
// on failure, which ok() then reports.
template <class Sink>
class ChunkWriter {
  public:
    ChunkWriter(size_t offset, Sink& sink) : off_(offset), sink_(sink) {}
    void put(const void* src, size_t n) {
        const unsigned char* p = static_cast<const unsigned char*>(src);
        while (n > 0) {
            const size_t take = n < kArgChunkBytes - fill_ ? n : kArgChunkBytes - fill_;
            memcpy(chunk_.data + fill_, p, take);
            fill_ += (uint32_t)take;
            p += take;
            n -= take;
            if (fill_ == kArgChunkBytes) flush();
        }
    }
    void flush() {
        if (fill_ == 0) return;
        const uint32_t bytes = (fill_ + 15u) & ~15u;
        memset(chunk_.data + fill_, 0, bytes - fill_);
        if (!sink_(chunk_, bytes, off_)) ok_ = false;
        off_ += bytes;
        fill_ = 0;
    }
    bool ok() const { return ok_; }

  private:
    ArgChunk chunk_;
    size_t off_;
    Sink& sink_;
    uint32_t fill_ = 0;
    bool ok_ = true;
};

// Every byte of the plan tables that a step over `count` tensors reads, in
// the sections of layout L (plan_layout(count) for a caller's workspace,
// kStaticLayout for the static array), through `sink`: descriptors
// [0, count), the prefix of whole tiles [0, count] (first 0, last the total)
// and the indices of the tensors whose last tile is partial [0, n_partial).
// The 16-byte rounding of a chunk stays inside its 256-byte aligned section.
// False if the sink failed. The caller has checked the descriptors
// (scan_tensors) and that L holds `count` tensors.
template <class Sink>
bool write_plan_tables(const coat_tensor* tensors, int32_t count, const PlanLayout& L, Sink& sink) {
    ChunkWriter<Sink> desc(L.desc, sink);
    desc.put(tensors, sizeof(TensorRef) * (size_t)count);
    desc.flush();
    ChunkWriter<Sink> fbw(L.fb, sink);
    int64_t acc = 0;
    for (int32_t i = 0; i < count; ++i) {
        fbw.put(&acc, sizeof(acc));
        acc += tensors[i].n / kPlanTile;
    }
    fbw.put(&acc, sizeof(acc));
    fbw.flush();
    ChunkWriter<Sink> pw(L.partial, sink);
    for (int32_t i = 0; i < count; ++i)
        if (tensors[i].n % kPlanTile) pw.put(&i, sizeof(i));
    pw.flush();
    return desc.ok() && fbw.ok() && pw.ok();
}

}  // namespace
