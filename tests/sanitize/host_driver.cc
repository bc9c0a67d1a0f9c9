// Drives the step library's host-side logic (coat_host.h: argument checks,
// the step constants, the multi-tensor plan tables and their chunked copy
// into a workspace or the static table array) under AddressSanitizer and
// UndefinedBehaviorSanitizer on the CPU (built by tests/test_host_sanitize.py).
// Descriptor arrays and table images are heap-allocated at exactly the size a
// call may touch, so any read or write past them is reported. Element
// pointers are aligned stand-in addresses: the host code checks them but
// never dereferences them.
//
//   host_driver <sizes-file>            every check; prints "ok" at the end
//   host_driver <sizes-file> overrun    scan_tensors over one descriptor more
//                                       than the array holds (must be reported)
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "coat_host.h"

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

// A descriptor with aligned stand-in addresses, distinct per tensor.
static coat_tensor fake_tensor(int64_t n, int i) {
    const uintptr_t base = 0x100000u + (uintptr_t)i * 0x1000u;
    coat_tensor t;
    t.params = reinterpret_cast<float*>(base);
    t.params_bf16 = reinterpret_cast<uint16_t*>(base + 0x100);
    t.grads = reinterpret_cast<const uint16_t*>(base + 0x200);
    t.m_q = reinterpret_cast<uint8_t*>(base + 0x300);
    t.m_s = reinterpret_cast<double*>(base + 0x400);
    t.m_k = reinterpret_cast<float*>(base + 0x500);
    t.v_q = reinterpret_cast<uint8_t*>(base + 0x600);
    t.v_s = reinterpret_cast<double*>(base + 0x700);
    t.v_k = reinterpret_cast<float*>(base + 0x800);
    t.n = n;
    return t;
}

// t with field f (0 .. 9, in declaration order) replaced by the bits v
static coat_tensor with_field(coat_tensor t, int f, uintptr_t v) {
    static_assert(sizeof(coat_tensor) == 10 * sizeof(uintptr_t), "descriptor layout");
    uintptr_t a[10];
    memcpy(a, &t, sizeof(t));
    a[f] = v;
    memcpy(&t, a, sizeof(t));
    return t;
}
static uintptr_t field(const coat_tensor& t, int f) {
    uintptr_t a[10];
    memcpy(a, &t, sizeof(t));
    return a[f];
}

static TensorRef as_ref(const coat_tensor& t) {
    TensorRef r;
    memcpy(&r, &t, sizeof(r));
    return r;
}

static void check_consts() {
    StepConsts c;
    const float nan = nanf(""), inf = INFINITY;
    // valid
    CHECK(make_consts(128, COAT_FMT_E4M3, COAT_FMT_E5M2, 1e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 10, &c) == COAT_OK);
    CHECK(c.lg2_group == 7 && c.expand_m == 1 && c.expand_v == 1);
    CHECK(c.c1 == 1.0 - (double)0.9f && c.c2 == 1.0 - (double)0.95f);
    CHECK(c.ssz == (float)(1e-4 / (1.0 - pow((double)0.9f, 10.0))));
    CHECK(make_consts(16, COAT_FMT_E4M3 | COAT_FMT_NO_EXPAND, COAT_FMT_E4M3, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 1,
                      &c) == COAT_OK);
    CHECK(c.lg2_group == 4 && c.expand_m == 0 && c.expand_v == 1 && c.decay == 1.0f);
    CHECK(make_consts(1024, COAT_FMT_E5M2, COAT_FMT_E5M2, 1e-3f, 0.0f, 0.0f, 0.0f, 0.0f, 1, &c) == COAT_OK);
    CHECK(make_consts(64, COAT_FMT_NO_EXPAND, COAT_FMT_E5M2 | COAT_FMT_NO_EXPAND, 1e-3f, 0.5f, 0.5f, 1e-8f, 0.0f, 2,
                      &c) == COAT_OK);  // E4M3 is format 0
    CHECK(c.expand_m == 0 && c.expand_v == 0);
    // group sizes
    const int32_t bad_groups[] = {0, 1, 8, 15, 17, 48, 100, 2048, -128, 1 << 30};
    for (int32_t g : bad_groups)
        CHECK(make_consts(g, COAT_FMT_E4M3, COAT_FMT_E4M3, 1e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1, &c) == COAT_EINVAL);
    // formats
    const int32_t bad_fmts[] = {-1, 2, 3, 255, COAT_FMT_NO_EXPAND | 2, COAT_FMT_NO_EXPAND << 1, (int32_t)0x80000000};
    for (int32_t f : bad_fmts) {
        CHECK(make_consts(128, f, COAT_FMT_E4M3, 1e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1, &c) == COAT_EINVAL);
        CHECK(make_consts(128, COAT_FMT_E4M3, f, 1e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1, &c) == COAT_EINVAL);
    }
    // steps and hyperparameters
    CHECK(make_consts(128, 0, 0, 1e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 0, &c) == COAT_EINVAL);
    CHECK(make_consts(128, 0, 0, 1e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, -5, &c) == COAT_EINVAL);
    const float bad_vals[] = {nan, inf, -inf};
    for (float v : bad_vals) {
        CHECK(make_consts(128, 0, 0, v, 0.9f, 0.95f, 1e-8f, 0.1f, 1, &c) == COAT_EINVAL);
        CHECK(make_consts(128, 0, 0, 1e-4f, v, 0.95f, 1e-8f, 0.1f, 1, &c) == COAT_EINVAL);
        CHECK(make_consts(128, 0, 0, 1e-4f, 0.9f, v, 1e-8f, 0.1f, 1, &c) == COAT_EINVAL);
        CHECK(make_consts(128, 0, 0, 1e-4f, 0.9f, 0.95f, v, 0.1f, 1, &c) == COAT_EINVAL);
        CHECK(make_consts(128, 0, 0, 1e-4f, 0.9f, 0.95f, 1e-8f, v, 1, &c) == COAT_EINVAL);
    }
    // a bias correction of zero (beta = 1) or a negative second one
    CHECK(make_consts(128, 0, 0, 1e-4f, 1.0f, 0.95f, 1e-8f, 0.1f, 3, &c) == COAT_EINVAL);
    CHECK(make_consts(128, 0, 0, 1e-4f, 0.9f, 1.0f, 1e-8f, 0.1f, 3, &c) == COAT_EINVAL);
    CHECK(make_consts(128, 0, 0, 1e-4f, 0.9f, 1.5f, 1e-8f, 0.1f, 1, &c) == COAT_EINVAL);
    // a huge step: b^t underflows to 0, the corrections are 1
    CHECK(make_consts(128, 0, 0, 1e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, (int64_t)1 << 62, &c) == COAT_OK);
    CHECK(c.ssz == 1e-4f && c.ib2 == 1.0f);
}

static void check_tensors() {
    coat_tensor t = fake_tensor(4096, 0);
    CHECK(check_tensor(as_ref(t)) == COAT_OK);
    coat_tensor u = t;
    u.params_bf16 = nullptr;  // the bf16 copy is optional
    CHECK(check_tensor(as_ref(u)) == COAT_OK);
    u = t;
    u.n = -1;
    CHECK(check_tensor(as_ref(u)) == COAT_EINVAL);
    coat_tensor empty{};
    CHECK(check_tensor(as_ref(empty)) == COAT_OK);  // n = 0: nothing is read
    // each required array missing
    for (int f = 0; f < 9; ++f) {
        if (f == 1) continue;  // params_bf16
        CHECK(check_tensor(as_ref(with_field(t, f, 0))) == COAT_EINVAL);
    }
    // misalignment of each array by the smallest step that breaks it
    const uintptr_t need[9] = {16, 16, 16, 16, 8, 4, 16, 8, 4};
    for (int f = 0; f < 9; ++f) {
        CHECK(check_tensor(as_ref(with_field(t, f, field(t, f) + need[f] / 2))) == COAT_EALIGN);
    }
}

// A sink that copies each chunk into a host image of exactly `cap` bytes
// (the workspace or static array it stands for), rejecting a chunk that is
// empty, oversized, unaligned or past the end.
struct CopySink {
    unsigned char* dst;
    size_t cap;
    int calls;
    bool operator()(const ArgChunk& c, uint32_t bytes, size_t off) {
        if (bytes == 0 || bytes > kArgChunkBytes || bytes % 16 || off % 16 || off + bytes > cap) return false;
        memcpy(dst + off, c.data, bytes);
        ++calls;
        return true;
    }
};

// The tables written in layout L, checked field by field against a direct
// recount of the list.
static void check_tables(const coat_tensor* ts, const std::vector<int64_t>& sizes, const PlanLayout& L) {
    const int32_t count = (int32_t)sizes.size();
    unsigned char* image = static_cast<unsigned char*>(malloc(L.total));
    memset(image, 0xA5, L.total);
    CopySink sink{image, L.total, 0};
    CHECK(write_plan_tables(ts, count, L, sink));
    CHECK(sink.calls >= 1);  // the prefix is written even for an empty list
    const int64_t* fb = reinterpret_cast<const int64_t*>(image + L.fb);
    const int32_t* part = reinterpret_cast<const int32_t*>(image + L.partial);
    int64_t full = 0;
    int32_t np = 0;
    for (int32_t i = 0; i < count; ++i) {
        CHECK(memcmp(image + L.desc + sizeof(TensorRef) * (size_t)i, &ts[i], sizeof(TensorRef)) == 0);
        CHECK(fb[i] == full);
        full += sizes[(size_t)i] / 1024;
        if (sizes[(size_t)i] % 1024) CHECK(part[np++] == i);
    }
    CHECK(fb[count] == full);
    // a failing sink is reported
    struct FailSink {
        bool operator()(const ArgChunk&, uint32_t, size_t) { return false; }
    } fail;
    CHECK(!write_plan_tables(ts, count, L, fail));
    free(image);
}

// The plan of a list: its summary and its tables in the workspace layout and,
// when the list fits, in the static array's layout.
static void check_plan(const std::vector<int64_t>& sizes) {
    const int32_t count = (int32_t)sizes.size();
    // exactly `count` descriptors on the heap (one allocation of that size)
    coat_tensor* ts = static_cast<coat_tensor*>(malloc(sizeof(coat_tensor) * (count ? count : 1)));
    for (int32_t i = 0; i < count; ++i) ts[i] = fake_tensor(sizes[(size_t)i], i);
    const PlanLayout L = plan_layout((size_t)count);
    CHECK(L.desc == 0 && L.fb % 256 == 0 && L.partial % 256 == 0 && L.total % 256 == 0);
    CHECK(L.fb >= sizeof(TensorRef) * (size_t)count && L.partial - L.fb >= 8 * ((size_t)count + 1));
    CHECK(L.total - L.partial >= 4 * (size_t)count);
    PlanSummary s;
    CHECK(scan_tensors(ts, count, &s) == COAT_OK);
    int64_t full = 0, tiles = 0, n_total = 0;
    int32_t np = 0;
    for (int32_t i = 0; i < count; ++i) {
        full += sizes[(size_t)i] / 1024;
        tiles += (sizes[(size_t)i] + 1023) / 1024;
        n_total += sizes[(size_t)i];
        np += sizes[(size_t)i] % 1024 ? 1 : 0;
    }
    CHECK(s.full == full && s.tiles == tiles && s.n_total == n_total && s.n_partial == np);
    check_tables(ts, sizes, L);
    if (count <= COAT_STATIC_MAX_TENSORS) check_tables(ts, sizes, kStaticLayout);
    // a bad descriptor anywhere in the list is found
    if (count > 0) {
        coat_tensor keep = ts[count - 1];
        ts[count - 1] = with_field(keep, 2, 0);  // no grads
        CHECK(scan_tensors(ts, count, &s) == (keep.n ? COAT_EINVAL : COAT_OK));
        ts[count - 1] = keep;
    }
    free(ts);
}

// Ragged lists built from a seed: sizes 0 .. 5000 and a few whole-tile ones.
static std::vector<int64_t> ragged_list(int count, uint32_t seed) {
    std::vector<int64_t> v((size_t)count);
    for (int i = 0; i < count; ++i) {
        seed = seed * 1664525u + 1013904223u;
        const uint32_t r = seed >> 8;
        v[(size_t)i] = (r % 7 == 0) ? (int64_t)(r % 5) * 1024 : (int64_t)(r % 5001);
    }
    return v;
}

int main(int argc, char** argv) {
    if (argc < 2) {
        fprintf(stderr, "usage: host_driver <sizes-file> [overrun]\n");
        return 2;
    }
    std::vector<int64_t> model;
    FILE* f = fopen(argv[1], "r");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", argv[1]);
        return 2;
    }
    long long x;
    while (fscanf(f, "%lld", &x) == 1) model.push_back((int64_t)x);
    fclose(f);

    if (argc > 2 && strcmp(argv[2], "overrun") == 0) {
        // descriptors for one tensor fewer than the count passed
        const int32_t count = (int32_t)model.size();
        coat_tensor* ts = static_cast<coat_tensor*>(malloc(sizeof(coat_tensor) * (size_t)(count - 1)));
        for (int32_t i = 0; i + 1 < count; ++i) ts[i] = fake_tensor(model[(size_t)i], i);
        PlanSummary s;
        const int rc = scan_tensors(ts, count, &s);
        printf("not reported: rc %d\n", rc);
        free(ts);
        return 0;
    }

    check_consts();
    check_tensors();
    check_plan(model);  // the model's list (e.g. 363 tensors)
    check_plan({});
    check_plan({1});
    check_plan({1024});
    check_plan({0, 0, 1023, 1025, 0});
    for (int c : {1, 2, 7, 64, 300}) check_plan(ragged_list(c, 17u + (uint32_t)c));
    // exactly the static table's capacity: every section filled to its end
    check_plan(ragged_list(COAT_STATIC_MAX_TENSORS, 5u));
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
