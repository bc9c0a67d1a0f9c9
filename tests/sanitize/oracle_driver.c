/*
 * Drives every entry point of the CPU oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_oracle_sanitize.py). Every
 * buffer is heap-allocated at exactly the size the call needs, so a read or
 * write past a ragged last group is reported. Inputs come from a small
 * linear congruential generator and include zeros, signed zeros, NaN, Inf,
 * subnormals and huge values; no result is checked here beyond the status
 * codes (the values are pinned by the Python tests).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double coat_oracle_fp8_decode(uint8_t code, int32_t fmt);
uint8_t coat_oracle_fp8_encode(double y, int32_t fmt);
void coat_oracle_fp8_decode_array(const uint8_t* q, int64_t n, int32_t fmt, double* out);
void coat_oracle_fp8_encode_array(const double* y, int64_t n, int32_t fmt, uint8_t* out);
double coat_oracle_fp8_range(int32_t fmt);
float coat_oracle_group_k(double amax, double amin, int32_t fmt);
int coat_oracle_quantize(const double* x, int64_t n, int32_t G, int32_t fmt, uint8_t* q, double* s, float* k);
int coat_oracle_dequantize(const uint8_t* q, const double* s, const float* k, int64_t n, int32_t G,
                           int32_t fmt, double* x);
int coat_oracle_adamw_dense(float* p, uint16_t* w, const uint16_t* g, double* m, double* v, int64_t n,
                            float lr, float b1, float b2, float eps, float wd, int64_t step);
int coat_oracle_adamw_step(float* p, uint16_t* w, const uint16_t* g, uint8_t* m_q, double* m_s, float* m_k,
                           uint8_t* v_q, double* v_s, float* v_k, int64_t n, int32_t G, int32_t fmt_m,
                           int32_t fmt_v, float lr, float b1, float b2, float eps, float wd, int64_t step);
int coat_oracle_act_quantize(const uint16_t* x, int64_t n, int32_t G, int32_t fmt, uint8_t* q, float* s);
int coat_oracle_act_dequantize(const uint8_t* q, const float* s, int64_t n, int32_t G, int32_t fmt,
                               uint16_t* x);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(state >> 32);
}
static double uniform(void) { return (next_u32() + 0.5) / 4294967296.0; }

/* A value of magnitude 10^[lo, hi], random sign, with a few special values mixed in. */
static double value(double lo, double hi, int i) {
    switch (i % 97) {
        case 3: return 0.0;
        case 5: return -0.0;
        case 11: return 4.9e-324;
        default: break;
    }
    double mag = pow(10.0, lo + (hi - lo) * uniform());
    return (next_u32() & 1u) ? -mag : mag;
}

static void* xmalloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int fails = 0;
static void expect_ok(int rc, const char* what, int64_t n, int G) {
    if (rc != 0) {
        fprintf(stderr, "%s n=%lld G=%d: status %d\n", what, (long long)n, G, rc);
        ++fails;
    }
}

int main(void) {
    const int64_t sizes[] = {0, 1, 5, 15, 16, 17, 127, 128, 129, 1000, 4099};
    const int groups[] = {16, 32, 128, 1024};
    const int fmts[] = {0, 1, 0x100, 0x101};
    for (int f = 0; f < 2; ++f) {
        for (int c = 0; c < 256; ++c) {
            double y = coat_oracle_fp8_decode((uint8_t)c, f);
            (void)coat_oracle_fp8_encode(y, f);
        }
        (void)coat_oracle_fp8_range(f);
        (void)coat_oracle_group_k(1.0, 1e-3, f);
        (void)coat_oracle_group_k(0.0, INFINITY, f);
    }
    for (size_t a = 0; a < sizeof sizes / sizeof *sizes; ++a) {
        const int64_t n = sizes[a];
        for (size_t b = 0; b < sizeof groups / sizeof *groups; ++b) {
            const int G = groups[b];
            const int64_t ng = (n + G - 1) / G;
            for (size_t c = 0; c < sizeof fmts / sizeof *fmts; ++c) {
                const int fmt = fmts[c];
                double* x = xmalloc(sizeof(double) * (size_t)n);
                double* back = xmalloc(sizeof(double) * (size_t)n);
                uint8_t* q = xmalloc((size_t)n);
                double* s = xmalloc(sizeof(double) * (size_t)ng);
                float* k = xmalloc(sizeof(float) * (size_t)ng);
                for (int64_t i = 0; i < n; ++i) x[i] = value(-9.0, 0.0, (int)i);
                if (n > 7) x[7] = NAN;
                if (n > 200) x[200] = INFINITY;
                if (n > 300) x[300] = 1e300;
                expect_ok(coat_oracle_quantize(x, n, G, fmt, q, s, k), "quantize", n, G);
                expect_ok(coat_oracle_dequantize(q, s, k, n, G, fmt & 0xFF, back), "dequantize", n, G);
                coat_oracle_fp8_encode_array(x, n, fmt & 0xFF, q);
                coat_oracle_fp8_decode_array(q, n, fmt & 0xFF, back);
                free(x); free(back); free(q); free(s); free(k);
            }
            /* the step, both moments, bf16 copy on and off */
            for (int withw = 0; withw < 2; ++withw) {
                float* p = xmalloc(sizeof(float) * (size_t)n);
                uint16_t* w = withw ? xmalloc(sizeof(uint16_t) * (size_t)n) : NULL;
                uint16_t* g = xmalloc(sizeof(uint16_t) * (size_t)n);
                double* m = xmalloc(sizeof(double) * (size_t)n);
                double* v = xmalloc(sizeof(double) * (size_t)n);
                uint8_t* mq = xmalloc((size_t)n);
                uint8_t* vq = xmalloc((size_t)n);
                double* ms = xmalloc(sizeof(double) * (size_t)ng);
                double* vs = xmalloc(sizeof(double) * (size_t)ng);
                float* mk = xmalloc(sizeof(float) * (size_t)ng);
                float* vk = xmalloc(sizeof(float) * (size_t)ng);
                for (int64_t i = 0; i < n; ++i) {
                    p[i] = (float)value(-4.0, -1.0, (int)i);
                    const float gf = (float)value(-5.0, -2.0, (int)i + 1);
                    uint32_t u;
                    memcpy(&u, &gf, 4);
                    g[i] = (uint16_t)(u >> 16);
                    m[i] = value(-8.0, -5.0, (int)i + 2);
                    v[i] = fabs(value(-10.0, -9.0, (int)i + 3));
                }
                if (n > 9) g[9] = 0x7FC0; /* NaN gradient: poisons its groups */
                expect_ok(coat_oracle_quantize(m, n, G, 0, mq, ms, mk), "quantize m", n, G);
                expect_ok(coat_oracle_quantize(v, n, G, 1, vq, vs, vk), "quantize v", n, G);
                for (int64_t t = 10; t < 13; ++t)
                    expect_ok(coat_oracle_adamw_step(p, w, g, mq, ms, mk, vq, vs, vk, n, G, 0, 1, 1e-4f, 0.9f,
                                                     0.95f, 1e-8f, 0.1f, t), "adamw_step", n, G);
                expect_ok(coat_oracle_adamw_dense(p, w, g, m, v, n, 1e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 10),
                          "adamw_dense", n, G);
                free(p); free(w); free(g); free(m); free(v); free(mq); free(vq);
                free(ms); free(vs); free(mk); free(vk);
            }
        }
        /* activation codec: per tensor and per group, ragged groups included */
        const int act_groups[] = {0, 7, 16, 128};
        for (size_t b = 0; b < sizeof act_groups / sizeof *act_groups; ++b) {
            const int G = act_groups[b];
            const int64_t ns = G == 0 ? 1 : (n + G - 1) / G;
            for (int fmt = 0; fmt < 2; ++fmt) {
                uint16_t* x = xmalloc(sizeof(uint16_t) * (size_t)n);
                uint16_t* back = xmalloc(sizeof(uint16_t) * (size_t)n);
                uint8_t* q = xmalloc((size_t)n);
                float* s = xmalloc(sizeof(float) * (size_t)(ns > 0 ? ns : 1));
                for (int64_t i = 0; i < n; ++i) {
                    const float xf = (float)value(-3.0, 1.0, (int)i);
                    uint32_t u;
                    memcpy(&u, &xf, 4);
                    x[i] = (uint16_t)(u >> 16);
                }
                if (n > 40) x[40] = 0x7F80; /* Inf */
                expect_ok(coat_oracle_act_quantize(x, n, G, fmt, q, s), "act_quantize", n, G);
                expect_ok(coat_oracle_act_dequantize(q, s, n, G, fmt, back), "act_dequantize", n, G);
                free(x); free(back); free(q); free(s);
            }
        }
    }
    if (fails) {
        fprintf(stderr, "%d calls failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
