/*
 * CPU oracle for the COAT FP8-optimizer-state AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or
 * load this file or the library built from it; only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark do. It shares no code,
 * header, table or constant with the HIP implementation.
 *
 * Plain, single-threaded, fp64 C with libm, written to be read against the
 * pages rather than to be fast:
 *
 *   - "COAT: FP8 training, 40% less memory, 1.4x faster" (blob.wenxiaobai.com),
 *     section "FP8 optimizer states": first and second Adam moments are kept
 *     per quantization group in FP8; E4M3 spans 0.00195 .. 448, a dynamic range
 *     of about 200000, while a group of the first moment spans about 1000:1 and
 *     one of the second moment about 10:1.
 *   - same page, section "Solution: dynamic range expansion": an expansion
 *     function f is applied before quantizing; k is computed on the fly, one k
 *     per group, and k > 1 widens the group's range toward the FP8 range.
 *     The page's formula for f is lost; f(x) = sign(x)|x|^k with
 *     k = ln(R_fp8) / ln(R_x) is the reading taken here.
 *   - same page: E4M3 suits the first moment better than E5M2; for the second
 *     moment both are close once expansion is applied.
 *   - zhanchiexpo.com mirror of the same article: the states are quantized
 *     per group ("per-group quantization").
 *   - maplevalley.com.cn FP8 guide, section "format choice": E4M3 is
 *     1 sign + 4 exponent + 3 mantissa bits, E5M2 is 1 + 5 + 2.
 *
 * Readings the pages leave open:
 *   - decode is OCP E4M3FN (bias 7, max 448, NaN 0x7F/0xFF, no Inf) and OCP
 *     E5M2 (bias 15, max 57344, Inf 0x7C/0xFC, NaN 0x7D-0x7F/0xFD-0xFF);
 *   - R_fp8 = max finite / min subnormal (229376 for E4M3, matching the page's
 *     0.00195 = 2^-9 lower end, and 3758096384 for E5M2);
 *   - encode rounds to nearest with ties to the even code and saturates at the
 *     largest finite value; NaN encodes to 0x7F;
 *   - k = 1 when the group is all zero or max/min <= 1 + 1e-6; no clamp on k
 *     otherwise, so k < 1 is allowed when a group spans more than R_fp8;
 *   - s = max|f| / fpmax is kept in fp64 and k in fp32; the stored fp32 k is
 *     the one used for s and for the codes, so (q, s, k) is self-consistent;
 *   - range guard: amax^k and amax^k / R_fp8 must both lie in [2^-1022, 2^1023];
 *     if not, k is lowered to the largest fp32 value for which they do;
 *   - a group holding a NaN or Inf moment is "poisoned": k = 1, s = NaN and
 *     every code is 0x7F, so that it decodes to NaN on the next step;
 *   - AdamW is the decoupled-weight-decay form with bias correction at t = step.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FMT_E4M3 0
#define FMT_E5M2 1
#define FMT_NO_EXPAND 0x100

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* ---------------------------------------------------------------------- */
/* FP8 codec (formats per the FP8 guide's bit layouts, OCP semantics)      */
/* ---------------------------------------------------------------------- */

static int fmt_exp_bits(int fmt) { return fmt == FMT_E4M3 ? 4 : 5; }
static int fmt_man_bits(int fmt) { return fmt == FMT_E4M3 ? 3 : 2; }
static int fmt_bias(int fmt) { return fmt == FMT_E4M3 ? 7 : 15; }
/* The largest finite magnitude code: 0x7E (448) for E4M3, 0x7B (57344) for E5M2. */
static int fmt_top_code(int fmt) { return fmt == FMT_E4M3 ? 0x7E : 0x7B; }

/* Value of an FP8 code, straight from its sign, exponent and mantissa fields. */
double coat_oracle_fp8_decode(uint8_t code, int32_t fmt) {
    int eb = fmt_exp_bits(fmt), mb = fmt_man_bits(fmt), bias = fmt_bias(fmt);
    int sign = code >> 7;
    int e = (code >> mb) & ((1 << eb) - 1);
    int m = code & ((1 << mb) - 1);
    double mag;
    if (fmt == FMT_E4M3 && e == 15 && m == 7) {
        mag = NAN;                                   /* E4M3FN: only S.1111.111 is NaN */
    } else if (fmt == FMT_E5M2 && e == 31) {
        mag = (m == 0) ? INFINITY : NAN;             /* E5M2: IEEE-style specials */
    } else if (e == 0) {
        mag = ldexp((double)m, 1 - bias - mb);       /* subnormal: m * 2^(1-bias-mb) */
    } else {
        mag = ldexp(1.0 + (double)m / (double)(1 << mb), e - bias);
    }
    return sign ? -mag : mag;
}

/*
 * Round y to the nearest FP8 value, ties to the even code (the code's low bit
 * is the mantissa's low bit), saturating at the largest finite value.
 * Implemented as a search over the table of finite magnitudes, which are
 * increasing in the code.
 */
uint8_t coat_oracle_fp8_encode(double y, int32_t fmt) {
    if (isnan(y)) return 0x7F;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs(y);
    int top = fmt_top_code(fmt);
    if (a >= coat_oracle_fp8_decode((uint8_t)top, fmt)) return (uint8_t)(sign | top);
    int lo = 0, hi = top; /* invariant: value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (coat_oracle_fp8_decode((uint8_t)mid, fmt) <= a) lo = mid;
        else hi = mid;
    }
    double vlo = coat_oracle_fp8_decode((uint8_t)lo, fmt);
    double vhi = coat_oracle_fp8_decode((uint8_t)hi, fmt);
    double midpoint = 0.5 * (vlo + vhi); /* exact: both are short dyadic numbers */
    int c;
    if (a < midpoint) c = lo;
    else if (a > midpoint) c = hi;
    else c = (lo & 1) ? hi : lo;
    return (uint8_t)(sign | c);
}

void coat_oracle_fp8_decode_array(const uint8_t* q, int64_t n, int32_t fmt, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = coat_oracle_fp8_decode(q[i], fmt);
}

void coat_oracle_fp8_encode_array(const double* y, int64_t n, int32_t fmt, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = coat_oracle_fp8_encode(y[i], fmt);
}

/* ---------------------------------------------------------------------- */
/* Per-group quantization with dynamic range expansion                    */
/* ---------------------------------------------------------------------- */

static double fmt_fpmax(int fmt) { return coat_oracle_fp8_decode((uint8_t)fmt_top_code(fmt), fmt); }
static double fmt_minsub(int fmt) { return coat_oracle_fp8_decode(0x01, fmt); }

/* R_fp8: the format's dynamic range, largest finite over smallest subnormal. */
double coat_oracle_fp8_range(int32_t fmt) { return fmt_fpmax(fmt) / fmt_minsub(fmt); }

/*
 * Range guard: the expanded extremes amax^k and amax^k / R_fp8 must lie in
 * [2^-1022, 2^1023], so that s, every expanded value and every (|q| * s)
 * product of the group is a normal fp64 number.
 */
static int guard_ok(double amax, float k, double rf) {
    double f_max = pow(amax, (double)k);
    return f_max <= 0x1p1023 && f_max / rf >= 0x1p-1022;
}

/*
 * The expansion exponent of one group, from its largest magnitude amax and
 * its smallest nonzero magnitude amin: k = ln(R_fp8) / ln(amax / amin),
 * stored as fp32. k = 1 for near-constant groups or without expansion.
 */
float coat_oracle_group_k(double amax, double amin, int32_t fmt) {
    int expand = !(fmt & FMT_NO_EXPAND);
    int f = fmt & 0xFF;
    double rf = coat_oracle_fp8_range(f);
    float k = 1.0f;
    if (expand && amax > 0.0) {
        double r = amax / amin;
        if (r > 1.0 + 1e-6) k = (float)(log(rf) / log(r));
    }
    if (amax > 0.0 && !guard_ok(amax, k, rf)) {
        /* Lower k to the largest fp32 value, not above the formula's k, that passes. */
        double l2 = log2(amax);
        double bound = (l2 < 0.0) ? (1022.0 - log2(rf)) / -l2 : 1023.0 / l2;
        float kk = (float)bound;
        if (kk > k) kk = k;
        while (kk > 0.0f && !guard_ok(amax, kk, rf)) kk = nextafterf(kk, 0.0f);
        while (nextafterf(kk, INFINITY) <= k && guard_ok(amax, nextafterf(kk, INFINITY), rf))
            kk = nextafterf(kk, INFINITY);
        k = kk;
    }
    return k;
}

/*
 * Quantize one group x[0..len): statistics, k, s = amax^k / fpmax, then each
 * element's expanded magnitude |f(x)| / s = fpmax * (|x| / amax)^k is rounded
 * to the FP8 grid (the quotient form is algebraically |x|^k / s and stays in
 * range). The sign goes into the code's sign bit.
 */
static void quantize_group(const double* x, int64_t len, int32_t fmt, uint8_t* q, double* s_out,
                           float* k_out) {
    int f = fmt & 0xFF;
    double fpmax = fmt_fpmax(f);
    for (int64_t i = 0; i < len; ++i) {
        if (!isfinite(x[i])) {
            for (int64_t j = 0; j < len; ++j) q[j] = 0x7F;
            *s_out = NAN;
            *k_out = 1.0f;
            return;
        }
    }
    double amax = 0.0, amin = INFINITY;
    for (int64_t i = 0; i < len; ++i) {
        double a = fabs(x[i]);
        if (a > amax) amax = a;
        if (a != 0.0 && a < amin) amin = a;
    }
    if (amax == 0.0) {
        for (int64_t i = 0; i < len; ++i) q[i] = signbit(x[i]) ? 0x80 : 0x00;
        *s_out = 0.0;
        *k_out = 1.0f;
        return;
    }
    float k = coat_oracle_group_k(amax, amin, fmt);
    double s = pow(amax, (double)k) / fpmax;
    for (int64_t i = 0; i < len; ++i) {
        uint8_t sign = signbit(x[i]) ? 0x80 : 0x00;
        if (x[i] == 0.0) {
            q[i] = sign;
            continue;
        }
        double y = fpmax * pow(fabs(x[i]) / amax, (double)k);
        q[i] = (uint8_t)(sign | coat_oracle_fp8_encode(y, f));
    }
    *s_out = s;
    *k_out = k;
}

/* x = sign(q) * (|q| * s)^(1/k): the inverse of the expansion, per element. */
static void dequantize_group(const uint8_t* q, int64_t len, int32_t fmt, double s, float k,
                             double* x) {
    int f = fmt & 0xFF;
    double r = 1.0 / (double)k;
    for (int64_t i = 0; i < len; ++i) {
        double v = coat_oracle_fp8_decode(q[i], f);
        double mag = pow(fabs(v) * s, r);
        x[i] = signbit(v) ? -mag : mag;
    }
}

static int check_group_args(int64_t n, int32_t G, int32_t fmt) {
    if (n < 0 || G < 1) return ORACLE_EINVAL;
    int f = fmt & 0xFF;
    if ((f != FMT_E4M3 && f != FMT_E5M2) || (fmt & ~(0xFF | FMT_NO_EXPAND))) return ORACLE_EINVAL;
    return ORACLE_OK;
}

int coat_oracle_quantize(const double* x, int64_t n, int32_t G, int32_t fmt, uint8_t* q, double* s,
                         float* k) {
    if (check_group_args(n, G, fmt)) return ORACLE_EINVAL;
    for (int64_t g0 = 0, gi = 0; g0 < n; g0 += G, ++gi) {
        int64_t len = (n - g0 < G) ? n - g0 : G;
        quantize_group(x + g0, len, fmt, q + g0, s + gi, k + gi);
    }
    return ORACLE_OK;
}

int coat_oracle_dequantize(const uint8_t* q, const double* s, const float* k, int64_t n, int32_t G,
                           int32_t fmt, double* x) {
    if (check_group_args(n, G, fmt)) return ORACLE_EINVAL;
    for (int64_t g0 = 0, gi = 0; g0 < n; g0 += G, ++gi) {
        int64_t len = (n - g0 < G) ? n - g0 : G;
        dequantize_group(q + g0, len, fmt, s[gi], k[gi], x + g0);
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* AdamW on dense fp64 moments                                             */
/* ---------------------------------------------------------------------- */

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round-to-nearest-even fp32 -> bf16; NaN becomes a quiet NaN of the same sign. */
static uint16_t float_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/*
 * One decoupled-weight-decay AdamW step on fp32 master weights with dense
 * fp64 moments m, v (updated in place):
 *   m' = b1 m + (1 - b1) g,   v' = b2 v + (1 - b2) g^2,
 *   p' = p (1 - lr wd) - (lr / (1 - b1^t)) m' / (sqrt(v' / (1 - b2^t)) + eps),
 * then p' is stored as fp32 and its bf16 copy (RNE of the stored fp32) is written.
 */
int coat_oracle_adamw_dense(float* p, uint16_t* w, const uint16_t* g, double* m, double* v,
                            int64_t n, float lr, float b1, float b2, float eps, float wd,
                            int64_t step) {
    if (n < 0 || step < 1) return ORACLE_EINVAL;
    double t = (double)step;
    double bc1 = 1.0 - pow((double)b1, t);
    double bc2 = 1.0 - pow((double)b2, t);
    for (int64_t i = 0; i < n; ++i) {
        double gd = bf16_to_double(g[i]);
        m[i] = (double)b1 * m[i] + (1.0 - (double)b1) * gd;
        v[i] = (double)b2 * v[i] + (1.0 - (double)b2) * gd * gd;
        double pd = (double)p[i] * (1.0 - (double)lr * (double)wd) -
                    ((double)lr / bc1) * m[i] / (sqrt(v[i] / bc2) + (double)eps);
        p[i] = (float)pd;
        if (w) w[i] = float_to_bf16(p[i]);
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* The step: dequantize, AdamW, requantize, group by group                */
/* ---------------------------------------------------------------------- */

int coat_oracle_adamw_step(float* p, uint16_t* w, const uint16_t* g, uint8_t* m_q, double* m_s,
                           float* m_k, uint8_t* v_q, double* v_s, float* v_k, int64_t n, int32_t G,
                           int32_t fmt_m, int32_t fmt_v, float lr, float b1, float b2, float eps,
                           float wd, int64_t step) {
    if (check_group_args(n, G, fmt_m) || check_group_args(n, G, fmt_v) || step < 1)
        return ORACLE_EINVAL;
    double* m = (double*)malloc(sizeof(double) * (size_t)(G > 0 ? G : 1));
    double* v = (double*)malloc(sizeof(double) * (size_t)(G > 0 ? G : 1));
    if (!m || !v) {
        free(m);
        free(v);
        return ORACLE_EINVAL;
    }
    for (int64_t g0 = 0, gi = 0; g0 < n; g0 += G, ++gi) {
        int64_t len = (n - g0 < G) ? n - g0 : G;
        dequantize_group(m_q + g0, len, fmt_m, m_s[gi], m_k[gi], m);
        dequantize_group(v_q + g0, len, fmt_v, v_s[gi], v_k[gi], v);
        coat_oracle_adamw_dense(p + g0, w ? w + g0 : NULL, g + g0, m, v, len, lr, b1, b2, eps, wd,
                                step);
        quantize_group(m, len, fmt_m, m_q + g0, m_s + gi, m_k + gi);
        quantize_group(v, len, fmt_v, v_q + g0, v_s + gi, v_k + gi);
    }
    free(m);
    free(v);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* FP8 activation codec, per tensor or per group                           */
/* ---------------------------------------------------------------------- */
/*
 * Article, section "Solution: mixed-granularity FP8 precision flow": the
 * inputs of linear and non-linear layers are kept in FP8 for the backward pass,
 * and the quantization granularity differs between layers. The page gives no
 * formula. Readings: plain absmax scaling (expansion is described for the
 * optimizer states only); one fp32 scale per tensor (G = 0) or per group of G
 * consecutive elements; bf16 values in and out:
 *   s = RN32(amax / fpmax), amax = max |x| over the tensor or group;
 *   code = encode(RN32(x / s)) if s > 0, else the sign of x alone (all-zero
 *   groups, or amax so small that s underflows to 0);
 *   a tensor or group holding a NaN or Inf: s = NaN and every code 0x7F;
 *   dequantize: RN_bf16(RN32(value(code) * s)).
 * RN32 of an fp64 quotient or product of these operands equals the fp32
 * operation itself: fp64 carries more than 2*24 + 2 bits, so rounding twice is
 * the same as rounding once.
 */
static void act_quantize_block(const uint16_t* x, int64_t len, int32_t fmt, uint8_t* q, float* s_out) {
    double amax = 0.0;
    int bad = 0;
    for (int64_t i = 0; i < len; ++i) {
        double v = bf16_to_double(x[i]);
        if (!isfinite(v)) bad = 1;
        else if (fabs(v) > amax) amax = fabs(v);
    }
    if (bad) {
        *s_out = NAN;
        for (int64_t i = 0; i < len; ++i) q[i] = 0x7F;
        return;
    }
    float s = (float)(amax / fmt_fpmax(fmt));
    *s_out = s;
    for (int64_t i = 0; i < len; ++i) {
        double v = bf16_to_double(x[i]);
        if (s == 0.0f) {
            q[i] = signbit(v) ? 0x80 : 0x00;
            continue;
        }
        float y = (float)(v / (double)s);
        q[i] = coat_oracle_fp8_encode((double)y, fmt);
    }
}

static int check_act_args(int64_t n, int32_t G, int32_t fmt) {
    if (n < 0 || G < 0 || (fmt != FMT_E4M3 && fmt != FMT_E5M2)) return ORACLE_EINVAL;
    return ORACLE_OK;
}

/* G = 0: one scale for the whole array (s[0]); else one per group of G. */
int coat_oracle_act_quantize(const uint16_t* x, int64_t n, int32_t G, int32_t fmt, uint8_t* q, float* s) {
    if (check_act_args(n, G, fmt)) return ORACLE_EINVAL;
    if (G == 0) {
        act_quantize_block(x, n, fmt, q, s);
        return ORACLE_OK;
    }
    for (int64_t g0 = 0, gi = 0; g0 < n; g0 += G, ++gi) {
        int64_t len = (n - g0 < G) ? n - g0 : G;
        act_quantize_block(x + g0, len, fmt, q + g0, s + gi);
    }
    return ORACLE_OK;
}

int coat_oracle_act_dequantize(const uint8_t* q, const float* s, int64_t n, int32_t G, int32_t fmt,
                               uint16_t* x) {
    if (check_act_args(n, G, fmt)) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        float si = s[G == 0 ? 0 : i / G];
        float p = (float)(coat_oracle_fp8_decode(q[i], fmt) * (double)si);
        x[i] = float_to_bf16(p);
    }
    return ORACLE_OK;
}
