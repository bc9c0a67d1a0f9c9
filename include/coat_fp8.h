/*
 * coat_fp8.h - C ABI of the MI355X (gfx950) FP8-optimizer-state AdamW step.
 *
 * The method is COAT's optimizer with FP8-compressed Adam state as described
 * in "COAT: FP8 training, 40% less memory, 1.4x faster" (blob.wenxiaobai.com),
 * sections "FP8 optimizer states" and "Solution: dynamic range expansion",
 * and in its mirror on zhanchiexpo.com (per-group quantization of the states).
 * The FP8 bit layouts are those of the FP8 guide on maplevalley.com.cn,
 * section "format choice" (E4M3 = 1+4+3 bits, E5M2 = 1+5+2 bits), with OCP
 * E4M3FN / E5M2 semantics.
 *
 * State layout (everything flat, row-major, owned by the caller):
 *   - a tensor of n parameters is cut into groups of G consecutive elements
 *     (the last group may be shorter); groups never span tensors;
 *   - for each of the two Adam moments (m: first, v: second) the state is
 *       q[n]            uint8 FP8 codes (sign bit | magnitude code),
 *       s[ceil(n/G)]    fp64 per-group scale,
 *       k[ceil(n/G)]    fp32 per-group expansion exponent,
 *     and a stored code decodes to x = sign(q) * (|q| * s)^(1/k);
 *   - requantizing a group takes amax = max|x| and amin = min over nonzero |x|,
 *     k = ln(R_fp8) / ln(amax/amin) (k = 1 if amax/amin <= 1 + 1e-6, if the
 *     group is all zero, or with COAT_FMT_NO_EXPAND), s = amax^k / fpmax, and
 *     rounds fpmax * (|x| / amax)^k to the FP8 grid, nearest, ties to even,
 *     saturating at fpmax. R_fp8 = fpmax / min subnormal: 448 / 2^-9 for E4M3,
 *     57344 / 2^-16 for E5M2. k is lowered when needed so that amax^k and
 *     amax^k / R_fp8 stay within [2^-1022, 2^1023]. A group holding a
 *     non-finite moment is stored with s = NaN, k = 1 and every code 0x7F.
 *
 * Conventions for every entry point:
 *   - all array pointers are device pointers (HIP device memory) owned by the
 *     caller; the library allocates nothing and keeps no state between calls,
 *     except the device table array of coat_fp8_adamw_step_multi_static;
 *   - work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting; device-side faults surface at the
 *     caller's next synchronization;
 *   - arrays must not overlap one another; in/out arrays are updated in place;
 *   - the byte arrays (codes), fp32 and bf16 arrays must start on a 16-byte
 *     boundary; s and k arrays need their natural alignment;
 *   - group G must be a power of two in [16, 1024];
 *   - return value: COAT_OK, or a negative status (see coat_strerror); on
 *     error nothing has been enqueued, except where COAT_EHIP is said to
 *     leave earlier launches of the same call.
 */
#ifndef COAT_FP8_H
#define COAT_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t, declared here so that this header needs no HIP include. */
typedef struct ihipStream_t* coat_stream_t;

enum {
    COAT_FMT_E4M3 = 0,          /* OCP E4M3FN: bias 7, max 448, NaN 0x7F/0xFF, no Inf */
    COAT_FMT_E5M2 = 1,          /* OCP E5M2: bias 15, max 57344, Inf 0x7C/0xFC */
    COAT_FMT_NO_EXPAND = 0x100  /* flag OR-ed into a format: force k = 1 (plain absmax) */
};

enum {
    COAT_OK = 0,
    COAT_EINVAL = -1, /* null pointer with n > 0, n < 0, bad group or format, step < 1,
                         non-finite hyperparameter, workspace too small */
    COAT_EALIGN = -2, /* a pointer does not meet the alignment stated above */
    COAT_EHIP = -3,   /* the HIP runtime refused the launch */
    COAT_ERANGE = -4  /* more tensors than COAT_STATIC_MAX_TENSORS (static-table entry point) */
};

/*
 * One AdamW step over FP8-compressed moments of one tensor (COAT's optimizer
 * step, article section "FP8 optimizer states"; the update is decoupled
 * weight decay AdamW with bias correction at t = step):
 *   m' = b1 m + (1 - b1) g,  v' = b2 v + (1 - b2) g^2,
 *   p' = p (1 - lr wd) - (lr / (1 - b1^t)) m' / (sqrt(v' / (1 - b2^t)) + eps),
 * where m, v are the dequantized stored moments; then m', v' are requantized
 * group by group with dynamic range expansion.
 *
 *   params       fp32 master weights, n, in/out
 *   params_bf16  bf16 copy of the new master weights (RNE), n, out; may be NULL
 *   grads        bf16 gradients, n, in
 *   m_q,m_s,m_k  first-moment codes (n), scales and exponents (ceil(n/G)), in/out
 *   v_q,v_s,v_k  second-moment state, same shapes, in/out
 *   fmt_m/fmt_v  COAT_FMT_E4M3 or COAT_FMT_E5M2, optionally | COAT_FMT_NO_EXPAND
 *   step         t >= 1, the step being taken
 * The stored moments are states written by coat_fp8_quantize or by an earlier
 * step (an all-zero group stores s = 0 with signed-zero codes, a poisoned
 * group s = NaN with NaN codes). For states neither writes (an Inf code under
 * a zero or NaN scale, a scale of +Inf) the result is unspecified.
 */
int coat_fp8_adamw_step(float* params, uint16_t* params_bf16, const uint16_t* grads,
                        uint8_t* m_q, double* m_s, float* m_k,
                        uint8_t* v_q, double* v_s, float* v_k,
                        int64_t n, int32_t group, int32_t fmt_m, int32_t fmt_v,
                        float lr, float beta1, float beta2, float eps, float weight_decay,
                        int64_t step, coat_stream_t stream);

/* One tensor of a parameter list for the multi-tensor step; fields as above. */
typedef struct coat_tensor {
    float* params;
    uint16_t* params_bf16; /* may be NULL */
    const uint16_t* grads;
    uint8_t* m_q;
    double* m_s;
    float* m_k;
    uint8_t* v_q;
    double* v_s;
    float* v_k;
    int64_t n;            /* 0 allowed: the tensor is skipped */
} coat_tensor;

/* Bytes of device workspace a plan over `count` tensors needs. */
size_t coat_multi_workspace_bytes(int32_t count);

/*
 * A parameter list prepared for repeated multi-tensor steps: the descriptor
 * table and the tile table live in caller-owned device workspace.
 */
typedef struct coat_multi_plan {
    void* workspace;    /* device memory holding the tables */
    int32_t count;      /* tensors */
    int64_t tiles;      /* 1024-element tiles across all tensors */
    int64_t n_total;    /* parameters across all tensors */
    int32_t n_partial;  /* tensors whose size is not a multiple of 1024 */
} coat_multi_plan;

/*
 * Validate `count` descriptors (host array) and enqueue on `stream` their copy,
 * with a tile table, into `workspace` (device memory, 256-byte aligned, at
 * least coat_multi_workspace_bytes(count) bytes). The tables travel in the
 * arguments of small copy launches, one per 3 KB of tables (11 for the 363
 * tensors of a Llama-2-13B list), so the call neither stages through host
 * memory nor waits: it returns once they are enqueued, and the host array
 * `tensors` is read during the call only. Steps
 * enqueued after it on the same stream see the tables; a step on another
 * stream must be ordered after them by the caller. The plan stays valid while
 * the tensors' buffers and the workspace do. COAT_EHIP (a refused launch) may
 * leave the copies before it enqueued.
 */
int coat_multi_plan_init(coat_multi_plan* plan, const coat_tensor* tensors, int32_t count,
                         void* workspace, size_t workspace_bytes, coat_stream_t stream);

/*
 * One step over every tensor of a plan, asynchronous: one kernel launch over
 * the whole list (for G >= 128 a second, small one when some tensor ends
 * inside a 1024-element tile: its last tile). The result equals calling
 * coat_fp8_adamw_step on each tensor in turn, bit for bit.
 */
int coat_fp8_adamw_step_planned(const coat_multi_plan* plan, int32_t group, int32_t fmt_m,
                                int32_t fmt_v, float lr, float beta1, float beta2, float eps,
                                float weight_decay, int64_t step, coat_stream_t stream);

/*
 * Convenience: coat_multi_plan_init followed by coat_fp8_adamw_step_planned
 * (it enqueues the table copies, then the step, all on `stream`, and returns
 * without waiting).
 */
int coat_fp8_adamw_step_multi(const coat_tensor* tensors, int32_t count, int32_t group,
                              int32_t fmt_m, int32_t fmt_v, float lr, float beta1, float beta2,
                              float eps, float weight_decay, int64_t step, void* workspace,
                              size_t workspace_bytes, coat_stream_t stream);

/* Largest parameter list coat_fp8_adamw_step_multi_static accepts. */
#define COAT_STATIC_MAX_TENSORS 4096

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * multi-tensor step of coat_fp8_adamw_step_multi with its plan tables kept in
 * a device array inside the library instead of a caller workspace. It takes
 * the same arguments minus the workspace, calls no allocator (no hipMalloc,
 * no hipFree, no host staging buffer) and does not synchronize: it enqueues a
 * few small copy launches that carry the tables in their kernel arguments,
 * then the step, all on `stream`, and returns. The result equals
 * coat_fp8_adamw_step_multi's bit for bit.
 *   - count <= COAT_STATIC_MAX_TENSORS (4096), else COAT_ERANGE before anything
 *     is enqueued; other errors as for coat_fp8_adamw_step_multi;
 *   - each GPU holds one copy of the table array (about 377 KB) from its
 *     first call until the process ends; it is looked up once per device with
 *     that device current, so `stream` must belong to the current device;
 *   - every call on a GPU rewrites that GPU's one array: calls that may
 *     overlap on one GPU (other streams, other host threads without ordering)
 *     race, so they must be serialized, e.g. issued on one stream; the array
 *     keeps the last call's tables, and every entry the step reads is
 *     written by the call itself, so nothing has to start cleared;
 *   - the host array `tensors` is read during the call only;
 *   - COAT_EHIP (a refused launch) may leave the copies before it enqueued.
 */
int coat_fp8_adamw_step_multi_static(const coat_tensor* tensors, int32_t count, int32_t group,
                                     int32_t fmt_m, int32_t fmt_v, float lr, float beta1,
                                     float beta2, float eps, float weight_decay, int64_t step,
                                     coat_stream_t stream);

/*
 * Quantize an fp32 array into FP8 state (q, s, k) with per-group dynamic
 * range expansion, exactly as the step requantizes a moment (article section
 * "Solution: dynamic range expansion"). Used to initialise or import state.
 *   x in (n), q out (n), s/k out (ceil(n/G)).
 */
int coat_fp8_quantize(const float* x, int64_t n, int32_t group, int32_t fmt, uint8_t* q,
                      double* s, float* k, coat_stream_t stream);

/*
 * Dequantize FP8 state to fp32: x = sign(q) (|q| s)^(1/k), the value the step
 * starts from (in fp64), to within one fp32 ulp (the power is evaluated to
 * about 2^-28 before the rounding to fp32). Used to export state.
 */
int coat_fp8_dequantize(const uint8_t* q, const double* s, const float* k, int64_t n,
                        int32_t group, int32_t fmt, float* x, coat_stream_t stream);

/*
 * Plain FP8 codec on fp32 values (no scaling, no expansion): encode rounds to
 * nearest, ties to even, saturating at the largest finite value, NaN -> 0x7F;
 * decode is exact. Formats as in the FP8 guide, section "format choice".
 */
int coat_fp8_encode(const float* y, int64_t n, int32_t fmt, uint8_t* q, coat_stream_t stream);
int coat_fp8_decode(const uint8_t* q, int64_t n, int32_t fmt, float* y, coat_stream_t stream);

/*
 * FP8 activation codec with per-tensor or per-group granularity (article
 * section "Solution: mixed-granularity FP8 precision flow": layer inputs are
 * kept in FP8 for the backward pass, the quantization granularity varying
 * between layers; which layer takes which granularity is the caller's
 * choice). Plain absmax scaling of bf16 values, no expansion:
 *   group == 0: one scale for the whole array (scale[1]);
 *   group = G, a power of two in [16, 1024]: one scale per G consecutive
 *   values (scale[ceil(n/G)], the last group may be short);
 *   s = RN32(amax / fpmax); code = encode(RN32(x / s)) rounded to nearest,
 *   ties to even, saturating (for s = 0, an all-zero group, the sign alone);
 *   a tensor or group holding a NaN or Inf: s = NaN and every code 0x7F.
 * Dequantize writes RN_bf16(RN32(decode(code) * s)).
 *   x bf16 in (n), q out (n), scale out; fmt COAT_FMT_E4M3 or COAT_FMT_E5M2
 *   (no flags). x, q 16-byte aligned (COAT_EALIGN), scale 4-byte aligned.
 * Per tensor, the quantizer uses scale[0] as its accumulator while it runs
 * (it enqueues four small launches); the caller must not read it until the
 * stream reaches the end of the call.
 */
int coat_fp8_act_quantize(const uint16_t* x, int64_t n, int32_t group, int32_t fmt, uint8_t* q,
                          float* scale, coat_stream_t stream);
int coat_fp8_act_dequantize(const uint8_t* q, const float* scale, int64_t n, int32_t group,
                            int32_t fmt, uint16_t* x, coat_stream_t stream);

/* Static description of a status code. */
const char* coat_strerror(int status);

/* ABI version of this library (major * 100 + minor). */
int coat_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* COAT_FP8_H */
