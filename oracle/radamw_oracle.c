/*
 * radamw_oracle.c -- reference oracle for the fused AdamW / AMSGrad step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (libradamw.so and its Python binding) never calls it and shares no code,
 * header, constant or helper with it.
 *
 * Plain scalar C, one element at a time in index order, no blocking, no
 * vectorisation hints.  Built with -O2 -ffp-contract=off -fno-fast-math so
 * every float operation below is one IEEE-754 binary32 rounding (x86-64 SSE,
 * FLT_EVAL_METHOD == 0) and nothing is fused or reassociated.
 *
 * Page abbreviations used in the citations:
 *   FA-ja  = RUDA docs page "実験的なデバイス上の融合 AdamW / AMSGrad" (Japanese)
 *   FA-zh  = RUDA docs page "实验性融合 AdamW / AMSGrad" (Chinese)
 *   TR-zh  = RUDA docs page "训练与状态保存" (Chinese)
 *
 * Precision: the pages fix it.  Host coefficients are formed in FP64 with an
 * integer power and then cast to FP32; all per-element arithmetic is FP32
 * (FA-ja, section "この演算子を使用する理由", paragraph after the formula).
 * Gradient statistics are accumulated in FP64 (a reading; see below).
 *
 * Readings where the pages leave a step open (each one is also listed in
 * the design notes of the repository):
 *   - bc1 = 1 - beta1^t and bc2 = 1 - beta2^t are the cast coefficients and
 *     the per-element code divides by them literally;
 *   - 1 - beta1, 1 - beta2 and the decay factor 1 - lr*wd are formed in FP64
 *     on the host and cast to FP32 like the bias factors;
 *   - the unscale divides by the FP32 cast of the (clip-folded) scale, and
 *     maximize negates g after the unscale;
 *   - global-norm clipping is folded into the scale: the scale used is
 *     gradient_scale / clip with clip = min(1, max_norm / (norm + 1e-6)),
 *     norm = sqrt(sum of squares of the stored gradient) / gradient_scale;
 *   - the statistics report holds the FP64 sum of squares of the finite
 *     stored gradient values and the count of non-finite ones, saturating
 *     at 2^32 - 1.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int32_t amsgrad, maximize;
} oracle_options;

typedef struct {
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float bc1, bc2, lr, eps, decay;
} oracle_coefs;

/* beta^t as t successive FP64 multiplications: the plain meaning of an
 * integer power (FA-ja, "この演算子を使用する理由": FP64 integer power on
 * the host). */
static double oracle_int_pow(double base, uint64_t t)
{
    double r = 1.0;
    for (uint64_t k = 0; k < t; ++k)
        r = r * base;
    return r;
}

/* Host-side coefficients for the 1-based update number t: formed once per
 * call in FP64, then cast to FP32 (FA-ja, "この演算子を使用する理由"). */
void oracle_coefficients(const oracle_options *o, uint64_t t, oracle_coefs *c)
{
    c->beta1 = (float)o->beta1;
    c->one_minus_beta1 = (float)(1.0 - o->beta1);
    c->beta2 = (float)o->beta2;
    c->one_minus_beta2 = (float)(1.0 - o->beta2);
    c->bc1 = (float)(1.0 - oracle_int_pow(o->beta1, t));
    c->bc2 = (float)(1.0 - oracle_int_pow(o->beta2, t));
    c->lr = (float)o->lr;
    c->eps = (float)o->eps;
    c->decay = (float)(1.0 - o->lr * o->weight_decay);
}

/* IEEE-754 binary16 -> binary32, exact, written out from the format's
 * definition (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits). */
static float oracle_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exponent = (h >> 10) & 0x1f;
    int fraction = h & 0x3ff;
    float magnitude;
    if (exponent == 0) {
        /* zero or subnormal: fraction * 2^-24 (exact in binary32) */
        magnitude = ldexpf((float)fraction, -24);
    } else if (exponent == 31) {
        magnitude = fraction == 0 ? INFINITY : NAN;
    } else {
        /* (1024 + fraction) * 2^(exponent - 25) */
        magnitude = ldexpf((float)(1024 + fraction), exponent - 25);
    }
    return sign ? -magnitude : magnitude;
}

/* bfloat16 -> binary32: the stored 16 bits are the upper half of a binary32. */
static float oracle_bf16_to_float(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Widen element i of a stored gradient of the given dtype to FP32 (exact). */
float oracle_widen(const void *grad, int32_t dtype, int64_t i)
{
    if (dtype == ORACLE_F32)
        return ((const float *)grad)[i];
    if (dtype == ORACLE_F16)
        return oracle_half_to_float(((const uint16_t *)grad)[i]);
    return oracle_bf16_to_float(((const uint16_t *)grad)[i]);
}

/*
 * One AdamW / AMSGrad update over n elements, in place on host arrays.
 *
 * Formula: FA-ja, section "この演算子を使用する理由" (the per-element block
 * and the paragraph after it): unscale (negate when maximizing), first and
 * second moment EMAs, AMSGrad running max kept uncorrected, bias correction
 * with epsilon added after the square root, decoupled weight decay applied
 * to p only.
 *
 * *step is the number of completed updates; this call performs update
 * t = *step + 1.  *step == 0 means there is no state yet (the Rust API's
 * state None, FA-ja "低レベルの使用"): the moments start from zero inside
 * the update and m, v, vmax are written without being read (FA-zh
 * "增加的实际能力").  skip_update or n == 0 returns 0 before anything is
 * touched and leaves *step unchanged (FA-zh "增加的实际能力").
 * vmax is used only when o->amsgrad is set.
 *
 * gradient_scale is the divisor applied to the stored gradient (already
 * folded with any clip coefficient).  Returns 1 when the update ran.
 */
int32_t oracle_adamw_step(float *p, const void *grad, int32_t dtype, int64_t n,
                          float *m, float *v, float *vmax, uint64_t *step,
                          const oracle_options *o, double gradient_scale,
                          int32_t skip_update)
{
    if (skip_update || n == 0)
        return 0;

    uint64_t t = *step + 1;
    oracle_coefs c;
    oracle_coefficients(o, t, &c);
    float scale = (float)gradient_scale;
    int first = (*step == 0);

    for (int64_t i = 0; i < n; ++i) {
        float x = oracle_widen(grad, dtype, i);
        float g = x / scale;
        if (o->maximize)
            g = -g;

        float m_old = first ? 0.0f : m[i];
        float v_old = first ? 0.0f : v[i];

        float m_new = c.beta1 * m_old + c.one_minus_beta1 * g;
        float v_new = c.beta2 * v_old + (c.one_minus_beta2 * g) * g;

        float v_used = v_new;
        if (o->amsgrad) {
            float vmax_old = first ? 0.0f : vmax[i];
            v_used = fmaxf(vmax_old, v_new);
            vmax[i] = v_used; /* saved without bias correction */
        }

        float m_hat = m_new / c.bc1;
        float v_hat = v_used / c.bc2;
        float denom = sqrtf(v_hat) + c.eps;
        float update = (c.lr * m_hat) / denom;

        p[i] = p[i] * c.decay - update;
        m[i] = m_new;
        v[i] = v_new;
    }
    *step = t;
    return 1;
}

/*
 * Gradient statistics (the read-only analysis pass of FA-ja "ネイティブ
 * PyTorch ストレージと階層統計" and TR-zh "在 ruda:0 上进行原生 PyTorch
 * 训练"): adds the squares of the finite stored values, in index order in
 * FP64, to *sumsq, and the number of non-finite values to *nonfinite,
 * saturating at 2^32 - 1.  Continuing the running pair over several
 * tensors gives the statistics of their concatenation.
 */
void oracle_grad_stats_accumulate(const void *grad, int32_t dtype, int64_t n,
                                  double *sumsq, uint32_t *nonfinite)
{
    double s = *sumsq;
    uint32_t count = *nonfinite;
    for (int64_t i = 0; i < n; ++i) {
        float x = oracle_widen(grad, dtype, i);
        if (isfinite(x)) {
            double d = (double)x;
            s = s + d * d;
        } else if (count != UINT32_MAX) {
            count = count + 1;
        }
    }
    *sumsq = s;
    *nonfinite = count;
}

/*
 * Merge plan for the hierarchical statistics (FA-ja "ネイティブ PyTorch
 * ストレージと階層統計"; TR-zh "在 ruda:0 上进行原生 PyTorch 训练"):
 * rows must lie in 1..4,194,304; while more than 1024 records remain, one
 * extra merge level reduces each group of up to 1024 records to one.
 * *scratch_elements counts FP32 elements (three per 12-byte record) of all
 * intermediate levels, excluding the initial rows and the final report.
 * Returns 0, or -1 when rows is out of range.
 */
int32_t oracle_stats_plan(int64_t rows, int64_t *scratch_elements,
                          int32_t *extra_merge_kernels)
{
    if (rows < 1 || rows > 4194304)
        return -1;
    int64_t remaining = rows;
    int64_t records = 0;
    int32_t levels = 0;
    while (remaining > 1024) {
        remaining = (remaining + 1023) / 1024;
        records += remaining;
        levels += 1;
    }
    *scratch_elements = 3 * records;
    *extra_merge_kernels = levels;
    return 0;
}

/* Global-norm clip coefficient, applied after unscaling (TR-zh "在 ruda:0 上
 * 进行原生 PyTorch 训练").  norm = sqrt(sumsq) / gradient_scale;
 * coefficient = min(1, max_norm / (norm + 1e-6)); max_norm <= 0 means no
 * clipping. */
double oracle_clip_coefficient(double sumsq, double gradient_scale,
                               double max_norm)
{
    if (max_norm <= 0.0)
        return 1.0;
    double norm = sqrt(sumsq) / gradient_scale;
    double coef = max_norm / (norm + 1e-6);
    return coef < 1.0 ? coef : 1.0;
}

/*
 * Low-precision copy of the updated FP32 master parameters (the model copy
 * an FP32-master optimizer maintains; TR-zh "训练与状态保存": FP32 master
 * parameters, FP16 / BF16 model storage).  Round to nearest, ties to even,
 * written out from the two formats' definitions.
 */

/* bfloat16: keep the upper 16 bits of the binary32 encoding, rounding on the
 * lower 16 (ties to the even upper half); a NaN stays a (quiet) NaN. */
uint16_t oracle_round_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if (isnan(x))
        return (uint16_t)((u >> 16) | 0x0040);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1; /* a carry into the exponent is the correct next value */
    return (uint16_t)upper;
}

/* IEEE binary16: the representable values near |x| are multiples of the
 * quantum 2^(E-10) for a normal binade [2^E, 2^(E+1)) and 2^-24 below 2^-14;
 * round |x| to the nearest multiple (ties to even, rint in the default
 * rounding mode), saturate to infinity above 65504, then encode. */
uint16_t oracle_round_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return sign | 0x7e00;
    double a = fabs((double)x);
    if (isinf(a))
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1): binade exponent e2 - 1 */
    int binade = e2 - 1;
    int qexp = binade < -14 ? -24 : binade - 10;
    double q = rint(ldexp(a, -qexp)); /* quanta, exact integer */
    double v = ldexp(q, qexp);        /* the rounded magnitude */
    if (v > 65504.0)
        return sign | 0x7c00;
    if (qexp == -24)
        return sign | (uint16_t)q; /* subnormal count; q == 1024 encodes 2^-14 */
    frexp(v, &e2);
    binade = e2 - 1; /* may have moved up one binade by rounding */
    uint16_t mant = (uint16_t)(ldexp(v, 10 - binade) - 1024.0);
    return sign | (uint16_t)((binade + 15) << 10) | mant;
}

/* Round n FP32 values to the copy's dtype (ORACLE_F16 or ORACLE_BF16). */
void oracle_round_copy(const float *p, int64_t n, int32_t dtype, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == ORACLE_F16 ? oracle_round_f16(p[i]) : oracle_round_bf16(p[i]);
}
