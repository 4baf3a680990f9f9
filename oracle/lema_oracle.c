/*
 * lema_oracle.c -- plain CPU oracle for the mixed-precision AdamW path.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  The product
 * path (optimizer_step_lema_amd/) never links, loads or calls it, and this
 * file shares no code, header or table with the product.
 *
 * What it computes (one trained tensor, element by element):
 *
 *   LEMA README, "Quick Start": every trainable parameter is handed to
 *   torch.optim.AdamW with lr = 1e-4 and otherwise default settings, i.e.
 *   the AdamW algorithm (decoupled weight decay, bias-corrected first and
 *   second moments, no AMSGrad).
 *   LEMA README, "Selective Full Fine-Tuning": the optimizer runs per layer
 *   and its states and the gradient accumulators are fp32.
 *   LLMScale fine-tuning VRAM page, memory note and FAQ: mixed-precision
 *   Adam keeps a bf16 working weight, a bf16 gradient and fp32 master,
 *   m and v (16 bytes per trained parameter).
 *   LEMA README, "Selective Full Fine-Tuning" (checkpoint paragraph): a
 *   checkpoint stores an fp32 delta, updated weight minus original weight.
 *
 * The pages print no formula, so the rounding points are fixed here (each
 * reading is listed in the design notes of the repository):
 *   - the eight fp32 constants are derived in double precision and each is
 *     rounded once to fp32; beta^t uses square-and-multiply in double;
 *   - per element every operation is one IEEE binary32 operation rounded to
 *     nearest even, in the order written below, with no fused multiply-add
 *     (build with -ffp-contract=off, no fast-math, SSE arithmetic);
 *   - sqrt and division are the correctly rounded binary32 operations;
 *   - the bf16 working weight is round-to-nearest-even of the fp32 master.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ bits */

static float bits_to_float(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t float_to_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* bf16 -> fp32 is exact: the bf16 pattern is the upper half of an fp32. */
float oracle_bf16_to_f32(uint16_t b)
{
    return bits_to_float((uint32_t)b << 16);
}

/*
 * fp32 -> bf16, IEEE round to nearest, ties to even, on the 16 dropped
 * bits.  A carry out of the mantissa moves into the exponent, so the largest
 * finite values round up to infinity exactly as IEEE prescribes.  NaN stays
 * NaN: its sign and top payload bits are kept and the quiet bit is set.
 */
uint16_t oracle_rne16(float x)
{
    uint32_t u = float_to_bits(x);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;

    if ((u & 0x7FFFFFFFu) > 0x7F800000u)          /* NaN */
        return (uint16_t)(kept | 0x0040u);

    if (dropped > 0x8000u)                         /* above the half-way point */
        kept += 1u;
    else if (dropped == 0x8000u && (kept & 1u))    /* tie: go to the even one */
        kept += 1u;
    return (uint16_t)kept;
}

void oracle_rne16_array(int64_t n, const float *x, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_rne16(x[i]);
}

/* ------------------------------------------------------------- constants */

/* beta^t by square-and-multiply, scanning t from its least significant bit. */
static double power_by_squaring(double base, int64_t t)
{
    double result = 1.0;
    while (t > 0) {
        if (t & 1)
            result = result * base;
        base = base * base;
        t >>= 1;
    }
    return result;
}

/*
 * The eight per-call fp32 constants of one AdamW step number t (t >= 1 is
 * the step being taken).  Order of the output array:
 *   [0] beta1          [1] 1 - beta1
 *   [2] beta2          [3] 1 - beta2
 *   [4] eps            [5] 1 - lr*wd          (decoupled weight decay factor)
 *   [6] lr / (1 - beta1^t)                    (step size with bias correction 1)
 *   [7] 1 / sqrt(1 - beta2^t)                 (inverse bias correction 2 root)
 * Each value is computed in double and rounded to fp32 once.
 */
void oracle_adamw_constants(double lr, double beta1, double beta2, double eps,
                            double weight_decay, int64_t t, float out[8])
{
    double bc1 = 1.0 - power_by_squaring(beta1, t);
    double bc2 = 1.0 - power_by_squaring(beta2, t);

    out[0] = (float)beta1;
    out[1] = (float)(1.0 - beta1);
    out[2] = (float)beta2;
    out[3] = (float)(1.0 - beta2);
    out[4] = (float)eps;
    out[5] = (float)(1.0 - lr * weight_decay);
    out[6] = (float)(lr / bc1);
    out[7] = (float)(1.0 / sqrt(bc2));
}

/* ------------------------------------------------------------ AdamW step */

/*
 * One AdamW step over n elements of one tensor, in place on master, m, v.
 *   grad        : n bf16 patterns (grad_is_f32 == 0) or n fp32 values
 *   weight_out  : n bf16 patterns, rne16 of the new master
 *   orig, delta : both NULL, or n bf16 base weights and n fp32 outputs
 *                 delta = new master - f32(orig)
 *   c           : constants from oracle_adamw_constants
 */
void oracle_adamw(int64_t n, float *master, float *m, float *v,
                  const void *grad, int grad_is_f32, uint16_t *weight_out,
                  const uint16_t *orig, float *delta, const float c[8])
{
    const float b1 = c[0], one_minus_b1 = c[1];
    const float b2 = c[2], one_minus_b2 = c[3];
    const float eps = c[4], decay = c[5], step_size = c[6], inv_bc2_root = c[7];
    const uint16_t *grad_bf16 = (const uint16_t *)grad;
    const float *grad_f32 = (const float *)grad;

#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float g = grad_is_f32 ? grad_f32[i] : oracle_bf16_to_f32(grad_bf16[i]);

        /* decoupled weight decay on the weight before the update */
        float w_decayed = master[i] * decay;

        /* first and second moments */
        float m_old_part = b1 * m[i];
        float m_new_part = one_minus_b1 * g;
        float m_new = m_old_part + m_new_part;

        float g_squared = g * g;
        float v_old_part = b2 * v[i];
        float v_new_part = one_minus_b2 * g_squared;
        float v_new = v_old_part + v_new_part;

        /* bias-corrected denominator: sqrt(v_hat) + eps */
        float root = sqrtf(v_new);
        float root_hat = root * inv_bc2_root;
        float denom = root_hat + eps;

        /* bias-corrected update */
        float ratio = m_new / denom;
        float update = step_size * ratio;
        float w_new = w_decayed - update;

        master[i] = w_new;
        m[i] = m_new;
        v[i] = v_new;
        weight_out[i] = oracle_rne16(w_new);
        if (delta)
            delta[i] = w_new - oracle_bf16_to_f32(orig[i]);
    }
}

/* ------------------------------------------------- gradient accumulation */

/*
 * fp32 accumulation of one bf16 micro-batch gradient (LEMA README,
 * "Selective Full Fine-Tuning": gradient accumulation is fp32).
 *   overwrite != 0 : acc = f32(g)           (first micro-batch; -0 is kept)
 *   overwrite == 0 : acc = acc + f32(g)     (later micro-batches, in order)
 */
void oracle_accum(int64_t n, float *acc, const uint16_t *g, int overwrite)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float gi = oracle_bf16_to_f32(g[i]);
        if (overwrite)
            acc[i] = gi;
        else
            acc[i] = acc[i] + gi;
    }
}

/* ---------------------------------------------------------- merge delta */

/*
 * A servable bf16 weight from a base checkpoint and a saved delta (LEMA
 * README, "Selective Full Fine-Tuning": merge_delta(base, delta, merged)
 * produces a full model from the base weights and the fp32 delta):
 *   merged = rne16(f32(base) + delta)      one binary32 addition, then bf16
 */
void oracle_merge_delta(int64_t n, const uint16_t *base, const float *delta, uint16_t *merged)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float sum = oracle_bf16_to_f32(base[i]) + delta[i];
        merged[i] = oracle_rne16(sum);
    }
}

/* ------------------------------------------------- int8 rows with scales */

/*
 * The int8 + per-row-scale storage of quantized optimizer moments and
 * gradient accumulators (LEMA README, "Quantization": opt_state_bits = 8 and
 * grad_acc_bits = 8 keep these classes as int8 codes with one scale per row,
 * dequantized only inside the per-layer AdamW step).  The pages name the
 * format but give no formula; the reading fixed here is symmetric absmax
 * scaling:
 *
 *   A tensor of n elements is cut into rows of row_len consecutive elements
 *   (the last row may be shorter), rows = ceil(n / row_len).  For a 2-D
 *   [out x in] weight row_len = in gives the matrix rows.
 *   Row r holds int8 codes q[i] in [-127, 127] and one fp32 scale s[r].
 *   dequantize: x[i] = (float)q[i] * s[r]        one binary32 multiplication
 *   quantize  : a    = max |x[i]| over the row   (NaN if the row has a NaN)
 *               s[r] = a / 127                   binary32 division
 *               if s[r] is finite and > 0:
 *                   q[i] = round-half-even(x[i] / s[r]) clamped to [-127, 127]
 *                   (x[i] / s[r] is a binary32 division)
 *               otherwise q[i] = 0 (an all-zero row, an absmax whose division
 *               underflows to 0, or a row holding an infinity or a NaN; the
 *               last two dequantize to NaN everywhere since 0*inf and 0*NaN
 *               are NaN)
 */
static float row_absmax(const float *x, int64_t len)
{
    float a = 0.0f;
    int saw_nan = 0;
    for (int64_t i = 0; i < len; ++i) {
        float ax = fabsf(x[i]);
        if (isnan(ax))
            saw_nan = 1;
        else if (ax > a)
            a = ax;
    }
    return saw_nan ? NAN : a;
}

static int8_t quantize_one(float x, float scale)
{
    if (!(isfinite(scale) && scale > 0.0f))
        return 0;
    float r = x / scale;
    float k = rintf(r);                /* default rounding mode: half to even */
    if (k > 127.0f)
        k = 127.0f;
    if (k < -127.0f)
        k = -127.0f;
    return (int8_t)k;
}

void oracle_quantize_rows(int64_t n, int64_t row_len, const float *x, int8_t *q, float *scale)
{
    int64_t rows = (n + row_len - 1) / row_len;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t lo = r * row_len;
        int64_t len = (n - lo < row_len) ? n - lo : row_len;
        float s = row_absmax(x + lo, len) / 127.0f;
        scale[r] = s;
        for (int64_t i = 0; i < len; ++i)
            q[lo + i] = quantize_one(x[lo + i], s);
    }
}

void oracle_dequantize_rows(int64_t n, int64_t row_len, const int8_t *q, const float *scale,
                            float *x)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        x[i] = (float)q[i] * scale[i / row_len];
}

/* Threads the OpenMP runtime will use for the loops above. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads of later loops (n >= 1); results do not depend on it,
 * every element being computed alone. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}
