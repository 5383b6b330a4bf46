/*
 * ck_oracle.c -- plain CPU oracle for the INT8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path
 * (int8_weight_quantized_amd/) never loads, calls or links it, and this file
 * shares no code, header, table or constant with the HIP kernels.
 *
 * What it computes is the plain definition of the three-step INT8 linear
 * layer that the comfy-kitchen pages describe:
 *
 *   1. per-row (or tensor-wide) activation quantisation, bf16 -> int8 codes
 *      plus an fp32 scale  (comfy-kitchen #278 "int8_linear silently falls
 *      back ... on Volta", section "Two separate problems", item 2, names the
 *      operation quantize_int8_rowwise; #280 "INT8 linears on sm_121 ...",
 *      Summary, names the tensor-wide variant);
 *   2. an int8 x int8 product with an int32 accumulator over K, which is
 *      exact (#280, sections "Kernel used" and "Exactness");
 *   3. an fp32 epilogue acc * x_scale[m] * w_scale[n] (+ bias[n]) evaluated
 *      left to right and rounded once to the output type (#280, sections
 *      "Kernel used" and "Exactness"): bf16, or fp16 or fp32, the other two
 *      output types that page's exactness audit covered.
 *
 * Readings taken where the pages are silent:
 *   - scale s = amax / 127 as a correctly rounded fp32 division, where amax
 *     is the largest |x| of the row (or of the tensor);
 *   - code q = clamp(rint(x / s), -127, 127): x widened exactly to fp32,
 *     true fp32 division (not a multiply by 127/amax), rint in the default
 *     round-half-to-even mode; an all-zero row has s = 0 and all codes 0;
 *   - int32 -> fp32 rounds to nearest even; each epilogue operation is one
 *     fp32 rounding, with no fused multiply-add (build with
 *     -ffp-contract=off); the fp32 -> bf16 and fp32 -> fp16 output roundings
 *     are round-to-nearest-even (fp16 overflows to infinity from 65520 on);
 *     fp32 output is the fp32 result itself;
 *   - the bias has the output's type (fp32 for fp32 output) and is widened
 *     exactly to fp32 before the add.
 *
 * Precision: the pages fix the epilogue at fp32 and the accumulator at
 * int32.  They do not fix the quantisation precision; the code is an integer
 * decided by floating point, so the oracle takes that decision in the same
 * precision as the kernel, fp32.  Accumulation here is done in int64 and the
 * result is checked to fit in int32 (a return value of -1 reports overflow).
 *
 * Parallelism: OpenMP over independent output elements only; no blocking,
 * no reordering of any sum.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

/* ---- bf16 <-> fp32 -------------------------------------------------------
 * A bf16 value is the upper 16 bits of the binary32 value with the same
 * sign, exponent and top 7 fraction bits, so widening is exact. */
float ck_oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static double f32_bits_value(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* fp32 -> bf16, round to nearest, ties to even, written as the definition:
 * the two bf16 candidates are the truncation toward zero and the next bf16
 * away from zero; take the nearer, and on a tie the one whose last stored
 * fraction bit is 0.  Distances are computed in double, where the
 * difference of two floats of this size is exact.  Past the largest finite
 * bf16 the upper candidate is 2^128 (infinity once chosen). */
uint16_t ck_oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u) {           /* inf or NaN */
        if (u & 0x007fffffu) return (uint16_t)((u >> 16) | 0x0040u);
        return (uint16_t)(u >> 16);
    }
    uint32_t lo = u & 0xffff0000u;
    if (lo == u) return (uint16_t)(u >> 16);           /* already a bf16 */
    uint32_t hi = lo + 0x00010000u;
    double x = (double)f;
    double vlo = f32_bits_value(lo);
    double vhi;
    if ((hi & 0x7f800000u) == 0x7f800000u)
        vhi = (u & 0x80000000u) ? -ldexp(1.0, 128) : ldexp(1.0, 128);
    else
        vhi = f32_bits_value(hi);
    double dlo = fabs(x - vlo);
    double dhi = fabs(vhi - x);
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

/* Element-wise form of the rounding above, for arrays. */
void ck_oracle_f32_to_bf16_array(const float *f, uint16_t *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) out[i] = ck_oracle_f32_to_bf16(f[i]);
}

/* ---- fp16 <-> fp32 ---------------------------------------------------------
 * IEEE binary16: sign, 5 exponent bits (bias 15), 10 fraction bits; exponent
 * field 0 holds zero and the subnormals f * 2^-24; field 31 holds infinity
 * and NaN.  Every binary16 value is exactly a binary32 value. */
float ck_oracle_f16_to_f32(uint16_t h)
{
    const int neg = (h >> 15) & 1;
    const int e = (h >> 10) & 31;
    const int f = h & 1023;
    double v;
    if (e == 31) {
        if (f) return NAN;
        v = INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, -24);
    } else {
        v = ldexp((double)(f + 1024), e - 25);      /* (1 + f/1024) * 2^(e-15) */
    }
    return (float)(neg ? -v : v);
}

/* fp32 -> fp16, round to nearest, ties to even, written as the definition:
 * within the binade of |x| (the subnormals share the spacing 2^-24 of the
 * smallest one) the candidates are the multiples of the spacing; take the
 * nearest, and on a tie the even multiple.  A result of 2^16 or more (that
 * is, |x| >= 65520) is infinity.  All arithmetic below is exact in double:
 * |x| has 24 significant bits and the spacing is a power of two. */
uint16_t ck_oracle_f32_to_f16(float x)
{
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
    if (isinf(x)) return (uint16_t)(sign | 0x7c00u);
    const double a = fabs((double)x);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                                  /* 2^(e-1) <= a < 2^e */
    int be = e - 1;
    if (be < -14) be = -14;
    const double spacing = ldexp(1.0, be - 10);
    const double n = a / spacing;
    double r = floor(n);
    const double rem = n - r;
    if (rem > 0.5 || (rem == 0.5 && fmod(r, 2.0) == 1.0)) r += 1.0;
    const double v = r * spacing;
    if (v >= 65536.0) return (uint16_t)(sign | 0x7c00u);
    if (v < ldexp(1.0, -14))                       /* subnormal */
        return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -24)));
    frexp(v, &e);
    const int ve = e - 1;                          /* 2^ve <= v < 2^(ve+1) */
    const uint16_t frac = (uint16_t)(v / ldexp(1.0, ve - 10) - 1024.0);
    return (uint16_t)(sign | (uint16_t)((ve + 15) << 10) | frac);
}

void ck_oracle_f32_to_f16_array(const float *f, uint16_t *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) out[i] = ck_oracle_f32_to_f16(f[i]);
}

void ck_oracle_f16_to_f32_array(const uint16_t *h, float *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) out[i] = ck_oracle_f16_to_f32(h[i]);
}

/* ---- step 1: quantisation --------------------------------------------- */

/* One code: q = clamp(rint(x / s), -127, 127); s == 0 only for an all-zero
 * row or tensor, whose codes are all 0. */
static int8_t quant_code(float xv, float s)
{
    if (s == 0.0f) return 0;
    float t = xv / s;          /* correctly rounded fp32 division */
    t = rintf(t);              /* default mode: round half to even */
    if (t > 127.0f) t = 127.0f;
    if (t < -127.0f) t = -127.0f;
    return (int8_t)t;
}

/* Per-row quantisation of x[m, k] (bf16 bits, row stride ldx elements):
 * scale[r] = amax_r / 127, q[r, j] = code(x[r, j], scale[r]). */
void ck_oracle_quantize_rowwise(const uint16_t *x, int64_t m, int64_t k,
                                int64_t ldx, int8_t *q, int64_t ldq,
                                float *scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r) {
        float amax = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            float a = fabsf(ck_oracle_bf16_to_f32(x[r * ldx + j]));
            if (a > amax) amax = a;
        }
        float s = amax / 127.0f;
        scale[r] = s;
        for (int64_t j = 0; j < k; ++j)
            q[r * ldq + j] = quant_code(ck_oracle_bf16_to_f32(x[r * ldx + j]), s);
    }
}

/* Per-row quantisation of fp32 rows (the rotated activations): the same
 * formula, amax and codes taken on the fp32 values. */
void ck_oracle_quantize_rowwise_f32(const float *x, int64_t m, int64_t k,
                                    int64_t ldx, int8_t *q, int64_t ldq,
                                    float *scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r) {
        float amax = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            float a = fabsf(x[r * ldx + j]);
            if (a > amax) amax = a;
        }
        float s = amax / 127.0f;
        scale[r] = s;
        for (int64_t j = 0; j < k; ++j)
            q[r * ldq + j] = quant_code(x[r * ldx + j], s);
    }
}

/* Tensor-wide quantisation of fp32 rows: one amax, one scale. */
void ck_oracle_quantize_tensorwise_f32(const float *x, int64_t m, int64_t k,
                                       int64_t ldx, int8_t *q, int64_t ldq,
                                       float *scale)
{
    float amax = 0.0f;
    for (int64_t r = 0; r < m; ++r)
        for (int64_t j = 0; j < k; ++j) {
            float a = fabsf(x[r * ldx + j]);
            if (a > amax) amax = a;
        }
    float s = amax / 127.0f;
    scale[0] = s;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r)
        for (int64_t j = 0; j < k; ++j)
            q[r * ldq + j] = quant_code(x[r * ldx + j], s);
}

/* Tensor-wide quantisation: one amax over all m*k elements, one scale. */
void ck_oracle_quantize_tensorwise(const uint16_t *x, int64_t m, int64_t k,
                                   int64_t ldx, int8_t *q, int64_t ldq,
                                   float *scale)
{
    float amax = 0.0f;
    for (int64_t r = 0; r < m; ++r)
        for (int64_t j = 0; j < k; ++j) {
            float a = fabsf(ck_oracle_bf16_to_f32(x[r * ldx + j]));
            if (a > amax) amax = a;
        }
    float s = amax / 127.0f;
    scale[0] = s;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r)
        for (int64_t j = 0; j < k; ++j)
            q[r * ldq + j] = quant_code(ck_oracle_bf16_to_f32(x[r * ldx + j]), s);
}

/* ---- step 0 (ConvRot checkpoints): the online rotation -------------------
 * #278 "int8_linear silently falls back ...", section "Suggested fix": a
 * ConvRot weight is stored rotated, W_rot = W H^T, and the activation is
 * rotated online, x_rot = x H, so the product runs in the rotated basis.
 * The page does not give H.  Reading taken: H is block diagonal, K/b copies
 * of the Sylvester-Hadamard matrix of order b (a power of two dividing K)
 * scaled by 1/sqrt(b), which makes H symmetric and orthogonal.
 *
 * x_rot is computed in fp32 from the exact fp32 value of each bf16 x: per
 * block, the fast Walsh-Hadamard butterflies in stages h = 1, 2, 4, ...,
 * b/2, where elements i and i+h (bit h of i clear) become (u + v, u - v);
 * then every value is multiplied by r = fl(1/sqrt(b)).  Each operation is
 * one fp32 rounding; the stage order fixes which additions round. */
float ck_oracle_rot_scale(int64_t b)
{
    return (float)(1.0 / sqrt((double)b));
}

/* x_rot of one row of k bf16 values (k a multiple of b) into out[k]. */
static void rotate_row(const uint16_t *x, int64_t k, int64_t b, float *out)
{
    const float r = ck_oracle_rot_scale(b);
    for (int64_t j = 0; j < k; ++j) out[j] = ck_oracle_bf16_to_f32(x[j]);
    for (int64_t base = 0; base < k; base += b)
        for (int64_t h = 1; h < b; h *= 2)
            for (int64_t i = 0; i < b; ++i)
                if ((i & h) == 0) {
                    const float u = out[base + i], v = out[base + i + h];
                    out[base + i] = u + v;
                    out[base + i + h] = u - v;
                }
    for (int64_t j = 0; j < k; ++j) out[j] = out[j] * r;
}

/* x_rot[m, k] (fp32, row stride k) of x[m, k] (bf16 bits, row stride ldx). */
void ck_oracle_rotate(const uint16_t *x, int64_t m, int64_t k, int64_t ldx,
                      int64_t b, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) rotate_row(x + i * ldx, k, b, out + i * k);
}

/* ---- step 2: the integer product --------------------------------------- */

/* acc[i, j] = sum_t q[i, t] * w[j, t]; q is [m, k] and w is [n, k], both
 * K-contiguous.  The sum is exact in int64; returns -1 if any result does
 * not fit in int32 (acc then holds the value truncated to 32 bits). */
int ck_oracle_gemm_i32(const int8_t *q, int64_t ldq, const int8_t *w,
                       int64_t ldw, int32_t *acc, int64_t ldacc, int64_t m,
                       int64_t n, int64_t k)
{
    int overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : overflow)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            int64_t sum = 0;
            for (int64_t t = 0; t < k; ++t)
                sum += (int64_t)q[i * ldq + t] * (int64_t)w[j * ldw + t];
            if (sum > INT32_MAX || sum < INT32_MIN) overflow = 1;
            acc[i * ldacc + j] = (int32_t)sum;
        }
    return overflow ? -1 : 0;
}

/* ---- step 3: the fp32 epilogue ----------------------------------------- */

/* Output (and bias) element types of the epilogue. */
enum { OUT_BF16 = 0, OUT_FP16 = 1, OUT_FP32 = 2 };

/* bias[j] widened to fp32 (exact for all three types). */
static float bias_value(const void *bias, int64_t j, int dtype)
{
    if (dtype == OUT_FP32) return ((const float *)bias)[j];
    const uint16_t b = ((const uint16_t *)bias)[j];
    return dtype == OUT_FP16 ? ck_oracle_f16_to_f32(b) : ck_oracle_bf16_to_f32(b);
}

/* One output: t = fp32(acc); t = t * xs; t = t * ws; t = t + fp32(bias);
 * then t rounded to the output type.  Each line is one fp32 rounding. */
static void epilogue_one(int32_t a, float xs, float ws, const void *bias,
                         int64_t j, void *out, int64_t idx, int dtype)
{
    float t = (float)a;
    t = t * xs;
    t = t * ws;
    if (bias) t = t + bias_value(bias, j, dtype);
    if (dtype == OUT_FP32) ((float *)out)[idx] = t;
    else if (dtype == OUT_FP16) ((uint16_t *)out)[idx] = ck_oracle_f32_to_f16(t);
    else ((uint16_t *)out)[idx] = ck_oracle_f32_to_bf16(t);
}

/* Epilogue over an int32 matrix.  xs has m entries when xs_per_row, else
 * one; ws has n entries when ws_per_col, else one; bias is [n] (of the
 * output type) or NULL; out is [m, ldo] of type dtype. */
void ck_oracle_epilogue_ex(const int32_t *acc, int64_t ldacc, const float *xs,
                           int xs_per_row, const float *ws, int ws_per_col,
                           const void *bias, void *out, int64_t ldo,
                           int64_t m, int64_t n, int dtype)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            epilogue_one(acc[i * ldacc + j], xs[xs_per_row ? i : 0],
                         ws[ws_per_col ? j : 0], bias, j, out, i * ldo + j, dtype);
}

void ck_oracle_epilogue(const int32_t *acc, int64_t ldacc, const float *xs,
                        int xs_per_row, const float *ws, int ws_per_col,
                        const uint16_t *bias, uint16_t *out, int64_t ldo,
                        int64_t m, int64_t n)
{
    ck_oracle_epilogue_ex(acc, ldacc, xs, xs_per_row, ws, ws_per_col, bias, out,
                          ldo, m, n, OUT_BF16);
}

/* Steps 2 and 3 together, element by element, without storing the int32
 * matrix: the form used to check sampled rows of very large outputs.
 * Returns -1 if any accumulator overflows int32 (that output is then
 * computed from the truncated value). */
int ck_oracle_linear_ex(const int8_t *q, int64_t ldq, const float *xs,
                        int xs_per_row, const int8_t *w, int64_t ldw,
                        const float *ws, int ws_per_col, const void *bias,
                        void *out, int64_t ldo, int64_t m, int64_t n,
                        int64_t k, int dtype)
{
    int overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : overflow)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            int64_t sum = 0;
            for (int64_t t = 0; t < k; ++t)
                sum += (int64_t)q[i * ldq + t] * (int64_t)w[j * ldw + t];
            if (sum > INT32_MAX || sum < INT32_MIN) overflow = 1;
            epilogue_one((int32_t)sum, xs[xs_per_row ? i : 0], ws[ws_per_col ? j : 0],
                         bias, j, out, i * ldo + j, dtype);
        }
    return overflow ? -1 : 0;
}

int ck_oracle_linear(const int8_t *q, int64_t ldq, const float *xs,
                     int xs_per_row, const int8_t *w, int64_t ldw,
                     const float *ws, int ws_per_col, const uint16_t *bias,
                     uint16_t *out, int64_t ldo, int64_t m, int64_t n,
                     int64_t k)
{
    return ck_oracle_linear_ex(q, ldq, xs, xs_per_row, w, ldw, ws, ws_per_col,
                               bias, out, ldo, m, n, k, OUT_BF16);
}

/* ---- the dequant-on-the-fly path (W8A16) ----------------------------------
 * #278 "int8_linear silently falls back ...", section "Suggested fix": the
 * int8 weight is dequantised to the 16-bit compute type on the fly and the
 * product runs on 16-bit matrix cores, without quantising x; the weight
 * stays int8 in memory.  Reading taken: the compute type is bf16 (the
 * activations' type here), the dequantised weight is
 *   wdq[j, t] = bf16(fp32(w[j, t]) * w_scale[j])     (fp32 multiply, then RNE)
 * and the output is round_out(S + bias[j]) with S = sum_t x[i, t] * wdq[j, t].
 *
 * Products of two bf16 values are exact in fp32; the hardware sums them in
 * fp32 in an order of its own, so the path is not bit-reproducible.  The
 * oracle returns S exactly rounded to fp32 (the double sum of exact products
 * is exact to far below an fp32 ulp for these sizes) and, per output, the
 * magnitude sum A = sum_t |x[i, t] * wdq[j, t]| from which the test derives
 * the fp32 accumulation bound. */
uint16_t ck_oracle_dequant_weight_one(int8_t w, float ws)
{
    float t = (float)w * ws;
    return ck_oracle_f32_to_bf16(t);
}

void ck_oracle_dequant_weight(const int8_t *w, int64_t n, int64_t k, int64_t ldw,
                              const float *ws, int ws_per_col, uint16_t *wdq)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        for (int64_t t = 0; t < k; ++t)
            wdq[j * k + t] = ck_oracle_dequant_weight_one(w[j * ldw + t], ws[ws_per_col ? j : 0]);
}

/* out[i, j] = round_out(fl32(S) + bias[j]); sum_out[i, j] = fl32(S) and
 * mag_out[i, j] = A (both fp64).  wdq is the dequantised weight [n, k]
 * (bf16 bits, row stride k).  x is [m, ldx] bf16 bits. */
void ck_oracle_linear_dequant(const uint16_t *x, int64_t ldx, const uint16_t *wdq,
                              const void *bias, void *out, int64_t ldo, int64_t m,
                              int64_t n, int64_t k, int dtype, double *sum_out,
                              double *mag_out)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double sum = 0.0, mag = 0.0;
            for (int64_t t = 0; t < k; ++t) {
                const double p = (double)ck_oracle_bf16_to_f32(x[i * ldx + t]) *
                                 (double)ck_oracle_bf16_to_f32(wdq[j * k + t]);
                sum += p;
                mag += fabs(p);
            }
            float s = (float)sum;
            if (sum_out) sum_out[i * n + j] = (double)s;
            if (mag_out) mag_out[i * n + j] = mag;
            if (bias) s = s + bias_value(bias, j, dtype);
            if (dtype == OUT_FP32) ((float *)out)[i * ldo + j] = s;
            else if (dtype == OUT_FP16) ((uint16_t *)out)[i * ldo + j] = ck_oracle_f32_to_f16(s);
            else ((uint16_t *)out)[i * ldo + j] = ck_oracle_f32_to_bf16(s);
        }
}

/* Number of threads an OpenMP region here will use. */
int ck_oracle_num_threads(void)
{
    return omp_get_max_threads();
}
