/*
 * qk_oracle.cpp - plain, slow CPU oracle for ggml block-quantized
 * dequantize, GEMV and GEMM (formats Q4_0, Q4_1, Q8_0, Q5_0, Q5_1), in plain
 * C++ (loops over arrays, no templates or containers) with a C interface.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference the GPU
 * library is checked against.  Only the test suite, the package smoke check
 * and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * Build: g++ -std=c++17 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (contraction off: every fp32 multiply and add below is rounded on its own,
 * in the order written).
 *
 * Sources (the pages this follows):
 *  - "llama_cpp 0.12.1 -> 0.12.2" diff of vendored ggml-cuda.cu (diffend page 4):
 *      hunk adding dequantize_block_q4_0 / dequantize_block_q4_1: block
 *      fields d (fp16 scale), dm (fp16 pair d, m), qs (16 nibble bytes);
 *      byte j holds element j in its low nibble and element j+16 in its high
 *      nibble; value computed in fp32 as d*q + (-8*d) (Q4_0) and
 *      d.x*q + d.y (Q4_1), then stored to the fp32 or fp16 destination.
 *    - hunk adding dequantize_block_q8_0_f16: a Q8_0 block is an fp16 d
 *      followed by 32 signed bytes (64 blocks fill 2176 bytes, so 34 bytes a
 *      block); value q*d.
 *    - the dequantize_row_*_cuda launchers: 32 weights per block (nb32 = k/32).
 *  - Q5_0 and Q5_1 are named only by the to_fp16 / to_fp32 dispatch of the
 *    same diff (dequantize_block_cuda with dequantize_q5_0 / dequantize_q5_1,
 *    blocks of QK5_0 / QK5_1 weights); their byte layout and arithmetic are
 *    not printed on the pages.  Reading taken (ggml's published block
 *    format): Q5_0 = d (fp16), qh (4 bytes, little-endian: bit t is bit 4 of
 *    code t), qs (16 bytes, low four bits as Q4_0); value (q - 16) * d.
 *    Q5_1 = d, m (fp16), qh, qs; value d*q + m.
 *  - The dot-product definition y[i,j] = sum_c W[i,c] * X[c,j] is the plain
 *    matrix-vector / matrix-matrix product that dequantize_mul_mat_vec and the
 *    mul_mat path compute (same diff page, ggml_cuda_op_mul_mat and the
 *    dmmv tuning block); the oracle evaluates it in fp64.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

/* Format ids used by this oracle's entry points (its own numbering). */
#define ORC_Q4_0 0
#define ORC_Q4_1 1
#define ORC_Q8_0 2
#define ORC_Q5_0 3
#define ORC_Q5_1 4

/* Entry points with C linkage, so that they load by name through ctypes. */
extern "C" {

/* ---------------------------------------------------------------------
 * IEEE-754 binary16 codec, written from the format definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * ------------------------------------------------------------------- */

/* Exact decode of binary16 bits to fp32 (every binary16 value is an fp32). */
float orc_half_to_float(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 31;
    const int f = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);              /* zero or subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;          /* infinity or NaN */
    } else {
        v = ldexp((double)(1024 + f), e - 25);  /* normal: (1 + f/1024) * 2^(e-15) */
    }
    if (isnan(v)) {
        return sign ? -NAN : NAN;
    }
    return (float)(sign ? -v : v);
}

/* Round a non-negative double holding an exact multiple of 2^-k (k small)
 * to the nearest integer, ties to even.  All steps are exact in double. */
static double orc_round_half_even(double q)
{
    const double fl = floor(q);
    const double frac = q - fl;
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* fp32 -> binary16, round to nearest even, overflow to infinity, subnormals
 * kept.  NaN maps to a quiet NaN of the same sign. */
uint16_t orc_float_to_half(float v)
{
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    const double a = fabs((double)v);
    if (a == 0.0) return sign;
    if (isinf(v)) return (uint16_t)(sign | 0x7C00u);
    int ex;
    frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;                /* a in [2^e, 2^(e+1)) */
    if (e < -14) {
        /* subnormal range: quantum 2^-24 */
        const double r = orc_round_half_even(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)r);   /* r == 1024 is the smallest normal */
    }
    double r = orc_round_half_even(ldexp(a, 10 - e));  /* in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        e += 1;
    }
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r - 1024.0));
}

/* ---------------------------------------------------------------------
 * Block layout
 * ------------------------------------------------------------------- */

int orc_block_bytes(int fmt)
{
    switch (fmt) {
    case ORC_Q4_0: return 2 + 16;        /* d, qs[16] */
    case ORC_Q4_1: return 2 + 2 + 16;    /* d, m, qs[16] */
    case ORC_Q8_0: return 2 + 32;        /* d, qs[32] (int8) */
    case ORC_Q5_0: return 2 + 4 + 16;    /* d, qh, qs[16] */
    case ORC_Q5_1: return 2 + 2 + 4 + 16; /* d, m, qh, qs[16] */
    default: return 0;
    }
}

static uint16_t orc_le16(const uint8_t *p)
{
    return (uint16_t)(p[0] | (p[1] << 8));
}

/* Integer code of element t (0..31) of one block. */
int orc_code(int fmt, const uint8_t *blk, int t)
{
    switch (fmt) {
    case ORC_Q4_0:
    case ORC_Q4_1: {
        const uint8_t *qs = blk + (fmt == ORC_Q4_0 ? 2 : 4);
        return (t < 16) ? (qs[t] & 0x0F) : (qs[t - 16] >> 4);
    }
    case ORC_Q8_0:
        return (int)(int8_t)blk[2 + t];
    case ORC_Q5_0:
    case ORC_Q5_1: {
        const uint8_t *qhp = blk + (fmt == ORC_Q5_0 ? 2 : 4);
        const uint8_t *qs = qhp + 4;
        const uint32_t qh = (uint32_t)qhp[0] | ((uint32_t)qhp[1] << 8) |
                            ((uint32_t)qhp[2] << 16) | ((uint32_t)qhp[3] << 24);
        const int low = (t < 16) ? (qs[t] & 0x0F) : (qs[t - 16] >> 4);
        return low | (int)(((qh >> t) & 1u) << 4);
    }
    default:
        return 0;
    }
}

/* fp32 value of element t of one block, in the pages' operation order,
 * each operation rounded separately (no contraction). */
float orc_value(int fmt, const uint8_t *blk, int t)
{
    const float d = orc_half_to_float(orc_le16(blk));
    const float c = (float)orc_code(fmt, blk, t);
    switch (fmt) {
    case ORC_Q4_0: {
        const float dm = -8.0f * d;
        const float p = d * c;
        return p + dm;
    }
    case ORC_Q4_1: {
        const float m = orc_half_to_float(orc_le16(blk + 2));
        const float p = d * c;
        return p + m;
    }
    case ORC_Q8_0:
        return d * c;
    case ORC_Q5_0: {
        const float cc = c - 16.0f;   /* exact: a small integer */
        return cc * d;
    }
    case ORC_Q5_1: {
        const float m = orc_half_to_float(orc_le16(blk + 2));
        const float p = d * c;
        return p + m;
    }
    default:
        return NAN;
    }
}

/* Element (i, c) of a rows x k matrix stored row after row, each row k/32
 * blocks back to back, no padding. */
static float orc_weight(int fmt, const uint8_t *w, int64_t k, int64_t i, int64_t c)
{
    const int64_t bs = orc_block_bytes(fmt);
    const uint8_t *blk = w + (i * (k / 32) + c / 32) * bs;
    return orc_value(fmt, blk, (int)(c % 32));
}

/* ---------------------------------------------------------------------
 * Dequantize: out[i*k + c] = W[i, c]
 * ------------------------------------------------------------------- */

void orc_dequantize_f32(int fmt, const uint8_t *w, int64_t rows, int64_t k, float *out)
{
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t c = 0; c < k; ++c)
            out[i * k + c] = orc_weight(fmt, w, k, i, c);
}

/* fp16 output: one round-to-nearest-even of the fp32 value. */
void orc_dequantize_f16(int fmt, const uint8_t *w, int64_t rows, int64_t k, uint16_t *out)
{
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t c = 0; c < k; ++c)
            out[i * k + c] = orc_float_to_half(orc_weight(fmt, w, k, i, c));
}

/* ---------------------------------------------------------------------
 * Products.  Activations X are n columns of length k, column j starting at
 * element j*ldx; either fp32 (x_is_f16 == 0) or binary16 bits (x_is_f16 == 1).
 * Result y[j*m + i] = sum_c W[i,c] * X[c,j] accumulated in fp64 from the
 * fp32 weight values, and s[j*m + i] = sum_c |W[i,c] * X[c,j]| (the
 * tolerance scale).
 * ------------------------------------------------------------------- */

static double orc_x(const void *x, int x_is_f16, int64_t idx)
{
    if (x_is_f16) return (double)orc_half_to_float(((const uint16_t *)x)[idx]);
    return (double)((const float *)x)[idx];
}

static void orc_dot_one(int fmt, const uint8_t *w, int64_t k, const void *x, int x_is_f16,
                        int64_t ldx, int64_t i, int64_t j, double *y, double *s)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t c = 0; c < k; ++c) {
        const double p = (double)orc_weight(fmt, w, k, i, c) * orc_x(x, x_is_f16, j * ldx + c);
        acc += p;
        mag += fabs(p);
    }
    *y = acc;
    *s = mag;
}

void orc_dot(int fmt, const uint8_t *w, int64_t m, int64_t k, const void *x, int x_is_f16,
             int64_t ldx, int64_t n, double *y, double *s)
{
    for (int64_t j = 0; j < n; ++j)
        for (int64_t i = 0; i < m; ++i)
            orc_dot_one(fmt, w, k, x, x_is_f16, ldx, i, j, &y[j * m + i], &s[j * m + i]);
}

/* Selected entries only: (ii[e], jj[e]) for e < count. */
void orc_dot_entries(int fmt, const uint8_t *w, int64_t k, const void *x, int x_is_f16,
                     int64_t ldx, const int64_t *ii, const int64_t *jj, int64_t count,
                     double *y, double *s)
{
    for (int64_t e = 0; e < count; ++e)
        orc_dot_one(fmt, w, k, x, x_is_f16, ldx, ii[e], jj[e], &y[e], &s[e]);
}

/* ---------------------------------------------------------------------
 * Expert-indexed products (mixture-of-experts decode).
 *
 * The tensor-parallel compare names ggml_cuda_mul_mat_id (a hunk of
 * ggml-cuda.cu) and the PR's commit list a Q4_0 expert model with an
 * intermediate dimension of 768; what the op computes is not printed on the
 * pages.  Reading taken (ggml's mul_mat_id): a stack of n_experts matrices of
 * the same shape, expert e at byte offset e*expert_stride; for token t and
 * slot s the selected expert is e = ids[t*ld_ids + s] and the output is the
 * plain product of that expert's matrix with that slot's activation vector,
 * x + t*x_tok + s*x_slot (x_slot = 0: every slot of a token reads the same
 * vector).
 *
 * Results go to y[(t*n_used + s)*m + i] and the tolerance scale to
 * s[(t*n_used + s)*m + i].  An id outside [0, n_experts) selects nothing:
 * its m outputs and scales are NaN.
 * ------------------------------------------------------------------- */
void orc_dot_id(int fmt, const uint8_t *w, int64_t n_experts, int64_t expert_stride,
                int64_t m, int64_t k, const int32_t *ids, int64_t ld_ids, int64_t n_used,
                int64_t n_tokens, const float *x, int64_t x_slot, int64_t x_tok,
                double *y, double *s)
{
    for (int64_t t = 0; t < n_tokens; ++t) {
        for (int64_t u = 0; u < n_used; ++u) {
            const int64_t e = ids[t * ld_ids + u];
            double *yo = y + (t * n_used + u) * m;
            double *so = s + (t * n_used + u) * m;
            if (e < 0 || e >= n_experts) {
                for (int64_t i = 0; i < m; ++i) {
                    yo[i] = NAN;
                    so[i] = NAN;
                }
                continue;
            }
            const uint8_t *we = w + e * expert_stride;
            const float *xv = x + t * x_tok + u * x_slot;
            for (int64_t i = 0; i < m; ++i)
                orc_dot_one(fmt, we, k, xv, 0, k, i, 0, &yo[i], &so[i]);
        }
    }
}

/* ---------------------------------------------------------------------
 * Products with 8-bit activations (integer dot products).
 *
 * The "llama_cpp 0.12.1 -> 0.12.2" diff names the integer-dot kernels
 * (mul_mat_vec_q / MMQ, fed by a quantize_q8_1 step) but prints neither their
 * activation layout nor their rounding.  Reading taken here (a design choice
 * of this library, stated as such):
 * each 32-element block of an activation column is quantized with a
 * power-of-two scale d = 2^e, e the smallest integer with 127 * 2^e >= amax
 * (amax = max |x| over the block), but at least -126; the codes are
 * q = round-half-even(x / d), so |q| <= 127 and every decision is exact (a
 * division by a power of two rounds nothing).  An all-zero block has d = 0
 * and q = 0.  The product then uses the dequantized activation x^ = d * q.
 * ------------------------------------------------------------------- */

/* Quantize one block of 32 fp32 values: codes q[32], returns d.  A block
 * holding an infinite or NaN value has no finite scale: its scale is NaN and
 * its codes 0, so every product that uses the block is NaN (as the plain
 * product with such an activation is infinite or NaN). */
float orc_quantize_x8_block(const float *x, int8_t *q)
{
    double amax = 0.0;
    for (int t = 0; t < 32; ++t) {
        if (!isfinite(x[t])) {
            for (int u = 0; u < 32; ++u) q[u] = 0;
            return NAN;
        }
    }
    for (int t = 0; t < 32; ++t) {
        const double a = fabs((double)x[t]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0) {
        for (int t = 0; t < 32; ++t) q[t] = 0;
        return 0.0f;
    }
    int e = -126;
    while (127.0 * ldexp(1.0, e) < amax) ++e;   /* smallest e >= -126 */
    const double d = ldexp(1.0, e);
    for (int t = 0; t < 32; ++t) {
        const double v = (double)x[t] / d;       /* exact: d is a power of two */
        double r = floor(v);
        const double frac = v - r;
        if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
        q[t] = (int8_t)r;
    }
    return (float)d;
}

/* Quantize n columns of length k (stride ldx): codes qx[j*k + c] and scales
 * dx[j*(k/32) + b]. */
void orc_quantize_x8(const float *x, int64_t k, int64_t n, int64_t ldx, int8_t *qx, float *dx)
{
    for (int64_t j = 0; j < n; ++j)
        for (int64_t b = 0; b < k / 32; ++b)
            dx[j * (k / 32) + b] = orc_quantize_x8_block(x + j * ldx + 32 * b, qx + j * k + 32 * b);
}

/* y[j*m + i] = sum_c W[i,c] * x^[j][c] in fp64 (x^ = d * q as above), and
 * the tolerance scale s[j*m + i]: the sum over blocks of |d_x * d * I| for
 * Q4_0 / Q8_0 / Q5_0 and |d_x * d * I| + |d_x * m * Q| for Q4_1 / Q5_1, where
 * I is the block's integer dot product of codes (Q4_0 codes taken as q - 8,
 * Q5_0 codes as q - 16) and Q the sum of the activation codes: the
 * magnitudes of the terms a kernel rounds. */
void orc_dot_x8(int fmt, const uint8_t *w, int64_t m, int64_t k, const float *x, int64_t n,
                int64_t ldx, double *y, double *s)
{
    const int64_t nb = k / 32;
    const int64_t bs = orc_block_bytes(fmt);
    int8_t q[32];
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t i = 0; i < m; ++i) {
            double acc = 0.0, mag = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const float dx = orc_quantize_x8_block(x + j * ldx + 32 * b, q);
                const uint8_t *blk = w + (i * nb + b) * bs;
                const double dw = (double)orc_half_to_float(orc_le16(blk));
                double isum = 0.0, qsum = 0.0;
                for (int t = 0; t < 32; ++t) {
                    int c = orc_code(fmt, blk, t);
                    if (fmt == ORC_Q4_0) c -= 8;
                    if (fmt == ORC_Q5_0) c -= 16;
                    isum += (double)c * (double)q[t];
                    qsum += (double)q[t];
                    /* the plain product with the dequantized activation */
                    acc += (double)orc_value(fmt, blk, t) * ((double)dx * (double)q[t]);
                }
                mag += fabs((double)dx * dw * isum);
                if (fmt == ORC_Q4_1 || fmt == ORC_Q5_1)
                    mag += fabs((double)dx * (double)orc_half_to_float(orc_le16(blk + 2)) * qsum);
            }
            y[j * m + i] = acc;
            s[j * m + i] = mag;
        }
    }
}

}  /* extern "C" */
