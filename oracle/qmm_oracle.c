/*
 * qmm_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU reference for the block-quantized
 * weight matmul y = x * W^T over GGUF Q4_0 / Q8_0 weight blocks (and Q4_K
 * super-blocks, further down). Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * this library; the product path never calls it and shares no code with it.
 *
 * What is computed (the plain definition, evaluated in f64):
 *   y[m][n] = sum_k x[m][k] * w[n][k],  w[n][k] = d * (q - 8)   (Q4_0)
 *                                        w[n][k] = d * q         (Q8_0)
 *   s[m][n] = sum_k |x[m][k] * w[n][k]|   (the scale of the error bound)
 * and, for the gated FFN front half over two Q4_0 matrices,
 *   h[m][n] = gelu_tanh(sum_k x w_gate[n][k]) * sum_k x w_up[n][k].
 * The pages ("Add generated quant-kernel JIT and accelerate Gemma4, BGE-M3,
 * and GLiNER2", section Validation) name the two formats by their GGUF
 * names (Q4_0, Q8_0) and count their dispatches; the block layout is GGUF's:
 *   Q4_0 block (18 B): fp16 d, then qs[16]; element j < 16 is the low
 *     nibble of qs[j], element j + 16 the high nibble of qs[j].
 *   Q8_0 block (34 B): fp16 d, then 32 int8 values, element j = qs[j].
 *
 * Exactness: d has at most 11 significant bits, (q - 8) at most 4, a Q8_0
 * value at most 8, and an f32 activation 24, so every product term fits in
 * 43 bits and is exact in f64; the only rounding is the f64 summation,
 * at most (K-1) * 2^-53 * s[m][n].
 *
 * Parallelism: OpenMP over independent (m, n) outputs only; each output is
 * summed serially in k order, so results do not depend on thread count.
 */
#include <math.h>
#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16 -> double, written from the format definition:
 * sign bit 15, exponent bits 14..10 (bias 15), fraction bits 9..0.
 * Exponent 0 is zero/subnormal (f * 2^-24), 31 is Inf/NaN. */
double qmm_oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

static double block_scale(const uint8_t *blk)
{
    return qmm_oracle_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
}

/* Dequantized weight k (0..31) of one Q4_0 block. */
static double q4_0_weight(const uint8_t *blk, double d, int j)
{
    int q = (j < 16) ? (blk[2 + j] & 15) : (blk[2 + j - 16] >> 4);
    return d * (double)(q - 8);
}

/* Dequantized weight k (0..31) of one Q8_0 block. */
static double q8_0_weight(const uint8_t *blk, double d, int j)
{
    return d * (double)(int8_t)blk[2 + j];
}

static void one_output(int fmt, const float *xrow, const uint8_t *wrow,
                       int64_t nblocks, double *y, double *s)
{
    const int64_t bs = fmt == 0 ? 18 : 34;
    double acc = 0.0, abs_acc = 0.0;
    for (int64_t b = 0; b < nblocks; ++b) {
        const uint8_t *blk = wrow + b * bs;
        double d = block_scale(blk);
        for (int j = 0; j < 32; ++j) {
            double w = fmt == 0 ? q4_0_weight(blk, d, j) : q8_0_weight(blk, d, j);
            double t = w * (double)xrow[b * 32 + j];
            acc += t;
            abs_acc += fabs(t);
        }
    }
    *y = acc;
    *s = abs_acc;
}

static void full(int fmt, const float *x, const uint8_t *w, int64_t M,
                 int64_t N, int64_t K, double *y, double *s)
{
    const int64_t nblocks = K / 32;
    const int64_t row_bytes = nblocks * (fmt == 0 ? 18 : 34);
    const int64_t total = M * N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = i / N, n = i % N;
        one_output(fmt, x + m * K, w + n * row_bytes, nblocks, y + i, s + i);
    }
}

static void at(int fmt, const float *x, const uint8_t *w, int64_t K,
               const int64_t *ms, const int64_t *ns, int64_t count, double *y,
               double *s)
{
    const int64_t nblocks = K / 32;
    const int64_t row_bytes = nblocks * (fmt == 0 ? 18 : 34);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        one_output(fmt, x + ms[i] * K, w + ns[i] * row_bytes, nblocks, y + i, s + i);
}

/* Full outputs: x f32[M][K] row-major, w N x (K/32) blocks, y and s
 * f64[M][N] row-major. K must be a multiple of 32 (checked by the caller). */
void qmm_oracle_q4_0(const float *x, const uint8_t *w, int64_t M, int64_t N,
                     int64_t K, double *y, double *s)
{
    full(0, x, w, M, N, K, y, s);
}

void qmm_oracle_q8_0(const float *x, const uint8_t *w, int64_t M, int64_t N,
                     int64_t K, double *y, double *s)
{
    full(1, x, w, M, N, K, y, s);
}

/* Sampled outputs: y[i], s[i] for the pair (ms[i], ns[i]), i < count. */
void qmm_oracle_q4_0_at(const float *x, const uint8_t *w, int64_t K,
                        const int64_t *ms, const int64_t *ns, int64_t count,
                        double *y, double *s)
{
    at(0, x, w, K, ms, ns, count, y, s);
}

void qmm_oracle_q8_0_at(const float *x, const uint8_t *w, int64_t K,
                        const int64_t *ms, const int64_t *ns, int64_t count,
                        double *y, double *s)
{
    at(1, x, w, K, ms, ns, count, y, s);
}

/*
 * Q4_K, the k-quant 4-bit format the pages keep for their CLIP/CLAP path
 * ("Add generated quant-kernel JIT and accelerate Gemma4, BGE-M3, and
 * GLiNER2", section Summary). The pages name it without a layout; GGUF's
 * is taken. A super-block of 256 weights takes 144 bytes:
 *   bytes 0-1   fp16 d      (scale of the sub-block scales)
 *   bytes 2-3   fp16 dmin   (scale of the sub-block minimums)
 *   bytes 4-15  eight 6-bit sub-block scales sc[j] and eight 6-bit
 *               minimums mn[j], j = 0..7 (bit placement below)
 *   bytes 16-143 nibbles: weight 64c + i (c = 0..3, i < 32) is the low
 *               nibble of byte 16 + 32c + i and belongs to sub-block 2c;
 *               weight 64c + 32 + i is the high nibble of the same byte
 *               and belongs to sub-block 2c + 1.
 *   w = d * sc[j] * q - dmin * mn[j] for a weight of sub-block j.
 * The twelve scale bytes b[0..11]: for j < 4, sc[j] is the low 6 bits of
 * b[j] and mn[j] the low 6 bits of b[4 + j]; for j >= 4, the low 4 bits of
 * sc[j] are the low nibble of b[4 + j] and of mn[j] its high nibble, and
 * their top 2 bits are the top 2 bits of b[j - 4] (sc) and b[j] (mn).
 *
 * Exactness: d * sc * q has at most 11 + 6 + 4 bits and dmin * mn 17; their
 * difference is exact in f64 unless d and dmin lie more than 2^32 apart,
 * and so is its product with an f32 activation unless that difference needs
 * more than 29 bits: outside those cases each term is exact, inside them it
 * carries one f64 rounding (2^-53 relative).
 */
static void q4_k_scales(const uint8_t *b, int sc[8], int mn[8])
{
    for (int j = 0; j < 4; ++j) {
        sc[j] = b[j] & 63;
        mn[j] = b[4 + j] & 63;
    }
    for (int j = 4; j < 8; ++j) {
        sc[j] = (b[4 + j] & 15) | ((b[j - 4] >> 6) << 4);
        mn[j] = (b[4 + j] >> 4) | ((b[j] >> 6) << 4);
    }
}

static void one_output_q4_k(const float *xrow, const uint8_t *wrow, int64_t nsuper,
                            double *y, double *s)
{
    double acc = 0.0, abs_acc = 0.0;
    for (int64_t b = 0; b < nsuper; ++b) {
        const uint8_t *blk = wrow + b * 144;
        const double d = qmm_oracle_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
        const double dmin = qmm_oracle_half_to_double((uint16_t)(blk[2] | (blk[3] << 8)));
        int sc[8], mn[8];
        q4_k_scales(blk + 4, sc, mn);
        for (int e = 0; e < 256; ++e) {
            const int c = e / 64, i = e % 64;
            const int j = 2 * c + (i >= 32);
            const uint8_t byte = blk[16 + 32 * c + (i % 32)];
            const int q = i < 32 ? (byte & 15) : (byte >> 4);
            const double w = d * (double)sc[j] * (double)q - dmin * (double)mn[j];
            const double t = w * (double)xrow[b * 256 + e];
            acc += t;
            abs_acc += fabs(t);
        }
    }
    *y = acc;
    *s = abs_acc;
}

/* Full Q4_K outputs: w is N x (K/256) super-blocks; K a multiple of 256. */
void qmm_oracle_q4_k(const float *x, const uint8_t *w, int64_t M, int64_t N,
                     int64_t K, double *y, double *s)
{
    const int64_t nsuper = K / 256, row_bytes = nsuper * 144, total = M * N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = i / N, n = i % N;
        one_output_q4_k(x + m * K, w + n * row_bytes, nsuper, y + i, s + i);
    }
}

void qmm_oracle_q4_k_at(const float *x, const uint8_t *w, int64_t K, const int64_t *ms,
                        const int64_t *ns, int64_t count, double *y, double *s)
{
    const int64_t nsuper = K / 256, row_bytes = nsuper * 144;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        one_output_q4_k(x + ms[i] * K, w + ns[i] * row_bytes, nsuper, y + i, s + i);
}

/*
 * Gated FFN front half (the step either side of the path: gate and up
 * projections of one FFN read the same x, then the activation of the gate
 * multiplies the up projection). The pages credit fused FFN paths ("Add
 * generated quant-kernel JIT and accelerate Gemma4, BGE-M3, and GLiNER2",
 * section Summary) without fixing an activation; the Gemma family's gated
 * FFN uses the tanh form of GELU, taken here:
 *   gelu(g) = g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3)))
 */
double qmm_oracle_gelu_tanh(double g)
{
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * g * (1.0 + tanh(c * (g + 0.044715 * g * g * g)));
}

/* For every (m, n): g = sum_k x[m][k] w_gate[n][k], u = the same over w_up,
 * h = gelu(g) * u, and the two abs-sums s_g, s_u; all f64[M][N]. The sums
 * are the plain matmul above. */
void qmm_oracle_ffn_gate_up_q4_0(const float *x, const uint8_t *w_gate,
                                 const uint8_t *w_up, int64_t M, int64_t N, int64_t K,
                                 double *h, double *g, double *u, double *sg,
                                 double *su)
{
    full(0, x, w_gate, M, N, K, g, sg);
    full(0, x, w_up, M, N, K, u, su);
    for (int64_t i = 0; i < M * N; ++i)
        h[i] = qmm_oracle_gelu_tanh(g[i]) * u[i];
}

/* Threads an OpenMP region of this library uses (1 without OpenMP). */
int qmm_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
