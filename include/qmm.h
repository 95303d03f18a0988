/*
 * qmm.h -- block-quantized weight matmul on AMD Instinct MI355X (gfx950).
 *
 * y[m][n] = sum_k x[m][k] * w[n][k]   (y = x * W^T), with W stored as GGUF
 * weight blocks of 32 consecutive k:
 *   Q4_0 block, 18 bytes: fp16 scale d (little-endian), then 16 bytes qs;
 *        element j < 16 is the low nibble of qs[j], element j + 16 its high
 *        nibble; w = d * (q - 8).
 *   Q8_0 block, 34 bytes: fp16 scale d, then 32 int8 q; w = d * q.
 * The pages "Add generated quant-kernel JIT and accelerate Gemma4, BGE-M3,
 * and GLiNER2" (section Validation) count these two formats among the
 * generated quant dispatches of one Gemma4 decode (Q4_0 for all but one
 * projection, Q8_0 for the remaining one); the same pages' Benchmarks
 * section measures decode and prefill (TTFT) of those models, the two
 * regimes the entry points below serve.
 *
 * Layouts (all row-major, contiguous, no padding):
 *   x : float32 [M][K]
 *   w : N rows of K/32 blocks; row n starts at byte n * (K/32) * block_bytes
 *   y : float32 [M][N], overwritten (no accumulation into y, no bias)
 *
 * Ownership and execution: every pointer is a DEVICE pointer owned by the
 * caller. The library allocates no memory, keeps no pointer after a call
 * returns, and enqueues its work asynchronously on `stream` (NULL = the
 * null stream); it never synchronizes. Calls are thread-safe.
 *
 * Errors: arguments are validated on the host before any HIP call, so a
 * rejected call has no effect on the device. Every entry point returns a
 * qmm_status; qmm_last_error() gives a thread-local description of the last
 * non-OK status returned on the calling thread.
 *   QMM_EINVAL       null pointer; M, N or K < 1; K not a multiple of 32;
 *                    M > 16 for a GEMV entry point; y overlapping x or w;
 *                    a byte size that overflows int64.
 *   QMM_EALIGN       x or w not 16-byte aligned, y not 4-byte aligned.
 *   QMM_EUNSUPPORTED K not a multiple of 64 (every weight row then holds
 *                    whole, dword-aligned pairs of blocks), or K > QMM_MAX_K;
 *                    for the GEMM entry
 *                    points also N > QMM_GEMM_MAX_N or more than
 *                    INT32_MAX - 8 output tiles of 256 x 256.
 *   QMM_EHIP         the HIP runtime reported an error at launch.
 *
 * Accuracy contract, with s[m][n] = sum_k |x[m][k] * w[n][k]|:
 *   GEMV entry points (f32 arithmetic):  |y - y_exact| <= 1e-4 * s
 *   qmm_gemm_q4_0, qmm_gemm_q8_0 (bf16 MFMA, f32 acc): |y - y_exact| <= 8e-3 * s
 * for finite inputs whose f32 products do not underflow. Results are
 * bitwise reproducible from call to call (no atomics, fixed reduction order).
 *
 * Non-finite scales: with finite x, y[m][n] is non-finite exactly when
 * weight row n holds a block whose fp16 scale (Q4_K: d or dmin) is +Inf,
 * -Inf or NaN; every other output keeps the bound above. Which non-finite
 * value comes out (NaN, +Inf or -Inf) is not specified and may differ from
 * the definition evaluated weight by weight: the GEMV kernels apply d to a
 * block's partial sum, so an infinite scale over a zero code (q = 8) gives
 * +-Inf where d * (q - 8) * x would give NaN. The gated entry point's h[m][n] is
 * non-finite exactly when row n of W_gate or of W_up holds such a scale.
 */
#ifndef QMM_H
#define QMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define QMM_API __attribute__((visibility("default")))
#else
#define QMM_API
#endif

typedef enum qmm_status {
    QMM_OK = 0,
    QMM_EINVAL = 1,
    QMM_EALIGN = 2,
    QMM_EUNSUPPORTED = 3,
    QMM_EHIP = 4
} qmm_status;

/* Largest K accepted by any entry point. */
#define QMM_MAX_K 65536
/* Largest M accepted by the GEMV entry points. */
#define QMM_GEMV_MAX_M 16
/* Largest N accepted by the GEMM entry points (a 256-row band of y stays below 2 GiB). */
#define QMM_GEMM_MAX_N 2097151

/*
 * Decode GEMV over Q4_0 weights, 1 <= M <= 16 activation rows (M = 1 for
 * one decoded token, M = 2..16 for batched or speculative decode, where
 * several tokens share one pass over the weights). f32 accumulation; the
 * weights stream from HBM once per call. Up to 4 rows take f32 FMAs on
 * codes converted exactly to f32, and each row rounds as in a one-row call
 * of the same launch shape; 5 to 16 rows, and 3 or 4 rows where K is a
 * multiple of 256 and either K >= 4096 with N >= 4096, K > 2048 with
 * 2048 < N < 4096, 1024 <= N <= 2048 with 8192 < K <= 11264 (Q4_0) or
 * K <= 9216 (Q8_0), or (Q4_0) N >= 16384 with K >= 1536, take the bf16
 * matrix cores: the
 * codes are exact in bf16 and x is carried as two bf16 terms, hi = bf16(x)
 * and lo = bf16(x - hi), which represent x to within 2^-17 |x| (about 16 of
 * its 24 significand bits); each code-term product is exact, sums are f32
 * and the fp16 scale is applied per block in f32.
 */
QMM_API int qmm_gemv_q4_0(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream);

/*
 * Decode GEMV over Q8_0 weights (the one Q8_0 projection of a decode step,
 * typically the vocabulary head), 1 <= M <= 16. Same contract as
 * qmm_gemv_q4_0.
 */
QMM_API int qmm_gemv_q8_0(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream);

/*
 * Prefill GEMM over Q4_0 weights, any M >= 1 (M = prompt tokens). x is
 * rounded to bf16 (round-to-nearest-even) and each weight d * (q - 8) to
 * bf16 inside the kernel; products accumulate in f32 on the matrix cores.
 * M <= 4, and M <= 16 with N <= 4096, run qmm_gemv_q4_0's kernels instead
 * (the same results, bit for bit), which are faster there and well inside
 * this bound.
 */
QMM_API int qmm_gemm_q4_0(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream);

/*
 * Prefill GEMM over Q8_0 weights (a Q8_0 projection, e.g. the vocabulary
 * head, over many tokens): same contract as qmm_gemm_q4_0, each weight
 * d * q rounded once to bf16 (M <= 4, and M <= 16 with N <= 4096: as
 * qmm_gemv_q8_0).
 */
QMM_API int qmm_gemm_q8_0(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream);

/*
 * Gated FFN front half over Q4_0 weights for 1 <= M <= 16 tokens (M = 1 for
 * one decoded token, 2..16 for batched or speculative decode; the step
 * either side of the path):
 *   h[m][n] = gelu_tanh(g[m][n]) * u[m][n],  g = x * W_gate^T,  u = x * W_up^T,
 *   gelu_tanh(g) = g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3))).
 * The pages ("Add generated quant-kernel JIT and accelerate Gemma4, BGE-M3,
 * and GLiNER2", section Summary) credit fused FFN paths without naming the
 * activation; the tanh form of GELU is the Gemma family's. W_gate and W_up
 * are both N rows of K/32 Q4_0 blocks (same layout as the GEMV's w); both
 * stream in one launch that reads x once. x is f32[M][K], h f32[M][N],
 * overwritten; each weight is decoded once for all rows. Up to 4 rows take
 * f32 FMAs, and a row of h equals the one-row result bit for bit; 5 to 16
 * rows, and 3 or 4 where K % 256 == 0, K >= 1024 and N >= 3072, except
 * K > 1024 with 4096 < N < 8192 and K < 4096 with N > 16384, take the
 * bf16 matrix cores with x as two bf16 terms (as qmm_gemv_q4_0). Errors as above, plus QMM_EINVAL for a null or
 * overlapping w_up and QMM_EALIGN for a w_up not 16-byte aligned.
 * Accuracy: g and u within the GEMV bound (1e-4 of their abs-sums); the
 * activation and product in f32.
 */
QMM_API int qmm_ffn_gate_up_q4_0(const float *x, const void *w_gate, const void *w_up,
                                 float *h, int64_t M, int64_t N, int64_t K,
                                 hipStream_t stream);

/*
 * Decode GEMV over Q4_K super-blocks, 1 <= M <= 16 activation rows. Q4_K is the
 * k-quant 4-bit format the pages ("Add generated quant-kernel JIT and
 * accelerate Gemma4, BGE-M3, and GLiNER2", section Summary) keep for their
 * CLIP/CLAP path; they give no layout, and GGUF's is taken. w is N rows of
 * K/256 super-blocks of 144 bytes each, rows contiguous, no padding:
 *   bytes 0-1 fp16 d, bytes 2-3 fp16 dmin, bytes 4-15 eight 6-bit sub-block
 *   scales sc[j] and minimums mn[j] (j < 4: low 6 bits of byte 4+j and
 *   8+j; j >= 4: low 4 bits from the low / high nibble of byte 8+j, top 2
 *   bits from the top bits of byte j and 4+j), bytes 16-143 nibbles
 *   (weight 64c+i, i < 32, is the low nibble of byte 16+32c+i, weight
 *   64c+32+i its high nibble); weight e is in sub-block e/32 and
 *   w = d * sc * q - dmin * mn.
 * x is f32[M][K], y f32[M][N] (overwritten); the weights stream from HBM
 * once per call. Errors as for qmm_gemv_q4_0, plus QMM_EINVAL for K not a
 * multiple of 256 (qmm_gemm_q4_k takes any M).
 * Accuracy, 1 to 4 rows on the f32 FMA kernels: each weight is formed once
 * in f32 (one rounding) and applied to every activation row in f32; a row
 * of the result does not depend on the other rows;
 * |y - sum_k x w| <= 1e-4 * sum_k |x w|.
 * 5 to 16 rows, and 3 or 4 rows where N > 2048 and K >= 14336, N < 4096
 * with K > 2048, N = 4096 with K >= 8192, or 8192 < N <= 12288 with
 * K >= 4096 (bf16 matrix cores): the nibbles are exact in bf16, x is
 * carried as two bf16 terms (within 2^-17 |x|, as in qmm_gemv_q4_0), and
 * per sub-block the f32 result is d*sc * sum(q x) - dmin*mn * sum(x), the
 * two sums taken from the same bf16 terms; since the two parts are rounded
 * apart, the bound is |y - sum_k x w| <= 1e-4 * sum_k (|d sc q| + |dmin mn|) |x|,
 * which equals the one above where no sub-block has both a scale and a
 * minimum (and exceeds it only where the two parts cancel).
 */
QMM_API int qmm_gemv_q4_k(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream);

/*
 * Prefill GEMM over Q4_K super-blocks (the layout of qmm_gemv_q4_k; the
 * pages' CLIP/CLAP path runs whole sequences through it): the contract of
 * qmm_gemm_q4_0, any M >= 1, with each weight d * sc * q - dmin * mn formed
 * in f32 (rounded once) and rounded to bf16 (nearest even); x rounded to
 * bf16, f32 accumulation. M <= 4, and M <= 16 with N <= 4096, run
 * qmm_gemv_q4_k's kernels instead (the same results, bit for bit). Errors
 * as for qmm_gemm_q4_0, plus QMM_EINVAL for K not a multiple of 256.
 * Accuracy: |y - sum_k x w| <= 8e-3 * sum_k |x w|; where qmm_gemv_q4_k's
 * kernels run, its bound, which for 5 to 16 rows exceeds this one only
 * where the weights' scale and minimum terms cancel:
 * sum_k (|d sc q| + |dmin mn|) |x| > 80 * sum_k |x w|.
 */
QMM_API int qmm_gemm_q4_k(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream);

/* Static English name of a status code ("QMM_OK", ...). */
QMM_API const char *qmm_status_string(int status);

/* Thread-local detail for the last non-OK status on this thread ("" if none). */
QMM_API const char *qmm_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
QMM_API int qmm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
