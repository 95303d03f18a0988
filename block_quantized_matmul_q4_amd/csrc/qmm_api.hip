// C-ABI layer of libqmm: argument validation, status codes, the
// thread-local error string, and dispatch to the gfx950 kernels.
// Every check runs on the host before any HIP call, so a rejected call
// leaves the device untouched.
#include <climits>
#include <cstdarg>
#include <cstdio>

#include "../../include/qmm.h"
#include "qmm_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

bool overlaps(uintptr_t a, uint64_t a_len, uintptr_t b, uint64_t b_len)
{
    return a < b + b_len && b < a + a_len;
}

// Shared checks. block_bytes is 18 (Q4_0) or 34 (Q8_0); max_m bounds M.
int validate(const char *fn, const float *x, const void *w, const float *y,
             int64_t M, int64_t N, int64_t K, int block_bytes, int64_t max_m)
{
    if (!x || !w || !y)
        return fail(QMM_EINVAL, "%s: null pointer (x=%p w=%p y=%p)", fn,
                    (const void *)x, w, (const void *)y);
    if (M < 1 || N < 1 || K < 1)
        return fail(QMM_EINVAL, "%s: M, N, K must be >= 1 (M=%lld N=%lld K=%lld)", fn,
                    (long long)M, (long long)N, (long long)K);
    if (M > max_m)
        return fail(QMM_EINVAL, "%s: M=%lld exceeds %lld", fn, (long long)M,
                    (long long)max_m);
    if (K % 32)
        return fail(QMM_EINVAL, "%s: K=%lld is not a multiple of 32 (the block size)", fn,
                    (long long)K);
    if (K % 64 || K > QMM_MAX_K)
        return fail(QMM_EUNSUPPORTED,
                    "%s: K=%lld unsupported (need K %% 64 == 0 and K <= %d)", fn,
                    (long long)K, QMM_MAX_K);
    // Sizes: every index the kernels form fits in int32 element counts for
    // x and y rows, and byte offsets are 64-bit.
    if (N > INT_MAX / 2 || M > INT_MAX / 2 || M > INT64_MAX / K / 4 ||
        M > INT64_MAX / N / 4 || N > INT64_MAX / (K / 32) / block_bytes)
        return fail(QMM_EINVAL, "%s: sizes overflow (M=%lld N=%lld K=%lld)", fn,
                    (long long)M, (long long)N, (long long)K);
    const uintptr_t xa = (uintptr_t)x, wa = (uintptr_t)w, ya = (uintptr_t)y;
    if (xa % 16 || wa % 16 || ya % 4)
        return fail(QMM_EALIGN,
                    "%s: misaligned pointer (x and w need 16-byte, y 4-byte alignment)", fn);
    const uint64_t x_len = (uint64_t)M * (uint64_t)K * 4u;
    const uint64_t w_len = (uint64_t)N * (uint64_t)(K / 32) * (uint64_t)block_bytes;
    const uint64_t y_len = (uint64_t)M * (uint64_t)N * 4u;
    if (overlaps(ya, y_len, xa, x_len) || overlaps(ya, y_len, wa, w_len))
        return fail(QMM_EINVAL, "%s: y overlaps x or w", fn);
    return QMM_OK;
}

int finish(const char *fn, hipError_t err)
{
    if (err != hipSuccess)
        return fail(QMM_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
    return QMM_OK;
}

// The Q4_0 / Q8_0 GEMV for 1 <= M <= 16 (validated). Each route below was
// chosen by timing sweeps on random weights, cold copies:
//  * 1-4 rows: the f32 FMA kernel, which streams the weights once and
//    decodes each weight once for all rows (the FFN shapes: N = 8192,
//    K = 2048 level with the matrix cores at four rows; N = 2048, K = 8192
//    7.8 against 8.5 us);
//  * 3-4 rows take the 16x16 matrix-core kernel where the FMA kernel's four
//    FMAs per weight, or its activation staging, cost more:
//    - K, N >= 4096 (Q4_0, M = 4: N = 13824, K = 5120 30.3 -> 17.9 us;
//      N = 4096, K = 14336 18.9 -> 13.5 us);
//    - 2048 < N < 4096 above K = 2048 (N = 2304, K = 8192 13.2 -> 8.5 us;
//      N = 2560, K = 2560 6.0 -> 4.8 us; Q8_0 N = 3072, K = 8192 15.3 ->
//      10.9 us);
//    - 1024 <= N <= 2048 just past K = 8192, where the FMA kernel stages
//      four rows of x in chunks of 128 pairs and the second, nearly empty
//      chunk costs almost as much as the first (Q4_0, N = 1536, K = 8960:
//      11.3 -> 9.1 us; level from K = 12288, Q8_0 from K = 9728);
//    - Q4_0 from N = 16384 at K >= 1536 (N = 151936, K = 1536: 60.6 -> 44.6
//      us; N = 262144, K = 2048: 104.0 -> 91.3 us; level at N = 65536),
//      while Q8_0's FMA kernel stays faster there (N = 262144: 122 against
//      147 us);
//  * 5-16 rows: the 16x16 matrix-core kernel, and 9-16 rows the 32-row
//    weight-slice kernel above N = 4096 and, from N = 3072, at K <= 2048 (a
//    sweep at M = 16, N = 3072-7168, K = 2048-14336, all three formats:
//    Q4_0, N = 6144, K = 2048 9.6 -> 6.7 us; Q4_K, K = 8192 27.9 -> 21.0 us;
//    Q8_0, N = 5120, K = 4096 16.9 -> 13.6 us; at N <= 4096 from K = 4096
//    the 16x16 kernel stays faster, N = 4096, K = 14336 24.7 against 34.2
//    us), as does any K that is not a multiple of 256 (the 16x16 kernel
//    takes K in slices of 256).
bool rows_on_slices(int64_t M, int64_t N, int64_t K)
{
    return M > 8 && (N > 4096 || (N >= 3072 && K <= 2048));
}

hipError_t gemv_launch(int fmt, const float *x, const uint8_t *w, float *y, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream)
{
    const bool large = (N >= 4096 && K >= 4096) || (N > 2048 && N < 4096 && K > 2048);
    const bool past_chunk = N >= 1024 && N <= 2048 && K > 8192 &&
                            K <= (fmt == qmm::FMT_Q4_0 ? 11264 : 9216);
    const bool wide = fmt == qmm::FMT_Q4_0 && N >= 16384 && K >= 1536;
    const bool matrix_cores = M > 2 && (large || past_chunk || wide) && K % 256 == 0;
    if (M <= qmm::kGemvRowsMax && !matrix_cores)
        return qmm::launch_gemv_m1(fmt, x, w, y, (int)M, (int)N, (int)K, stream);
    if (rows_on_slices(M, N, K) || K % 256)
        return qmm::launch_gemv_slices(fmt, x, w, y, (int)M, (int)N, (int)K, stream);
    return qmm::launch_gemv_small_m(fmt, x, w, y, (int)M, (int)N, (int)K, stream);
}

// The Q4_K GEMV (validated, K % 256 == 0), routed like the Q4_0 one:
//  * 1-4 rows: f32 FMAs on each weight formed once;
//  * 3-4 rows take the 16x16 matrix-core kernel where a sweep (N =
//    2048-28672, K = 2048-14336, four rows, ten FMA launch shapes) found it
//    faster than every FMA shape: 2048 < N < 4096 above K = 2048 (N = 3072,
//    K = 8192 14.4 -> 10.5 us; K = 3072 7.7 -> 5.5 us), N = 4096 from
//    K = 8192 (K = 14336 18.9 -> 15.7 us), 8192 < N <= 12288 from K = 4096
//    (N = 11008, K = 8192 28.6 -> 24.5 us) and any N > 2048 from K = 14336
//    (N = 28672 100.3 -> 89.5 us); the FMA kernels are faster or level
//    elsewhere (N <= 2048, K = 2048, N = 4097-8192 below K = 14336,
//    N > 12288 below K = 14336);
//  * 5-16 rows: the matrix-core kernels (codes exact in bf16, x as two bf16
//    terms), 9-16 rows on the weight slices where the Q4_0 GEMV takes them
//    (N = 8192, K = 2048, M = 16: 7.9 against 11.4 us; N = 6144, K = 8192:
//    21.0 against 27.9 us).
bool q4_k_rows_on_matrix_cores(int64_t M, int64_t N, int64_t K)
{
    if (M < 3 || N <= 2048) return false;
    return K >= 14336 || (N < 4096 && K > 2048) || (N == 4096 && K >= 8192) ||
           (N > 8192 && N <= 12288 && K >= 4096);
}

hipError_t gemv_q4_k_launch(const float *x, const uint8_t *w, float *y, int64_t M, int64_t N,
                            int64_t K, hipStream_t stream)
{
    if (rows_on_slices(M, N, K))
        return qmm::launch_gemv_slices(qmm::FMT_Q4_K, x, w, y, (int)M, (int)N, (int)K, stream);
    if (M > qmm::kGemvRowsMax || q4_k_rows_on_matrix_cores(M, N, K))
        return qmm::launch_gemv_small_m(qmm::FMT_Q4_K, x, w, y, (int)M, (int)N, (int)K, stream);
    return qmm::launch_gemv_q4_k(x, w, y, (int)M, (int)N, (int)K, stream);
}

int gemm_entry(const char *fn, int fmt, int block_bytes, const float *x, const void *w,
               float *y, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    int st = validate(fn, x, w, y, M, N, K, block_bytes, INT_MAX / 2);
    if (st != QMM_OK) return st;
    // the kernel addresses a 256-row band of y with 32-bit byte offsets
    // (tiles rounded up to a multiple of 8 XCDs must still fit an int grid)
    if (N > QMM_GEMM_MAX_N || ((M + 255) / 256) * ((N + 255) / 256) > INT_MAX - 8)
        return fail(QMM_EUNSUPPORTED,
                    "%s: N=%lld M=%lld unsupported (need N <= %d and at most %d tiles)", fn,
                    (long long)N, (long long)M, QMM_GEMM_MAX_N, INT_MAX - 8);
    const uint8_t *wb = (const uint8_t *)w;
    // Q4_K: up to 4 rows, and up to 16 rows with N <= 4096, take its GEMV,
    // which streams the weights once (FFN shapes, M = 2 and 4: 5.1 and 8.3 us
    // against 9.6 us on the medium-M kernel; 6.3 and 8.1 against 20 us; M =
    // 6: N = 2048, K = 8192 19.1 -> 10.9 us, N = 4096, K = 14336 30.5 -> 16.4
    // us, N = 1024, K = 4096 9.9 -> 6.8 us)
    if (fmt == qmm::FMT_Q4_K) {
        if (M <= qmm::kGemvRowsMax || (M <= QMM_GEMV_MAX_M && N <= 4096))
            return finish(fn, gemv_q4_k_launch(x, wb, y, M, N, K, stream));
        return finish(fn, qmm::launch_gemm(fmt, x, wb, y, (int)M, (int)N, (int)K, stream));
    }
    // Up to 4 rows, and up to 16 rows with N <= 4096, the GEMV's kernels (one
    // pass over the weights, held to the tighter GEMV bound): faster than any
    // prefill tiling there (N = 2048, K = 8192: M = 5 19.3 -> 8.9 us, M = 16
    // 21.1 -> 15.2 us; N = 4096, K = 14336, M = 5: 27.8 -> 13.7 us), while
    // from N = 6144 the medium-M GEMM is level or faster from 9 rows.
    if (M <= qmm::kGemvRowsMax || (M <= QMM_GEMV_MAX_M && N <= 4096))
        return finish(fn, gemv_launch(fmt, x, wb, y, M, N, K, stream));
    return finish(fn, qmm::launch_gemm(fmt, x, wb, y, (int)M, (int)N, (int)K, stream));
}

}  // namespace

extern "C" {

QMM_API int qmm_gemv_q4_0(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream)
{
    const char *fn = "qmm_gemv_q4_0";
    int st = validate(fn, x, w, y, M, N, K, qmm::kQ4Bytes, QMM_GEMV_MAX_M);
    if (st != QMM_OK) return st;
    return finish(fn, gemv_launch(qmm::FMT_Q4_0, x, (const uint8_t *)w, y, M, N, K, stream));
}

QMM_API int qmm_gemv_q8_0(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream)
{
    const char *fn = "qmm_gemv_q8_0";
    int st = validate(fn, x, w, y, M, N, K, qmm::kQ8Bytes, QMM_GEMV_MAX_M);
    if (st != QMM_OK) return st;
    return finish(fn, gemv_launch(qmm::FMT_Q8_0, x, (const uint8_t *)w, y, M, N, K, stream));
}

QMM_API int qmm_gemm_q4_0(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream)
{
    return gemm_entry("qmm_gemm_q4_0", qmm::FMT_Q4_0, qmm::kQ4Bytes, x, w, y, M, N, K, stream);
}

QMM_API int qmm_gemm_q8_0(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream)
{
    return gemm_entry("qmm_gemm_q8_0", qmm::FMT_Q8_0, qmm::kQ8Bytes, x, w, y, M, N, K, stream);
}

QMM_API int qmm_gemm_q4_k(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream)
{
    if (K % 256 && K > 0)
        return fail(QMM_EINVAL,
                    "qmm_gemm_q4_k: K=%lld is not a multiple of 256 (the super-block size)",
                    (long long)K);
    // 144 bytes per 256 weights: Q4_0's byte rate, so its size checks apply
    return gemm_entry("qmm_gemm_q4_k", qmm::FMT_Q4_K, qmm::kQ4Bytes, x, w, y, M, N, K, stream);
}

QMM_API int qmm_ffn_gate_up_q4_0(const float *x, const void *w_gate, const void *w_up,
                                 float *h, int64_t M, int64_t N, int64_t K,
                                 hipStream_t stream)
{
    const char *fn = "qmm_ffn_gate_up_q4_0";
    int st = validate(fn, x, w_gate, h, M, N, K, qmm::kQ4Bytes, QMM_GEMV_MAX_M);
    if (st != QMM_OK) return st;
    if (!w_up) return fail(QMM_EINVAL, "%s: null pointer (w_up)", fn);
    if ((uintptr_t)w_up % 16)
        return fail(QMM_EALIGN, "%s: misaligned pointer (w_up needs 16-byte alignment)", fn);
    const uint64_t w_len = (uint64_t)N * (uint64_t)(K / 32) * (uint64_t)qmm::kQ4Bytes;
    if (overlaps((uintptr_t)h, (uint64_t)M * (uint64_t)N * 4u, (uintptr_t)w_up, w_len))
        return fail(QMM_EINVAL, "%s: h overlaps w_up", fn);
    // 5-16 rows: the matrix-core kernels with gate and up tiles side by
    // side, as for the GEMV: 9-16 rows on the 32-row weight slices where the
    // GEMV takes them, and any K that is not a multiple of 256 there too
    // (the 16x16 kernel takes K in slices of 256); 3-4 rows on the 16x16 kernel where a
    // sweep (N = 2048-28672, K = 1024-8192) found it faster than the f32
    // FMA kernel: from K = 1024 and N = 3072, except above K = 1024 between
    // N = 4096 and 8192 and below K = 4096 beyond N = 16384 (M = 4: N =
    // 4096, K = 2048 7.7 -> 6.6 us; N = 8192, K = 2048 10.4 -> 9.7 us; N =
    // 11008, K = 1024 10.5 -> 8.8 us; N = 14336, K = 4096, M = 3 26.4 -> 23.7
    // us; N = 28672, K = 8192 89.4 -> 74.8 us; N = 6144 from K = 2048 and N =
    // 28672 at K = 2048 stay 2-9 % faster on the FMA kernel, and two rows
    // are faster on it everywhere)
    const bool rows_on_matrix_cores = M >= 3 && K % 256 == 0 && K >= 1024 && N >= 3072 &&
                                      !(N > 4096 && N < 8192 && K > 1024) &&
                                      !(N > 16384 && K < 4096);
    if (M > qmm::kGemvRowsMax && (rows_on_slices(M, N, K) || K % 256))
        return finish(fn, qmm::launch_ffn_gate_up_slices(x, (const uint8_t *)w_gate,
                                                         (const uint8_t *)w_up, h, (int)M,
                                                         (int)N, (int)K, stream));
    if (M > qmm::kGemvRowsMax || rows_on_matrix_cores)
        return finish(fn, qmm::launch_ffn_gate_up_small_m(x, (const uint8_t *)w_gate,
                                                          (const uint8_t *)w_up, h, (int)M,
                                                          (int)N, (int)K, stream));
    return finish(fn, qmm::launch_ffn_gate_up(x, (const uint8_t *)w_gate,
                                              (const uint8_t *)w_up, h, (int)M, (int)N, (int)K,
                                              stream));
}

QMM_API int qmm_gemv_q4_k(const float *x, const void *w, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream)
{
    const char *fn = "qmm_gemv_q4_k";
    if (K % 256 && K > 0)
        return fail(QMM_EINVAL, "%s: K=%lld is not a multiple of 256 (the super-block size)",
                    fn, (long long)K);
    // a super-block row takes 144 bytes per 256 weights, the same bytes per
    // weight as Q4_0's 18 per 32: the shared size and overlap checks apply
    int st = validate(fn, x, w, y, M, N, K, qmm::kQ4Bytes, QMM_GEMV_MAX_M);
    if (st != QMM_OK) return st;
    return finish(fn, gemv_q4_k_launch(x, (const uint8_t *)w, y, M, N, K, stream));
}

QMM_API const char *qmm_status_string(int status)
{
    switch (status) {
    case QMM_OK: return "QMM_OK";
    case QMM_EINVAL: return "QMM_EINVAL";
    case QMM_EALIGN: return "QMM_EALIGN";
    case QMM_EUNSUPPORTED: return "QMM_EUNSUPPORTED";
    case QMM_EHIP: return "QMM_EHIP";
    default: return "QMM_UNKNOWN_STATUS";
    }
}

QMM_API const char *qmm_last_error(void) { return g_last_error; }

QMM_API int qmm_version(void) { return 100; }

}  // extern "C"
