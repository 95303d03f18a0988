// Drives every C-ABI entry point of libqmm's host layer (csrc/qmm_api.hip,
// built with AddressSanitizer and UndefinedBehaviorSanitizer and linked with
// the launcher stand-ins of launch_stubs.cpp): argument validation for valid
// and invalid calls, extreme sizes, the route each valid call takes, the
// launch-error path and the thread-local error string. Exits non-zero on the
// first failed check; a sanitizer finding aborts the process.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>

#include "../../include/qmm.h"
#include "stub_record.h"

namespace {

int g_checks = 0;

#define CHECK(cond)                                                                   \
    do {                                                                              \
        ++g_checks;                                                                   \
        if (!(cond)) {                                                                \
            std::fprintf(stderr, "FAILED %s:%d: %s (last error: %s)\n", __FILE__,     \
                         __LINE__, #cond, qmm_last_error());                          \
            std::exit(1);                                                             \
        }                                                                             \
    } while (0)

// fake device addresses (never dereferenced: the launchers are stand-ins)
const uintptr_t A = 0x10000000, B = 0x200000000, C = 0x400000000000;

typedef int (*Entry)(const float *, const void *, float *, int64_t, int64_t, int64_t,
                     hipStream_t);

int call(Entry f, uintptr_t x, uintptr_t w, uintptr_t y, int64_t M, int64_t N, int64_t K)
{
    return f(reinterpret_cast<const float *>(x), reinterpret_cast<const void *>(w),
             reinterpret_cast<float *>(y), M, N, K, nullptr);
}

// a call that must be rejected with `status` before any launch
void rejected(Entry f, uintptr_t x, uintptr_t w, uintptr_t y, int64_t M, int64_t N, int64_t K,
              int status)
{
    const long before = g_stub.calls;
    const int st = call(f, x, w, y, M, N, K);
    CHECK(st == status);
    CHECK(g_stub.calls == before);
    CHECK(std::strlen(qmm_last_error()) > 0);
}

// a call that must launch through `route` with the same sizes
void routed(Entry f, int64_t M, int64_t N, int64_t K, const char *route)
{
    const long before = g_stub.calls;
    const int st = call(f, A, B, C, M, N, K);
    CHECK(st == QMM_OK);
    CHECK(g_stub.calls == before + 1);
    CHECK(std::strcmp(g_stub.route, route) == 0);
    CHECK(g_stub.M == M && g_stub.N == N && g_stub.K == K);
}

// k_status: the status for K a multiple of 32 but not of 64, or past
// QMM_MAX_K (the Q4_K entry points reject any K not a multiple of 256 as
// QMM_EINVAL first)
void common_rejections(Entry f, int64_t max_m, int k_status = QMM_EUNSUPPORTED)
{
    rejected(f, 0, B, C, 1, 8, 256, QMM_EINVAL);
    rejected(f, A, 0, C, 1, 8, 256, QMM_EINVAL);
    rejected(f, A, B, 0, 1, 8, 256, QMM_EINVAL);
    for (int64_t bad : {int64_t(0), int64_t(-1), INT64_MIN}) {
        rejected(f, A, B, C, bad, 8, 256, QMM_EINVAL);
        rejected(f, A, B, C, 1, bad, 256, QMM_EINVAL);
        rejected(f, A, B, C, 1, 8, bad, QMM_EINVAL);
    }
    rejected(f, A, B, C, max_m + 1, 8, 256, QMM_EINVAL);
    rejected(f, A, B, C, INT64_MAX, 8, 256, QMM_EINVAL);
    rejected(f, A, B, C, 1, 8, 48, QMM_EINVAL);                  // not a multiple of 32
    rejected(f, A, B, C, 1, 8, 96, k_status);                    // not a multiple of 64
    rejected(f, A, B, C, 1, 8, QMM_MAX_K + 64, k_status);
    rejected(f, A, B, C, 1, 8, INT64_MAX - 63, k_status);
    rejected(f, A, B, C, 1, INT64_MAX, 256, QMM_EINVAL);         // sizes overflow
    rejected(f, A, B, C, 1, (int64_t)INT_MAX / 2 + 1, 256, QMM_EINVAL);
    rejected(f, A + 4, B, C, 1, 8, 256, QMM_EALIGN);
    rejected(f, A, B + 2, C, 1, 8, 256, QMM_EALIGN);
    rejected(f, A, B, C + 2, 1, 8, 256, QMM_EALIGN);
    rejected(f, A, B, A + 256, 1, 8, 256, QMM_EINVAL);           // y inside x
    rejected(f, A, B, B + 64, 1, 8, 256, QMM_EINVAL);            // y inside w
    rejected(f, A, B, A - 16, 1, 8, 256, QMM_EINVAL);            // y's end inside x
    // the launch-error path: the stand-in reports a HIP error
    const long before = g_stub.calls;
    CHECK(call(f, A, B, C, 1, kFailN, 256) == QMM_EHIP);
    CHECK(g_stub.calls == before + 1);
    CHECK(std::strstr(qmm_last_error(), "launch failed") != nullptr);
}

void gemv_entries()
{
    for (Entry f : {qmm_gemv_q4_0, qmm_gemv_q8_0}) {
        common_rejections(f, QMM_GEMV_MAX_M);
        for (int64_t m = 1; m <= 4; ++m) routed(f, m, 1000, 2048, "gemv_m1");
        routed(f, 1, 1, 64, "gemv_m1");
        routed(f, 1, (int64_t)INT_MAX / 2, 64, "gemv_m1");
        routed(f, 12, 300, 320, "gemv_slices");                  // K % 256 != 0
    }
    routed(qmm_gemv_q4_0, 16, 33, QMM_MAX_K, "gemv_small_m");
    routed(qmm_gemv_q8_0, 16, 33, QMM_MAX_K, "gemv_small_m");
    routed(qmm_gemv_q4_0, 5, 300, 1024, "gemv_small_m");
    routed(qmm_gemv_q4_0, 8, 8192, 2048, "gemv_small_m");
    // 9-16 rows: weight slices above N = 4096, and from N = 3072 at K <= 2048
    routed(qmm_gemv_q4_0, 9, 300, 1024, "gemv_small_m");
    routed(qmm_gemv_q4_0, 9, 8192, 1024, "gemv_slices");
    routed(qmm_gemv_q8_0, 12, 300, 1024, "gemv_small_m");
    routed(qmm_gemv_q8_0, 12, 8192, 1024, "gemv_slices");
    routed(qmm_gemv_q4_0, 12, 4097, 8192, "gemv_slices");
    routed(qmm_gemv_q4_0, 12, 4096, 4096, "gemv_small_m");
    routed(qmm_gemv_q8_0, 16, 3072, 2048, "gemv_slices");
    routed(qmm_gemv_q8_0, 16, 3071, 2048, "gemv_small_m");
    routed(qmm_gemv_q4_0, 16, 3072, 2304, "gemv_small_m");
    // 3-4 rows at some shapes (K % 256 == 0 and K, N >= 4096, or K > 2048
    // with 2048 < N < 4096, or 1024 <= N <= 2048 with K just past 8192):
    // matrix cores
    for (Entry f : {qmm_gemv_q4_0, qmm_gemv_q8_0}) {
        routed(f, 2, 4096, 4096, "gemv_m1");
        routed(f, 3, 4096, 4096, "gemv_small_m");
        routed(f, 4, 14336, 4096, "gemv_small_m");
        routed(f, 4, 4095, 4096, "gemv_small_m");
        routed(f, 4, 4096, 4032, "gemv_m1");
        routed(f, 4, 4096, 4160, "gemv_m1");                      // K % 256 != 0
        routed(f, 3, 3072, 2304, "gemv_small_m");                 // 2048 < N < 4096, K > 2048
        routed(f, 4, 2049, 8192, "gemv_small_m");
        routed(f, 4, 2048, 8192, "gemv_m1");
        routed(f, 4, 3072, 2048, "gemv_m1");
        routed(f, 3, 1536, 8960, "gemv_small_m");                 // 1024 <= N <= 2048, K past 8192
        routed(f, 4, 1024, 12288, "gemv_m1");
        routed(f, 4, 1023, 8960, "gemv_m1");
    }
    routed(qmm_gemv_q4_0, 4, 2048, 10240, "gemv_small_m");       // up to K = 11264
    routed(qmm_gemv_q8_0, 4, 2048, 10240, "gemv_m1");            // up to K = 9216
    routed(qmm_gemv_q8_0, 4, 2048, 9216, "gemv_small_m");
    routed(qmm_gemv_q4_0, 4, 16384, 1536, "gemv_small_m");       // Q4_0, N >= 16384, K >= 1536
    routed(qmm_gemv_q8_0, 4, 16384, 1536, "gemv_m1");
    routed(qmm_gemv_q4_0, 4, 16384, 1280, "gemv_m1");
    routed(qmm_gemv_q4_0, 3, 16383, 2048, "gemv_m1");
}

void gemm_entries()
{
    for (Entry f : {qmm_gemm_q4_0, qmm_gemm_q8_0}) {
        common_rejections(f, (int64_t)INT_MAX / 2);
        for (int64_t m = 1; m <= 4; ++m) routed(f, m, 257, 512, "gemv_m1");
        routed(f, 4, 4096, 4096, "gemv_small_m");                 // as the GEMV
        routed(f, 5, 257, 512, "gemv_small_m");                   // M <= 16, N <= 4096
        routed(f, 16, 4096, 512, "gemv_slices");                  // as the GEMV
        routed(f, 16, 2048, 512, "gemv_small_m");
        routed(f, 12, 4096, 320, "gemv_slices");                  // K % 256 != 0
        routed(f, 17, 257, 512, "gemm");
        routed(f, 5, 4097, 512, "gemm");
        routed(f, 2048, 8192, 2048, "gemm");
        routed(f, (int64_t)INT_MAX / 2, 16, 64, "gemm");
        rejected(f, A, B, C, 5, QMM_GEMM_MAX_N + 1, 64, QMM_EUNSUPPORTED);
    }
    common_rejections(qmm_gemm_q4_k, (int64_t)INT_MAX / 2, QMM_EINVAL);
    rejected(qmm_gemm_q4_k, A, B, C, 5, 8, 320, QMM_EINVAL);    // not a multiple of 256
    routed(qmm_gemm_q4_k, 3, 257, 512, "gemv_q4_k");
    routed(qmm_gemm_q4_k, 5, 257, 512, "gemv_small_m");           // M <= 16, N <= 4096
    routed(qmm_gemm_q4_k, 16, 4096, 512, "gemv_slices");
    routed(qmm_gemm_q4_k, 16, 2048, 512, "gemv_small_m");
    routed(qmm_gemv_q4_k, 12, 5000, 8192, "gemv_slices");
    routed(qmm_gemv_q4_k, 12, 4096, 4096, "gemv_small_m");
    routed(qmm_gemm_q4_k, 5, 4097, 512, "gemm");
    routed(qmm_gemm_q4_k, 17, 257, 512, "gemm");
}

void q4_k_gemv()
{
    common_rejections(qmm_gemv_q4_k, QMM_GEMV_MAX_M, QMM_EINVAL);
    rejected(qmm_gemv_q4_k, A, B, C, 1, 8, 320, QMM_EINVAL);
    for (int64_t m = 1; m <= 4; ++m) routed(qmm_gemv_q4_k, m, 300, 1280, "gemv_q4_k");
    for (int64_t m = 5; m <= QMM_GEMV_MAX_M; ++m) routed(qmm_gemv_q4_k, m, 300, 1280, "gemv_small_m");
    routed(qmm_gemv_q4_k, 16, 33, QMM_MAX_K, "gemv_small_m");
    routed(qmm_gemv_q4_k, 8, 8192, 2048, "gemv_small_m");
    // three and four rows on the matrix cores at some shapes
    routed(qmm_gemv_q4_k, 4, 3072, 4096, "gemv_small_m");        // 2048 < N < 4096, K > 2048
    routed(qmm_gemv_q4_k, 4, 3072, 2304, "gemv_small_m");
    routed(qmm_gemv_q4_k, 4, 3072, 2048, "gemv_q4_k");
    routed(qmm_gemv_q4_k, 3, 4096, 8192, "gemv_small_m");        // N = 4096, K >= 8192
    routed(qmm_gemv_q4_k, 4, 4096, 7936, "gemv_q4_k");
    routed(qmm_gemv_q4_k, 4, 11008, 4096, "gemv_small_m");       // 8192 < N <= 12288, K >= 4096
    routed(qmm_gemv_q4_k, 4, 11008, 2048, "gemv_q4_k");
    routed(qmm_gemv_q4_k, 4, 12289, 4096, "gemv_q4_k");
    routed(qmm_gemv_q4_k, 4, 8192, 8192, "gemv_q4_k");
    routed(qmm_gemv_q4_k, 3, 28672, 14336, "gemv_small_m");      // any N > 2048, K >= 14336
    routed(qmm_gemv_q4_k, 4, 2048, 14336, "gemv_q4_k");
    routed(qmm_gemv_q4_k, 2, 3072, 8192, "gemv_q4_k");
    routed(qmm_gemm_q4_k, 4, 3072, 4096, "gemv_small_m");
    for (int64_t m = 9; m <= QMM_GEMV_MAX_M; ++m) routed(qmm_gemv_q4_k, m, 8192, 2048, "gemv_slices");
}

int gate_up(uintptr_t x, uintptr_t wg, uintptr_t wu, uintptr_t h, int64_t M, int64_t N,
            int64_t K)
{
    return qmm_ffn_gate_up_q4_0(reinterpret_cast<const float *>(x),
                                reinterpret_cast<const void *>(wg),
                                reinterpret_cast<const void *>(wu), reinterpret_cast<float *>(h),
                                M, N, K, nullptr);
}

void gated()
{
    const uintptr_t D = 0x600000000000;
    const long before = g_stub.calls;
    CHECK(gate_up(A, B, D, C, 1, 300, 2048) == QMM_OK);
    CHECK(g_stub.calls == before + 1 && std::strcmp(g_stub.route, "ffn_gate_up") == 0);
    CHECK(gate_up(A, B, 0, C, 1, 300, 2048) == QMM_EINVAL);       // null w_up
    CHECK(gate_up(A, B, D + 2, C, 1, 300, 2048) == QMM_EALIGN);
    CHECK(gate_up(A, B, D, D + 32, 1, 300, 2048) == QMM_EINVAL);  // h inside w_up
    CHECK(gate_up(A, B, D, C, 17, 300, 2048) == QMM_EINVAL);
    CHECK(gate_up(0, B, D, C, 1, 300, 2048) == QMM_EINVAL);
    CHECK(gate_up(A, B, D, C, 1, 300, 96) == QMM_EUNSUPPORTED);
    CHECK(g_stub.calls == before + 1);
    for (int64_t m = 2; m <= 4; ++m) {
        CHECK(gate_up(A, B, D, C, m, 300, 2048) == QMM_OK);
        CHECK(std::strcmp(g_stub.route, "ffn_gate_up") == 0 && g_stub.M == m && g_stub.N == 300);
    }
    CHECK(g_stub.calls == before + 4);
    // 3-4 rows on the matrix cores from K = 1024 and N = 3072, except above
    // K = 1024 at 4096 < N < 8192 and below K = 4096 beyond N = 16384
    CHECK(gate_up(A, B, D, C, 3, 3072, 4096) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up_small_m") == 0);
    CHECK(gate_up(A, B, D, C, 4, 8192, 4096) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up_small_m") == 0);
    CHECK(gate_up(A, B, D, C, 4, 6144, 4096) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up") == 0);
    CHECK(gate_up(A, B, D, C, 4, 8192, 2048) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up_small_m") == 0);
    CHECK(gate_up(A, B, D, C, 4, 6144, 1024) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up_small_m") == 0);
    CHECK(gate_up(A, B, D, C, 3, 3072, 768) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up") == 0);
    CHECK(gate_up(A, B, D, C, 4, 28672, 2048) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up") == 0);
    CHECK(gate_up(A, B, D, C, 4, 28672, 4096) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up_small_m") == 0);
    CHECK(gate_up(A, B, D, C, 4, 2048, 8192) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up") == 0);
    CHECK(gate_up(A, B, D, C, 2, 8192, 8192) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up") == 0);
    CHECK(gate_up(A, B, D, C, 4, 8192, 4160) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up") == 0);
    CHECK(g_stub.calls == before + 15);
    for (int64_t m = 5; m <= QMM_GEMV_MAX_M; ++m) {
        CHECK(gate_up(A, B, D, C, m, 300, 2048) == QMM_OK);
        CHECK(std::strcmp(g_stub.route, "ffn_gate_up_small_m") == 0 && g_stub.M == m &&
              g_stub.N == 300 && g_stub.K == 2048);
    }
    CHECK(g_stub.calls == before + 27);
    // 9-16 rows on the weight slices where the GEMV takes them, and 5-16
    // rows there for any K not a multiple of 256
    CHECK(gate_up(A, B, D, C, 9, 8192, 2048) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up_slices") == 0);
    CHECK(gate_up(A, B, D, C, 16, 3072, 2048) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up_slices") == 0);
    CHECK(gate_up(A, B, D, C, 16, 4096, 4096) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up_small_m") == 0);
    CHECK(gate_up(A, B, D, C, 8, 8192, 2048) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up_small_m") == 0);
    CHECK(gate_up(A, B, D, C, 5, 300, 2112) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up_slices") == 0);
    CHECK(gate_up(A, B, D, C, 4, 300, 2112) == QMM_OK && std::strcmp(g_stub.route, "ffn_gate_up") == 0);
    CHECK(g_stub.calls == before + 33);
}

void strings_and_threads()
{
    CHECK(std::string(qmm_status_string(QMM_OK)) == "QMM_OK");
    CHECK(std::string(qmm_status_string(QMM_EHIP)) == "QMM_EHIP");
    CHECK(std::string(qmm_status_string(-7)) == "QMM_UNKNOWN_STATUS");
    CHECK(qmm_version() >= 100);
    // the error string is per thread
    CHECK(call(qmm_gemv_q4_0, 0, B, C, 1, 8, 256) == QMM_EINVAL);
    std::string other = "unset";
    std::thread t([&] { other = qmm_last_error(); });
    t.join();
    CHECK(other.empty());
    CHECK(std::strlen(qmm_last_error()) > 0);
}

}  // namespace

int main()
{
    gemv_entries();
    gemm_entries();
    q4_k_gemv();
    gated();
    strings_and_threads();
    std::printf("abi checks passed: %d\n", g_checks);
    return 0;
}
