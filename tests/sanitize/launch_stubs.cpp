// Host-only stand-ins for the kernel launchers of libqmm, linked with the
// library's C-ABI layer (csrc/qmm_api.hip) into a sanitizer build that runs
// without a GPU. Each stub records which launcher the entry point chose and
// with which sizes; a stub returns a HIP error when N equals kFailN, so the
// entry points' launch-error path is exercised too.
#include "../../block_quantized_matmul_q4_amd/csrc/qmm_internal.h"

#include "stub_record.h"

StubRecord g_stub;

namespace {
hipError_t record(const char *route, int fmt, int M, int N, int K)
{
    g_stub.route = route;
    g_stub.fmt = fmt;
    g_stub.M = M;
    g_stub.N = N;
    g_stub.K = K;
    g_stub.calls += 1;
    return N == kFailN ? hipErrorInvalidValue : hipSuccess;
}
}  // namespace

namespace qmm {
hipError_t launch_gemv_m1(int fmt, const float *, const uint8_t *, float *, int M, int N, int K,
                          hipStream_t)
{
    return record("gemv_m1", fmt, M, N, K);
}
hipError_t launch_gemv_small_m(int fmt, const float *, const uint8_t *, float *, int M, int N,
                               int K, hipStream_t)
{
    return record("gemv_small_m", fmt, M, N, K);
}
hipError_t launch_gemv_slices(int fmt, const float *, const uint8_t *, float *, int M, int N,
                              int K, hipStream_t)
{
    return record("gemv_slices", fmt, M, N, K);
}
hipError_t launch_ffn_gate_up(const float *, const uint8_t *, const uint8_t *, float *, int M,
                              int N, int K, hipStream_t)
{
    return record("ffn_gate_up", FMT_Q4_0, M, N, K);
}
hipError_t launch_ffn_gate_up_small_m(const float *, const uint8_t *, const uint8_t *, float *,
                                      int M, int N, int K, hipStream_t)
{
    return record("ffn_gate_up_small_m", FMT_Q4_0, M, N, K);
}
hipError_t launch_ffn_gate_up_slices(const float *, const uint8_t *, const uint8_t *, float *,
                                     int M, int N, int K, hipStream_t)
{
    return record("ffn_gate_up_slices", FMT_Q4_0, M, N, K);
}
hipError_t launch_gemv_q4_k(const float *, const uint8_t *, float *, int M, int N, int K,
                            hipStream_t)
{
    return record("gemv_q4_k", FMT_Q4_K, M, N, K);
}
hipError_t launch_gemm(int fmt, const float *, const uint8_t *, float *, int M, int N, int K,
                       hipStream_t)
{
    return record("gemm", fmt, M, N, K);
}
}  // namespace qmm
