// Decode GEMV, one activation row: y[n] = sum_k x[k] * w[n][k] over GGUF
// Q4_0 or Q8_0 weight blocks, f32 arithmetic.
//
// The weights are read exactly once and dominate the traffic, so the
// kernel is built around streaming them from HBM:
//  * A thread owns one "pair" of consecutive blocks (64 weights; 36 bytes
//    for Q4_0, 68 for Q8_0) at the same K position in RPT different rows.
//    A pair always starts on a dword boundary, so it is fetched with
//    dwordx4 loads; the lanes of a row cover the row's bytes contiguously.
//  * The 64 activations of the thread's pair are loaded once into VGPRs and
//    reused for all RPT rows (x is tiny and cache-resident).
//  * All weight loads of a chunk are issued before any arithmetic, so each
//    thread keeps RPT * pair bytes in flight.
//  * Decode: Q4_0 nibbles become 16*(q-8) as signed bytes with two logic
//    ops per dword and one v_cvt_f32_i32 (SDWA byte select) per weight;
//    Q8_0 bytes convert directly. One FMA per weight; the scale d is
//    applied once per block, and Q4_0's factor 16 once per output.
//  * The T threads of a row reduce with DPP row operations (and through LDS
//    when a row spans several waves), in a fixed order.
#include "qmm_internal.h"

namespace qmm {
namespace {

template <int FMT> struct Pair;

template <> struct Pair<FMT_Q4_0> {
    static constexpr int kDwords = 9;
    static constexpr int kBytes = 36;
    static constexpr float kOutScale = 1.0f / 16.0f;

    __device__ static void load(const uint8_t *p, uint32_t (&D)[kDwords])
    {
        const u32x4_a4 a = *(const u32x4_a4 *)p;
        const u32x4_a4 b = *(const u32x4_a4 *)(p + 16);
        D[0] = a.x; D[1] = a.y; D[2] = a.z; D[3] = a.w;
        D[4] = b.x; D[5] = b.y; D[6] = b.z; D[7] = b.w;
        D[8] = *(const uint32_t *)(p + 32);
    }

    // Pair bytes: [0,2) d0, [2,18) qs of block 0, [18,20) d1, [20,36) qs of
    // block 1. qs[j] holds element j (low nibble) and j + 16 (high nibble).
    __device__ static float dot(const uint32_t (&D)[kDwords], const float (&xv)[64],
                                float acc)
    {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int pb = 2; pb < 18; ++pb) {
            const uint32_t v = D[pb >> 2];
            const int j = pb - 2, b = pb & 3;
            s0 = fmaf(sbyte(lo16(v), b), xv[j], s0);
            s0 = fmaf(sbyte(hi16(v), b), xv[j + 16], s0);
        }
#pragma unroll
        for (int pb = 20; pb < 36; ++pb) {
            const uint32_t v = D[pb >> 2];
            const int j = pb - 20, b = pb & 3;
            s1 = fmaf(sbyte(lo16(v), b), xv[32 + j], s1);
            s1 = fmaf(sbyte(hi16(v), b), xv[48 + j], s1);
        }
        acc = fmaf(half_lo(D[0]), s0, acc);
        acc = fmaf(half_hi(D[4]), s1, acc);
        return acc;
    }
};

template <> struct Pair<FMT_Q8_0> {
    static constexpr int kDwords = 17;
    static constexpr int kBytes = 68;
    static constexpr float kOutScale = 1.0f;

    __device__ static void load(const uint8_t *p, uint32_t (&D)[kDwords])
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4_a4 a = *(const u32x4_a4 *)(p + 16 * i);
            D[4 * i + 0] = a.x; D[4 * i + 1] = a.y;
            D[4 * i + 2] = a.z; D[4 * i + 3] = a.w;
        }
        D[16] = *(const uint32_t *)(p + 64);
    }

    // Pair bytes: [0,2) d0, [2,34) q of block 0, [34,36) d1, [36,68) q of
    // block 1; element j of a block is its byte j.
    __device__ static float dot(const uint32_t (&D)[kDwords], const float (&xv)[64],
                                float acc)
    {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int pb = 2; pb < 34; ++pb)
            s0 = fmaf(sbyte(D[pb >> 2], pb & 3), xv[pb - 2], s0);
#pragma unroll
        for (int pb = 36; pb < 68; ++pb)
            s1 = fmaf(sbyte(D[pb >> 2], pb & 3), xv[32 + pb - 36], s1);
        acc = fmaf(half_lo(D[0]), s0, acc);
        acc = fmaf(half_hi(D[8]), s1, acc);
        return acc;
    }
};

constexpr int kThreads = 256;

// T threads per row (power of two, 4..256), RPT rows per thread.
// Grid: ceil(N / (256 / T * RPT)) workgroups of 256 threads.
template <int FMT, int T, int RPT>
__global__ __launch_bounds__(kThreads) void gemv_m1_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ w,
    float *__restrict__ y, int N, int P)
{
    using L = Pair<FMT>;
    constexpr int RPAR = kThreads / T;          // rows in flight per workgroup
    constexpr int G = T < 64 ? T : 64;          // lanes of a row inside one wave
    constexpr int WPR = T > 64 ? T / 64 : 1;    // waves per row
    const int tid = threadIdx.x;
    const int t = tid % T;
    const int r = tid / T;
    const int64_t row_bytes = (int64_t)P * L::kBytes;
    const int n_first = blockIdx.x * (RPAR * RPT) + r;

    float acc[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) acc[j] = 0.f;

    for (int c = 0; c < P; c += T) {
        const int p = c + t;
        const bool pv = p < P;
        uint32_t D[RPT][L::kDwords];
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int n = n_first + RPAR * j;
            if (pv && n < N) {
                L::load(w + n * row_bytes + (int64_t)p * L::kBytes, D[j]);
            } else {
#pragma unroll
                for (int i = 0; i < L::kDwords; ++i) D[j][i] = 0u;
            }
        }
        float xv[64];
        if (pv) {
            const float4 *xp = reinterpret_cast<const float4 *>(x + 64 * p);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float4 v = xp[i];
                xv[4 * i + 0] = v.x; xv[4 * i + 1] = v.y;
                xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 64; ++i) xv[i] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < RPT; ++j) acc[j] = L::dot(D[j], xv, acc[j]);
    }

#pragma unroll
    for (int j = 0; j < RPT; ++j) acc[j] = group_sum<G>(acc[j]);

    if constexpr (WPR == 1) {
        if (t == T - 1) {
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int n = n_first + RPAR * j;
                if (n < N) y[n] = acc[j] * L::kOutScale;
            }
        }
    } else {
        __shared__ float red[kThreads / 64][RPT];
        const int wave = tid / 64, lane = tid % 64;
        if (lane == 63) {
#pragma unroll
            for (int j = 0; j < RPT; ++j) red[wave][j] = acc[j];
        }
        __syncthreads();
        if (tid < RPAR * RPT) {
            const int rr = tid % RPAR, j = tid / RPAR;
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < WPR; ++q) s += red[rr * WPR + q][j];
            const int n = blockIdx.x * (RPAR * RPT) + rr + RPAR * j;
            if (n < N) y[n] = s * L::kOutScale;
        }
    }
}

template <int FMT, int T, int RPT>
hipError_t launch(const float *x, const uint8_t *w, float *y, int N, int P,
                  hipStream_t stream)
{
    constexpr int rows_per_wg = kThreads / T * RPT;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((gemv_m1_kernel<FMT, T, RPT>), dim3(grid), dim3(kThreads), 0,
                       stream, x, w, y, N, P);
    return hipGetLastError();
}

// Rows per thread: as many as keep at least ~2 workgroups per compute unit
// (256 CUs) busy, so every thread streams several rows' pairs at once.
template <int FMT, int T>
hipError_t launch_t(const float *x, const uint8_t *w, float *y, int N, int P,
                    hipStream_t stream)
{
    constexpr int rpar = kThreads / T;
    const int64_t groups = (N + rpar - 1) / rpar;   // row groups of RPAR rows
    if (groups >= 4 * 512) return launch<FMT, T, 4>(x, w, y, N, P, stream);
    if (groups >= 2 * 512) return launch<FMT, T, 2>(x, w, y, N, P, stream);
    return launch<FMT, T, 1>(x, w, y, N, P, stream);
}

template <int FMT>
hipError_t launch_fmt(const float *x, const uint8_t *w, float *y, int N, int K,
                      hipStream_t stream)
{
    const int P = K / 64;  // pairs per row (K % 256 == 0, so P % 4 == 0)
    if (P <= 4) return launch_t<FMT, 4>(x, w, y, N, P, stream);
    if (P <= 8) return launch_t<FMT, 8>(x, w, y, N, P, stream);
    if (P <= 16) return launch_t<FMT, 16>(x, w, y, N, P, stream);
    if (P <= 32) return launch_t<FMT, 32>(x, w, y, N, P, stream);
    if (P <= 64) return launch_t<FMT, 64>(x, w, y, N, P, stream);
    if (P <= 128) return launch_t<FMT, 128>(x, w, y, N, P, stream);
    return launch_t<FMT, 256>(x, w, y, N, P, stream);
}

}  // namespace

hipError_t launch_gemv_m1(int fmt, const float *x, const uint8_t *w, float *y,
                          int N, int K, hipStream_t stream)
{
    return fmt == FMT_Q4_0 ? launch_fmt<FMT_Q4_0>(x, w, y, N, K, stream)
                           : launch_fmt<FMT_Q8_0>(x, w, y, N, K, stream);
}

}  // namespace qmm
