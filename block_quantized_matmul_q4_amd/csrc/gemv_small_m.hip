// Small-M GEMV (2 <= M <= 16 activation rows: batched or speculative
// decode) over GGUF Q4_0 / Q8_0 weights, on the bf16 matrix cores.
//
// With several activation rows the f32 FMA count (M per weight) outgrows
// the weight stream, so the contraction moves to v_mfma_f32_16x16x32_bf16:
// one instruction covers 16 activation rows x 16 weight rows x one 32-wide
// block. Exactness is kept where it matters:
//  * B operand (weights): the integer codes 16*(q-8) (Q4_0) or q (Q8_0),
//    exact in bf16. The fp16 scale d is applied in f32 to the block's
//    16x16 result, so no weight is rounded.
//  * A operand (activations): x = hi + lo with hi = bf16(x) and
//    lo = bf16(x - hi), both round-to-nearest-even; the two products are
//    exact and accumulate in f32. The representation error is at most
//    2^-17 |x| per term, far inside the 1e-4 relative bound.
// Within a block the k order is permuted identically in A and B so that
// each lane's eight weights come from one qs dword (Q4_0: bytes 4g..4g+3,
// i.e. elements 4g..4g+3 and 4g+16..4g+19; Q8_0: elements 8g..8g+7).
//
// Work split: a workgroup owns 16 weight rows; its four waves take
// interleaved pairs of blocks along K and are summed through LDS in a fixed
// order (bitwise reproducible).
#include "qmm_internal.h"

namespace qmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;

__device__ __forceinline__ void split8(const float4 a, const float4 b, bf16x8 &hi,
                                       bf16x8 &lo)
{
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const __bf16 h = (__bf16)v[i];
        hi[i] = h;
        lo[i] = (__bf16)(v[i] - (float)h);
    }
}

__device__ __forceinline__ uint32_t ld32(const uint8_t *p)
{
    return *(const uint32_t *)p;
}

template <int FMT> struct SmallM;

template <> struct SmallM<FMT_Q4_0> {
    static constexpr int kPairBytes = 36;
    static constexpr float kOutScale = 1.0f / 16.0f;

    // Lane group g of the pair starting at p: codes of block 0 and 1, scales.
    __device__ static void load(const uint8_t *p, int g, bf16x8 &b0, bf16x8 &b1,
                                float &d0, float &d1)
    {
        const uint32_t q0 = __builtin_amdgcn_alignbyte(ld32(p + 4 * g + 4),
                                                       ld32(p + 4 * g), 2);
        const uint32_t q1 = ld32(p + 20 + 4 * g);
        d0 = half_lo(ld32(p));
        d1 = half_hi(ld32(p + 16));
        const uint32_t l0 = lo16(q0), h0 = hi16(q0), l1 = lo16(q1), h1 = hi16(q1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            b0[e] = (__bf16)sbyte(l0, e);
            b0[4 + e] = (__bf16)sbyte(h0, e);
            b1[e] = (__bf16)sbyte(l1, e);
            b1[4 + e] = (__bf16)sbyte(h1, e);
        }
    }

    // Element offsets (within the pair's 64 k) of lane group g's first and
    // second four activations for block 0; block 1 adds 32.
    __device__ static int xoff_a(int g) { return 4 * g; }
    __device__ static int xoff_b(int g) { return 16 + 4 * g; }
};

template <> struct SmallM<FMT_Q8_0> {
    static constexpr int kPairBytes = 68;
    static constexpr float kOutScale = 1.0f;

    __device__ static void load(const uint8_t *p, int g, bf16x8 &b0, bf16x8 &b1,
                                float &d0, float &d1)
    {
        const uint32_t a0 = ld32(p + 8 * g), a1 = ld32(p + 8 * g + 4),
                       a2 = ld32(p + 8 * g + 8);
        const uint32_t q00 = __builtin_amdgcn_alignbyte(a1, a0, 2);
        const uint32_t q01 = __builtin_amdgcn_alignbyte(a2, a1, 2);
        const uint32_t q10 = ld32(p + 36 + 8 * g), q11 = ld32(p + 40 + 8 * g);
        d0 = half_lo(ld32(p));
        d1 = half_hi(ld32(p + 32));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            b0[e] = (__bf16)sbyte(q00, e);
            b0[4 + e] = (__bf16)sbyte(q01, e);
            b1[e] = (__bf16)sbyte(q10, e);
            b1[4 + e] = (__bf16)sbyte(q11, e);
        }
    }

    __device__ static int xoff_a(int g) { return 8 * g; }
    __device__ static int xoff_b(int g) { return 8 * g + 4; }
};

template <int FMT>
__global__ __launch_bounds__(64 * kWaves) void gemv_small_m_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ w,
    float *__restrict__ y, int M, int N, int K)
{
    using L = SmallM<FMT>;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int col = lane % 16, g = lane / 16;
    const int n = blockIdx.x * 16 + col;
    const int P = K / 64;
    const int64_t row_bytes = (int64_t)P * L::kPairBytes;
    // Rows past N / M read row 0 (always valid) and are never stored.
    const uint8_t *wrow = w + (n < N ? n : 0) * row_bytes;
    const bool mv = col < M;
    const float *xrow = x + (int64_t)(mv ? col : 0) * K;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int p = wave; p < P; p += kWaves) {
        bf16x8 b0, b1;
        float d0, d1;
        L::load(wrow + (int64_t)p * L::kPairBytes, g, b0, b1, d0, d1);
        const float *xp = xrow + 64 * p;
        float4 xa0 = *(const float4 *)(xp + L::xoff_a(g));
        float4 xb0 = *(const float4 *)(xp + L::xoff_b(g));
        float4 xa1 = *(const float4 *)(xp + 32 + L::xoff_a(g));
        float4 xb1 = *(const float4 *)(xp + 32 + L::xoff_b(g));
        if (!mv) {
            xa0 = xb0 = xa1 = xb1 = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        bf16x8 h0, l0, h1, l1;
        split8(xa0, xb0, h0, l0);
        split8(xa1, xb1, h1, l1);
        f32x4 c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h0, b0, zero, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l0, b0, c0, 0, 0, 0);
        f32x4 c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h1, b1, zero, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l1, b1, c1, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[i] = fmaf(d0, c0[i], acc[i]);
            acc[i] = fmaf(d1, c1[i], acc[i]);
        }
    }

    // acc[i] is C[m = 4g + i][n]; sum the four waves in a fixed order.
    __shared__ f32x4 red[kWaves][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f32x4 s = red[0][lane];
#pragma unroll
        for (int q = 1; q < kWaves; ++q) {
            const f32x4 v = red[q][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) s[i] += v[i];
        }
        if (n < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * g + i;
                if (m < M) y[(int64_t)m * N + n] = s[i] * L::kOutScale;
            }
        }
    }
}

}  // namespace

hipError_t launch_gemv_small_m(int fmt, const float *x, const uint8_t *w, float *y,
                               int M, int N, int K, hipStream_t stream)
{
    const int grid = (N + 15) / 16;
    if (fmt == FMT_Q4_0)
        hipLaunchKernelGGL((gemv_small_m_kernel<FMT_Q4_0>), dim3(grid),
                           dim3(64 * kWaves), 0, stream, x, w, y, M, N, K);
    else
        hipLaunchKernelGGL((gemv_small_m_kernel<FMT_Q8_0>), dim3(grid),
                           dim3(64 * kWaves), 0, stream, x, w, y, M, N, K);
    return hipGetLastError();
}

}  // namespace qmm
