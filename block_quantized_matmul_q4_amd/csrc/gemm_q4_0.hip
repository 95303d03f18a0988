// Prefill GEMM over GGUF Q4_0 weights on the bf16 matrix cores:
// y[m][n] = sum_k bf16(x[m][k]) * bf16(d * (q - 8)) with f32 accumulation.
//
// Per K step of 64 (one pair of blocks per weight row) the workgroup
//  * converts its 128 x 64 activation tile from f32 to bf16 (round to
//    nearest even) while staging it into LDS, and
//  * dequantizes its 128 x 64 weight tile: d * (q - 8) is exact in f32 and
//    is rounded once to bf16 (nearest even) on its way into LDS,
// then four waves, each owning a 64 x 64 sub-tile, run
// v_mfma_f32_16x16x32_bf16 over it. K = 32 per instruction, one block.
#include "qmm_internal.h"

namespace qmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;      // padded LDS row (bf16 elements)
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void gemm_q4_0_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ w,
    float *__restrict__ y, int M, int N, int K, int tiles_m)
{
    __shared__ __attribute__((aligned(16))) __bf16 As[BM * LDK];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[BN * LDK];

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int wm = wave / 2, wn = wave % 2;
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int P = K / 64;
    const int64_t row_bytes = (int64_t)P * 36;

    // A staging: 16 lanes per row, one float4 each, 16 rows per pass.
    const int a_col = (tid % 16) * 4;
    const int a_row = tid / 16;
    // B staging: two threads per weight row, one block each.
    const int b_row = tid / 2, b_blk = tid % 2;
    const int bn = n0 + b_row;
    const uint8_t *b_src = w + (int64_t)(bn < N ? bn : 0) * row_bytes + 16 * b_blk;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int col = lane % 16, g = lane / 16;

    for (int p = 0; p < P; ++p) {
        // ---- stage A (f32 -> bf16)
#pragma unroll
        for (int pass = 0; pass < BM / 16; ++pass) {
            const int r = pass * 16 + a_row;
            const int m = m0 + r;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m < M) v = *(const float4 *)(x + (int64_t)m * K + 64 * p + a_col);
            bf16x4 b;
            b[0] = (__bf16)v.x; b[1] = (__bf16)v.y; b[2] = (__bf16)v.z; b[3] = (__bf16)v.w;
            *(bf16x4 *)(As + r * LDK + a_col) = b;
        }
        // ---- stage B (Q4_0 block -> bf16 d*(q-8))
        {
            // Dwords [16*b_blk, 16*b_blk + 20) of the pair: block 0 uses
            // bytes 0..17 (d at 0, qs at 2), block 1 bytes 18..35 (d at 18,
            // qs at 20); loaded from the dword-aligned offsets 0 and 16.
            const uint8_t *src = b_src + (int64_t)p * 36;
            uint32_t D[5];
            if (bn < N) {
                const u32x4_a4 a = *(const u32x4_a4 *)src;
                D[0] = a.x; D[1] = a.y; D[2] = a.z; D[3] = a.w;
                D[4] = *(const uint32_t *)(src + 16);
            } else {
                D[0] = D[1] = D[2] = D[3] = D[4] = 0u;
            }
            // qs dwords of this block, realigned when the block starts at
            // byte 2 of the loaded window.
            uint32_t qs[4];
            float d;
            if (b_blk == 0) {
                d = half_lo(D[0]);
#pragma unroll
                for (int i = 0; i < 4; ++i) qs[i] = __builtin_amdgcn_alignbyte(D[i + 1], D[i], 2);
            } else {
                d = half_hi(D[0]);
#pragma unroll
                for (int i = 0; i < 4; ++i) qs[i] = D[i + 1];
            }
            const float dq = d * (1.0f / 16.0f);
            __bf16 *dst = Bs + b_row * LDK + 32 * b_blk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16x4 lo, hi;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo[e] = (__bf16)(sbyte(lo16(qs[i]), e) * dq);
                    hi[e] = (__bf16)(sbyte(hi16(qs[i]), e) * dq);
                }
                *(bf16x4 *)(dst + 4 * i) = lo;        // elements 4i..4i+3
                *(bf16x4 *)(dst + 16 + 4 * i) = hi;   // elements 16+4i..
            }
        }
        __syncthreads();
        // ---- MFMA over the 64-wide K step
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *(const bf16x8 *)(As + (wm * 64 + 16 * i + col) * LDK + 32 * kk + 8 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *(const bf16x8 *)(Bs + (wn * 64 + 16 * j + col) * LDK + 32 * kk + 8 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // ---- epilogue: acc[i][j][e] = C[16i + 4g + e][16j + col] of the wave tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + 16 * j + col;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * 64 + 16 * i + 4 * g + e;
                if (m < M && n < N) y[(int64_t)m * N + n] = acc[i][j][e];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_q4_0(const float *x, const uint8_t *w, float *y, int M,
                            int N, int K, hipStream_t stream)
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    hipLaunchKernelGGL(gemm_q4_0_kernel, dim3(tiles_m * tiles_n), dim3(kThreads), 0,
                       stream, x, w, y, M, N, K, tiles_m);
    return hipGetLastError();
}

}  // namespace qmm
