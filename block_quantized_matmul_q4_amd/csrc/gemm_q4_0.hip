// Prefill GEMM over GGUF Q4_0 weights on the bf16 matrix cores:
// y[m][n] = sum_k bf16(x[m][k]) * bf16(d * (q - 8)) with f32 accumulation.
//
// Workgroup tile BM x BN = 256 x 256, K step 64 (one pair of Q4_0 blocks per
// weight row), 8 waves each owning a 128 x 64 sub-tile as 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 (f32 accumulators, 128 per lane).
//
// Per K step every thread
//  * converts 32 activations (8 float4, one row) from f32 to bf16 (round to
//    nearest even, v_cvt_pk_bf16_f32) on their way into LDS, and
//  * dequantizes one Q4_0 block of one weight row: d * (q - 8) is exact in
//    f32 and is rounded once to bf16 (nearest even) into LDS.
// LDS is double buffered: the global loads of step s+1 are issued before the
// matrix-core work of step s, and their conversion into the other buffer is
// placed between the later substeps' matrix-core instructions; LDS
// fragments are prefetched one 16-wide substep ahead. One barrier per step.
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the
// eight XCDs, and consecutive tiles in band-major order (one 256-row band
// of x with all its column tiles) are given to the same XCD, so each XCD's
// L2 holds the activation band its compute units share.
#include "qmm_internal.h"

namespace qmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WAVES_M = 2, WAVES_N = 4;
constexpr int kThreads = 64 * WAVES_M * WAVES_N;       // 512
constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // 128 x 64 per wave
constexpr int TM = WTM / 32, TN = WTN / 32;            // 4 x 2 MFMA tiles
constexpr int LDK = BK + 8;                            // padded LDS row (bf16)
constexpr int kXcds = 8;
constexpr int A_F4 = BM * BK / 4 / kThreads;           // 8 float4 per thread

static_assert(BN * 2 == kThreads, "one Q4_0 block per thread per K step");

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(kThreads) void gemm_q4_0_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ w,
    float *__restrict__ y, int M, int N, int K, int tiles_m, int tiles_n,
    int per_xcd)
{
    __shared__ __attribute__((aligned(16))) __bf16 As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][BN * LDK];

    // ---- tile of this workgroup (XCD-aware, band-major)
    const int tile = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (tile >= tiles_m * tiles_n) return;
    const int tm = tile / tiles_n, tn = tile % tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int P = K / 64;
    const int64_t row_bytes = (int64_t)P * 36;

    // A staging: 16 threads per row (one float4 each), 32 rows per pass.
    // Rows past M read row M-1: their outputs are never stored.
    const int a_col = (tid % 16) * 4;
    const float *a_src[A_F4];
#pragma unroll
    for (int u = 0; u < A_F4; ++u) {
        const int m = min(m0 + tid / 16 + 32 * u, M - 1);
        a_src[u] = x + (int64_t)m * K + a_col;
    }
    // B staging: thread -> (row tid / 2, block tid % 2) of the tile; the
    // block's 18 bytes lie in the 20 bytes at pair offset 16 * blk.
    const int b_row = tid / 2, b_blk = tid % 2;
    const uint8_t *b_src = w + (int64_t)min(n0 + b_row, N - 1) * row_bytes + 16 * b_blk;

    float4 a_reg[A_F4];
    uint32_t b_reg[5];

    auto load_step = [&](int p) {
#pragma unroll
        for (int u = 0; u < A_F4; ++u)
            a_reg[u] = *reinterpret_cast<const float4 *>(a_src[u] + 64 * p);
        const uint8_t *src = b_src + (int64_t)p * 36;
        const u32x4_a4 v = *reinterpret_cast<const u32x4_a4 *>(src);
        b_reg[0] = v.x; b_reg[1] = v.y; b_reg[2] = v.z; b_reg[3] = v.w;
        b_reg[4] = *reinterpret_cast<const uint32_t *>(src + 16);
    };

    // Writes the prefetched step into LDS buffer buf, in two halves (part 0:
    // activations, part 1: weights) so that each half can be interleaved
    // with matrix-core work.
    auto store_part = [&](int buf, int part) {
        if (part == 0) {
            // A: f32 -> bf16 (RNE)
#pragma unroll
            for (int u = 0; u < A_F4; ++u) {
                const float4 v = a_reg[u];
                uint2 pk;
                pk.x = pack_bf16x2(v.x, v.y);
                pk.y = pack_bf16x2(v.z, v.w);
                *reinterpret_cast<uint2 *>(&As[buf][(tid / 16 + 32 * u) * LDK + a_col]) = pk;
            }
            return;
        }
        // B: block b_blk of the pair -> bf16(d * (q - 8)) (RNE)
        uint32_t qs[4];
        float d;
        if (b_blk == 0) {
            d = half_lo(b_reg[0]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qs[i] = __builtin_amdgcn_alignbyte(b_reg[i + 1], b_reg[i], 2);
        } else {
            d = half_hi(b_reg[0]);
#pragma unroll
            for (int i = 0; i < 4; ++i) qs[i] = b_reg[i + 1];
        }
        const float dq = d * (1.0f / 16.0f);
        __bf16 *dst = &Bs[buf][b_row * LDK + 32 * b_blk];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = lo16(qs[i]), hi = hi16(qs[i]);
            uint2 l, h;
            l.x = pack_bf16x2(sbyte(lo, 0) * dq, sbyte(lo, 1) * dq);
            l.y = pack_bf16x2(sbyte(lo, 2) * dq, sbyte(lo, 3) * dq);
            h.x = pack_bf16x2(sbyte(hi, 0) * dq, sbyte(hi, 1) * dq);
            h.y = pack_bf16x2(sbyte(hi, 2) * dq, sbyte(hi, 3) * dq);
            *reinterpret_cast<uint2 *>(dst + 4 * i) = l;        // elements 4i..4i+3
            *reinterpret_cast<uint2 *>(dst + 16 + 4 * i) = h;   // elements 16+4i..
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int frow = lane % 32, fk = 8 * (lane / 32);

    load_step(0);
    store_part(0, 0);
    store_part(0, 1);
    __syncthreads();

    for (int p = 0; p < P; ++p) {
        const int buf = p & 1;
        const bool more = p + 1 < P;
        if (more) load_step(p + 1);
        const __bf16 *as = &As[buf][(wm * WTM + frow) * LDK + fk];
        const __bf16 *bs = &Bs[buf][(wn * WTN + frow) * LDK + fk];
        // fragments double-buffered across the four 16-wide substeps
        bf16x8 a[2][TM], b[2][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            a[0][i] = *reinterpret_cast<const bf16x8 *>(as + 32 * i * LDK);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            b[0][j] = *reinterpret_cast<const bf16x8 *>(bs + 32 * j * LDK);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int cur = s & 1;
            if (s + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    a[cur ^ 1][i] =
                        *reinterpret_cast<const bf16x8 *>(as + 32 * i * LDK + 16 * (s + 1));
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    b[cur ^ 1][j] =
                        *reinterpret_cast<const bf16x8 *>(bs + 32 * j * LDK + 16 * (s + 1));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j],
                                                                       acc[i][j], 0, 0, 0);
            // the next step's conversions ride along the later substeps'
            // matrix-core work (its loads have had time to land)
            if (more && s >= 2) store_part(buf ^ 1, s - 2);
        }
        __syncthreads();
    }

    // ---- epilogue: acc[i][j][e] = C[32i + 8(e/4) + 4(lane/32) + e%4][32j + lane%32]
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * WTN + 32 * j + lane % 32;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * WTM + 32 * i + 8 * (e / 4) + 4 * (lane / 32) + e % 4;
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
    const int tiles = tiles_m * tiles_n;
    const int per_xcd = (tiles + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(gemm_q4_0_kernel, dim3(per_xcd * kXcds), dim3(kThreads), 0,
                       stream, x, w, y, M, N, K, tiles_m, tiles_n, per_xcd);
    return hipGetLastError();
}

}  // namespace qmm
