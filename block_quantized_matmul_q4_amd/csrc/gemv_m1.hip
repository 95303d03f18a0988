// Decode GEMV, one activation row: y[n] = sum_k x[k] * w[n][k] over GGUF
// Q4_0 or Q8_0 weight blocks, f32 arithmetic.
//
// The weights are read exactly once and dominate the traffic, so the
// kernel is built around streaming them from HBM:
//  * A thread owns one "pair" of consecutive blocks (64 weights; 36 bytes
//    for Q4_0, 68 for Q8_0) at the same K position in RPT different rows.
//    A pair always starts on a dword boundary, so it is fetched with
//    dwordx4 loads; the lanes of a row cover the row's bytes contiguously.
//  * The activations are staged once per workgroup into LDS with coalesced
//    loads; each thread reads the 64 of its pair into VGPRs and reuses them
//    for all RPT rows.
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

// Weight loads; NT marks them non-temporal (streamed once, not worth caching).
template <bool NT>
__device__ __forceinline__ u32x4_a4 ld(const u32x4_a4 *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ uint32_t ld(const uint32_t *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int FMT> struct Pair;

template <> struct Pair<FMT_Q4_0> {
    static constexpr int kDwords = 9;
    static constexpr int kBytes = 36;
    static constexpr float kOutScale = 1.0f / 16.0f;

    template <bool NT>
    __device__ static void load(const uint8_t *p, uint32_t (&D)[kDwords])
    {
        const u32x4_a4 a = ld<NT>((const u32x4_a4 *)p);
        const u32x4_a4 b = ld<NT>((const u32x4_a4 *)(p + 16));
        D[0] = a.x; D[1] = a.y; D[2] = a.z; D[3] = a.w;
        D[4] = b.x; D[5] = b.y; D[6] = b.z; D[7] = b.w;
        D[8] = ld<NT>((const uint32_t *)(p + 32));
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

    // dot() in chunks, for reuse of each activation chunk over several
    // weight rows: chunk i of block b covers elements 4i..4i+3 (low
    // nibbles) and 16+4i..16+4i+3 (high nibbles); chunk_fma runs exactly
    // dot()'s operations for them, in dot()'s order, so the chunks of a block
    // in turn round identically to dot().
    static constexpr int kChunks = 4;           // per block
    static constexpr int kChunkCodes = 8;
    static constexpr bool kHiHalf = true;       // chunks also read x[16 + ..]
    __device__ static void chunk_codes(const uint32_t (&D)[kDwords], int b, int i,
                                       float (&wc)[kChunkCodes])
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int pb = 2 + 18 * b + 4 * i + e;
            const uint32_t v = D[pb >> 2];
            wc[e] = sbyte(lo16(v), pb & 3);
            wc[4 + e] = sbyte(hi16(v), pb & 3);
        }
    }
    __device__ static float chunk_fma(float s, const float (&wc)[kChunkCodes], float4 lo,
                                      float4 hi)
    {
        s = fmaf(wc[0], lo.x, s); s = fmaf(wc[4], hi.x, s);
        s = fmaf(wc[1], lo.y, s); s = fmaf(wc[5], hi.y, s);
        s = fmaf(wc[2], lo.z, s); s = fmaf(wc[6], hi.z, s);
        s = fmaf(wc[3], lo.w, s); s = fmaf(wc[7], hi.w, s);
        return s;
    }
    __device__ static float scale(const uint32_t (&D)[kDwords], int b)
    {
        return b ? half_hi(D[4]) : half_lo(D[0]);
    }
};

template <> struct Pair<FMT_Q8_0> {
    static constexpr int kDwords = 17;
    static constexpr int kBytes = 68;
    static constexpr float kOutScale = 1.0f;

    template <bool NT>
    __device__ static void load(const uint8_t *p, uint32_t (&D)[kDwords])
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4_a4 a = ld<NT>((const u32x4_a4 *)(p + 16 * i));
            D[4 * i + 0] = a.x; D[4 * i + 1] = a.y;
            D[4 * i + 2] = a.z; D[4 * i + 3] = a.w;
        }
        D[16] = ld<NT>((const uint32_t *)(p + 64));
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

    // chunk i of block b: elements 4i..4i+3 (see Pair<FMT_Q4_0>)
    static constexpr int kChunks = 8;
    static constexpr int kChunkCodes = 4;
    static constexpr bool kHiHalf = false;
    __device__ static void chunk_codes(const uint32_t (&D)[kDwords], int b, int i,
                                       float (&wc)[kChunkCodes])
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int pb = 2 + 34 * b + 4 * i + e;
            wc[e] = sbyte(D[pb >> 2], pb & 3);
        }
    }
    __device__ static float chunk_fma(float s, const float (&wc)[kChunkCodes], float4 v, float4)
    {
        s = fmaf(wc[0], v.x, s); s = fmaf(wc[1], v.y, s);
        s = fmaf(wc[2], v.z, s); s = fmaf(wc[3], v.w, s);
        return s;
    }
    __device__ static float scale(const uint32_t (&D)[kDwords], int b)
    {
        return b ? half_hi(D[8]) : half_lo(D[0]);
    }
};

// T threads per row (power of two, 4..WG), RPT rows per thread, CH chunks
// of T pairs per pass along K, WG threads per workgroup, SX activations
// staged once per workgroup (else once per wave), NT non-temporal weight
// loads, MR activation rows (M <= MR; rows past M repeat row M-1 and are not
// stored). Grid: ceil(N / (WG / T * RPT)) workgroups.
//
// GATED (RPT = 2): the gated FFN front half. A thread's two rows are row n
// of the gate matrix w and row n of the up matrix w2, and the output is
// y[m][n] = gelu_tanh(gate) * up for each activation row m, with
// gelu_tanh(g) = g/2 (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))), evaluated in
// f32 once the two sums are complete. Grid: ceil(N / (WG / T)) workgroups.
//
// A wave owns TW = min(T, 64) consecutive pairs of each chunk for its rows
// (a row wider than one wave is split over T / 64 waves). Per pass of CH
// chunks along K:
//  1. the activations of the pass's pairs (64 floats each, MR rows) are
//     loaded with coalesced 16-byte loads (L2-resident after the first
//     workgroup): by the whole workgroup (SX) or by each wave for its own
//     pairs;
//  2. each thread issues the loads of all its CH * RPT weight pairs (HBM);
//  3. the activations go to LDS, in rows of 64 floats padded by 4 so that
//     consecutive lanes' 16-byte reads fall in distinct banks; SX needs one
//     workgroup barrier after the writes (the weights are already in
//     flight; where measured faster it waits for LDS only, so each wave
//     reads its activations while its weights arrive) and, from the second
//     pass on, one before them; per-wave staging none;
//  4. per chunk, each thread runs the FMAs for its RPT weight rows against
//     its 64 activations of each of the MR rows. With one activation row the
//     codes are converted as they are used; with several, a pair is decoded
//     once into 64 floats and reused for every activation row, in the same
//     order of operations, so each output row rounds exactly as in a
//     one-row call.
// Every load is unconditional from a clamped in-bounds address: rows past N
// are computed and dropped, pairs past P are masked by a select.
template <int FMT, int T, int RPT, int CH, int WG, bool SX, bool NT, bool GATED, int MR>
__global__ __launch_bounds__(WG) void gemv_m1_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ w,
    const uint8_t *__restrict__ w2, float *__restrict__ y, int M, int N, int P)
{
    using L = Pair<FMT>;
    static_assert(!GATED || RPT == 2, "gated: one gate row and one up row per thread");
    constexpr int RPAR = WG / T;                // rows in flight per workgroup
    constexpr int TW = T < 64 ? T : 64;         // pairs per wave per chunk
    constexpr int WPR = T / TW;                 // waves per row
    constexpr int XS = 68;                      // padded LDS row (floats)
    // staging unit: the whole workgroup for all T pairs of a chunk (SX), or
    // one wave for its TW pairs
    constexpr int SP = SX ? T : TW;             // pairs staged per unit and chunk
    constexpr int ST = SX ? WG : 64;            // threads per staging unit
    constexpr int XF4 = 16 * SP * CH / ST;      // float4s per thread, row and pass
    static_assert(16 * SP * CH % ST == 0, "staging must tile the pass exactly");
    constexpr int REGION = CH * SP * XS;        // floats per staging unit and row
    constexpr int UNITS = SX ? 1 : WG / 64;
    // After the shared staging, let each wave go on to its LDS reads while
    // its weights are still arriving. Measured faster with T = 128 (FFN
    // down, K = 8192, N = 2048: 4.87 -> 4.67 us; gated, 6.93 -> 6.47 us)
    // and with T = 32 in 256-thread workgroups (FFN up shape, 4 activation
    // rows: 6.62 -> 6.30 us); slower with 512-thread workgroups of T = 32 or
    // T = 64 (Q4_0, N = 262144, K = 2048: 58 -> 62 us).
    constexpr bool LB = SX && (T == 128 || (T == 32 && WG == 256));
    __shared__ __attribute__((aligned(16))) float xs_all[UNITS * MR * REGION];
    // per-wave partials of rows split over several waves, apart from the
    // activations so that no barrier has to wait for their last readers
    __shared__ float red[WPR > 1 ? WG / 64 * RPT * MR : 1];

    const int tid = threadIdx.x;
    const int lane = tid % 64, wave = tid / 64;
    const int t = tid % T;
    const int r = tid / T;
    const int tw0 = t - lane % TW;              // first pair index of this wave
    const int sid = SX ? tid : lane;            // thread index in its unit
    const int sp0 = SX ? 0 : tw0;               // first pair staged by the unit
    const int lp = SX ? t : lane % TW;          // this thread's pair in the unit
    float *xs = xs_all + (SX ? 0 : wave * MR * REGION);   // [MR][CH * SP][XS]
    const int64_t row_bytes = (int64_t)P * L::kBytes;
    const int n_first = blockIdx.x * (RPAR * (GATED ? 1 : RPT)) + r;

    const uint8_t *wrow[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        if constexpr (GATED)
            wrow[j] = (j == 0 ? w : w2) + (int64_t)min(n_first, N - 1) * row_bytes;
        else
            wrow[j] = w + (int64_t)min(n_first + RPAR * j, N - 1) * row_bytes;
    }
    const float *xrow[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) xrow[m] = x + (int64_t)min(m, M - 1) * (64 * P);

    float acc[RPT][MR];
#pragma unroll
    for (int j = 0; j < RPT; ++j)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[j][m] = 0.f;

    for (int c0 = 0; c0 < P; c0 += CH * T) {
        // 1. activations: float4 i of the unit's pass belongs to chunk
        //    i / (16 SP), pair (i / 16) % SP of that chunk (clamped to P-1).
        //    Four scalar arrays, not one of float4: the float4 array ends up
        //    in scratch memory once XF4 >= 4 with workgroup-wide staging.
        float xsx[MR][XF4], xsy[MR][XF4], xsz[MR][XF4], xsw[MR][XF4];
#pragma unroll
        for (int u = 0; u < XF4; ++u) {
            const int i = sid + ST * u;
            const int h = i / (16 * SP), q = (i / 16) % SP;
            const int pp = min(c0 + h * T + sp0 + q, P - 1);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float4 v =
                    *reinterpret_cast<const float4 *>(xrow[m] + 64 * pp + 4 * (i % 16));
                xsx[m][u] = v.x; xsy[m][u] = v.y; xsz[m][u] = v.z; xsw[m][u] = v.w;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // 2. weight pairs
        uint32_t D[CH][RPT][L::kDwords];
#pragma unroll
        for (int h = 0; h < CH; ++h) {
            const int pc = min(c0 + h * T + t, P - 1);
#pragma unroll
            for (int j = 0; j < RPT; ++j)
                L::template load<NT>(wrow[j] + (int64_t)pc * L::kBytes, D[h][j]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // 3. activations to LDS
        if constexpr (SX) {
            if (c0 != 0) __syncthreads();       // previous pass's readers done
        } else {
            wave_lds_sync();
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
#pragma unroll
            for (int u = 0; u < XF4; ++u) {
                const int i = sid + ST * u;
                *reinterpret_cast<float4 *>(&xs[m * REGION + (i / 16) * XS + 4 * (i % 16)]) =
                    make_float4(xsx[m][u], xsy[m][u], xsz[m][u], xsw[m][u]);
            }
        }
        if constexpr (LB) lds_only_barrier();
        else if constexpr (SX) __syncthreads();
        else wave_lds_sync();
        // 4. per chunk: FMAs
#pragma unroll
        for (int h = 0; h < CH; ++h) {
            const bool pv = c0 + h * T + t < P;
            if constexpr (MR == 1) {
                float xv[64];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float4 v = *reinterpret_cast<const float4 *>(
                        &xs[(h * SP + lp) * XS + 4 * i]);
                    xv[4 * i + 0] = v.x; xv[4 * i + 1] = v.y;
                    xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
                }
#pragma unroll
                for (int j = 0; j < RPT; ++j) {
                    const float part = L::dot(D[h][j], xv, 0.f);
                    acc[j][0] += pv ? part : 0.f;
                }
            } else {
                // chunk by chunk: each activation chunk is read from LDS once
                // for all RPT weight rows, each chunk of codes decoded once
                // for all MR activation rows
                float s[RPT][MR][2];
#pragma unroll
                for (int j = 0; j < RPT; ++j)
#pragma unroll
                    for (int m = 0; m < MR; ++m) s[j][m][0] = s[j][m][1] = 0.f;
#pragma unroll
                for (int b = 0; b < 2; ++b) {
#pragma unroll
                    for (int i = 0; i < L::kChunks; ++i) {
                        float4 xl[MR], xh[MR];
#pragma unroll
                        for (int m = 0; m < MR; ++m) {
                            const float *xp = &xs[m * REGION + (h * SP + lp) * XS + 32 * b + 4 * i];
                            xl[m] = *reinterpret_cast<const float4 *>(xp);
                            if constexpr (L::kHiHalf)
                                xh[m] = *reinterpret_cast<const float4 *>(xp + 16);
                            else
                                xh[m] = xl[m];
                        }
#pragma unroll
                        for (int j = 0; j < RPT; ++j) {
                            float wc[L::kChunkCodes];
                            L::chunk_codes(D[h][j], b, i, wc);
#pragma unroll
                            for (int m = 0; m < MR; ++m)
                                s[j][m][b] = L::chunk_fma(s[j][m][b], wc, xl[m], xh[m]);
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < RPT; ++j) {
                    const float d0 = L::scale(D[h][j], 0), d1 = L::scale(D[h][j], 1);
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const float part = fmaf(d1, s[j][m][1], fmaf(d0, s[j][m][0], 0.f));
                        acc[j][m] += pv ? part : 0.f;
                    }
                }
            }
        }
    }

#pragma unroll
    for (int j = 0; j < RPT; ++j)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[j][m] = group_sum<TW>(acc[j][m]);

    if constexpr (WPR == 1 && GATED) {
        if (t == T - 1 && n_first < N) {
#pragma unroll
            for (int m = 0; m < MR; ++m)
                if (m < M)
                    y[(int64_t)m * N + n_first] =
                        gelu_tanh(acc[0][m] * L::kOutScale) * (acc[1][m] * L::kOutScale);
        }
    } else if constexpr (WPR == 1) {
        if (t == T - 1) {
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int n = n_first + RPAR * j;
#pragma unroll
                for (int m = 0; m < MR; ++m)
                    if (n < N && m < M) y[(int64_t)m * N + n] = acc[j][m] * L::kOutScale;
            }
        }
    } else {
        // red[wave][RPT][MR]
        if (lane == 63) {
#pragma unroll
            for (int j = 0; j < RPT; ++j)
#pragma unroll
                for (int m = 0; m < MR; ++m) red[(wave * RPT + j) * MR + m] = acc[j][m];
        }
        __syncthreads();
        if constexpr (GATED) {
            if (tid < RPAR * MR) {
                const int m = tid % MR, rr = tid / MR;
                float sg = 0.f, su = 0.f;
#pragma unroll
                for (int q = 0; q < WPR; ++q) {
                    sg += red[((rr * WPR + q) * RPT + 0) * MR + m];
                    su += red[((rr * WPR + q) * RPT + 1) * MR + m];
                }
                const int n = blockIdx.x * RPAR + rr;
                if (n < N && m < M)
                    y[(int64_t)m * N + n] = gelu_tanh(sg * L::kOutScale) * (su * L::kOutScale);
            }
        } else if (tid < RPAR * RPT * MR) {
            const int m = tid % MR, rr = (tid / MR) % RPAR, j = tid / (MR * RPAR);
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < WPR; ++q) s += red[((rr * WPR + q) * RPT + j) * MR + m];
            const int n = blockIdx.x * (RPAR * RPT) + rr + RPAR * j;
            if (n < N && m < M) y[(int64_t)m * N + n] = s * L::kOutScale;
        }
    }
}

constexpr int kThreads = 256;

template <int FMT, int T, int RPT, int WG = kThreads, int CH = 1, bool SX = false,
          bool NT = false, int MR = 1>
hipError_t launch(const float *x, const uint8_t *w, float *y, int M, int N, int P,
                  hipStream_t stream)
{
    constexpr int rows_per_wg = WG / T * RPT;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((gemv_m1_kernel<FMT, T, RPT, CH, WG, SX, NT, false, MR>), dim3(grid),
                       dim3(WG), 0, stream, x, w, nullptr, y, M, N, P);
    return hipGetLastError();
}

template <int T, int WG = kThreads, bool SX = false, int MR = 1>
hipError_t launch_gated(const float *x, const uint8_t *wg, const uint8_t *wu, float *h, int M,
                        int N, int P, hipStream_t stream)
{
    constexpr int rows_per_wg = WG / T;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((gemv_m1_kernel<FMT_Q4_0, T, 2, 1, WG, SX, false, true, MR>), dim3(grid),
                       dim3(WG), 0, stream, x, wg, wu, h, M, N, P);
    return hipGetLastError();
}

// Launch shapes, from timing sweeps on MI355X over random weights (cold,
// 9 MB to 570 MB per call; uniform bytes draw more power than constant
// ones and change the ranking). P = pairs per row = K / 64; MR activation
// rows per launch (1, 2, or 4 for M = 3, 4).
//   P <= 16 : one wave-local chunk of T = P pairs, 2 rows per thread
//   P <= 32 : T = 32, one row per thread, workgroups sharing one
//             activation copy: 512 threads from N = 65536 (MR = 2: T = 16 x
//             2 chunks; MR = 4: 2 rows per thread), else 256
//   P <= 64 : T = 64, one row per thread, 512-thread workgroups sharing one
//             activation copy (MR = 1 with N >= 32768: T = 32 x 2 chunks;
//             Q4_0, N = 128256, K = 4096: 68-75 -> 57 us)
//   P > 64  : from N = 4096, T = 64 looping over K in chunks of 64 pairs,
//             512-thread workgroups sharing one activation copy, 2 rows per
//             thread with MR = 4, and with MR = 2 from N = 8192 and K = 8192
//             (N = 28672, K = 8192 against T = 128: Q4_0 43.7 -> 29.9 us at
//             M = 1, 50.1 -> 35.6 at M = 2, 82.9 -> 56.1 at M = 4; Q8_0
//             44.3 -> 42.9, 62.8 -> 47.9, 93.6 -> 62.3). Below N = 4096,
//             T = 128 (a row spans two waves) in 512 threads (MR = 4: 2 rows
//             per thread; Q8_0 with MR = 1 from N = 2048: 1024 threads)
template <int FMT, int MR>
hipError_t launch_fmt(const float *x, const uint8_t *w, float *y, int M, int N, int K,
                      hipStream_t stream)
{
    const int P = K / 64;  // K % 64 == 0
    if (P <= 4) return launch<FMT, 4, 2, 256, 1, false, false, MR>(x, w, y, M, N, P, stream);
    if (P <= 8) return launch<FMT, 8, 2, 256, 1, false, false, MR>(x, w, y, M, N, P, stream);
    if (P <= 16) return launch<FMT, 16, 2, 256, 1, false, false, MR>(x, w, y, M, N, P, stream);
    if (P <= 32) {
        if constexpr (MR == 1) {
            if (N >= 65536)
                return launch<FMT, 32, 1, 512, 1, true, false, 1>(x, w, y, M, N, P, stream);
            return launch<FMT, 32, 1, 256, 1, true, false, 1>(x, w, y, M, N, P, stream);
        } else if constexpr (MR == 2) {
            if (N >= 65536)
                return launch<FMT, 16, 1, 512, 2, true, false, 2>(x, w, y, M, N, P, stream);
            return launch<FMT, 32, 1, 256, 1, true, false, 2>(x, w, y, M, N, P, stream);
        } else {
            if (N >= 65536)
                return launch<FMT, 32, 2, 512, 1, true, false, MR>(x, w, y, M, N, P, stream);
            return launch<FMT, 32, 1, 256, 1, true, false, MR>(x, w, y, M, N, P, stream);
        }
    }
    if (P <= 64) {
        if (MR == 1 && N >= 32768)
            return launch<FMT, 32, 1, 512, 2, true, false, 1>(x, w, y, M, N, P, stream);
        return launch<FMT, 64, 1, 512, 1, true, false, MR>(x, w, y, M, N, P, stream);
    }
    if (N >= 4096) {
        if constexpr (MR == 4)
            return launch<FMT, 64, 2, 512, 1, true, false, MR>(x, w, y, M, N, P, stream);
        if constexpr (MR == 2)
            if (N >= 8192 && P >= 128)
                return launch<FMT, 64, 2, 512, 1, true, false, MR>(x, w, y, M, N, P, stream);
        return launch<FMT, 64, 1, 512, 1, true, false, MR>(x, w, y, M, N, P, stream);
    }
    if constexpr (FMT == FMT_Q8_0 && MR == 1)
        if (N >= 2048)
            return launch<FMT, 128, 1, 1024, 1, true, false, MR>(x, w, y, M, N, P, stream);
    if (MR == 4) return launch<FMT, 128, 2, 512, 1, true, false, MR>(x, w, y, M, N, P, stream);
    return launch<FMT, 128, 1, 512, 1, true, false, MR>(x, w, y, M, N, P, stream);
}

template <int FMT>
hipError_t launch_rows(const float *x, const uint8_t *w, float *y, int M, int N, int K,
                       hipStream_t stream)
{
    if (M == 1) return launch_fmt<FMT, 1>(x, w, y, M, N, K, stream);
    if (M == 2) return launch_fmt<FMT, 2>(x, w, y, M, N, K, stream);
    if (M <= kGemvRowsMax) return launch_fmt<FMT, 4>(x, w, y, M, N, K, stream);
    return hipErrorInvalidValue;
}

}  // namespace

// Gated FFN front half: a thread's two rows are one gate row and one up
// row; from P = 32 on, workgroups share one activation copy (timing sweeps
// as above). From N = 4096, rows of more than 32 pairs loop over K in
// chunks of 32 pairs in 256-thread workgroups (against T = 64 in 512
// threads: N = 28672, K = 8192 59.8 -> 50.9 us at M = 1, 108.0 -> 90.9 at
// M = 4; N = 13824, K = 5120 29.0 -> 20.5 and 53.2 -> 38.0 us; against
// T = 128: N = 4096, K = 14336 19.2 -> 16.0 and 41.9 -> 30.2 us); below
// N = 4096, T = 128 stays faster (N = 2048, K = 8192: 6.5 against 8.2 us).
// Several activation rows (MR = 2 or 4; M = 3 runs four and stores three)
// take the same launch shapes, so each row equals the one-row result bit
// for bit.
template <int MR>
hipError_t launch_gated_rows(const float *x, const uint8_t *w_gate, const uint8_t *w_up,
                             float *h, int M, int N, int P, hipStream_t stream)
{
    if (P <= 4) return launch_gated<4, kThreads, false, MR>(x, w_gate, w_up, h, M, N, P, stream);
    if (P <= 8) return launch_gated<8, kThreads, false, MR>(x, w_gate, w_up, h, M, N, P, stream);
    if (P <= 16)
        return launch_gated<16, kThreads, false, MR>(x, w_gate, w_up, h, M, N, P, stream);
    if (P <= 32 || N >= 4096)
        return launch_gated<32, 256, true, MR>(x, w_gate, w_up, h, M, N, P, stream);
    if (P <= 64) return launch_gated<64, 512, true, MR>(x, w_gate, w_up, h, M, N, P, stream);
    return launch_gated<128, 512, true, MR>(x, w_gate, w_up, h, M, N, P, stream);
}

hipError_t launch_ffn_gate_up(const float *x, const uint8_t *w_gate, const uint8_t *w_up,
                              float *h, int M, int N, int K, hipStream_t stream)
{
    const int P = K / 64;
    if (M == 1) return launch_gated_rows<1>(x, w_gate, w_up, h, M, N, P, stream);
    if (M == 2) return launch_gated_rows<2>(x, w_gate, w_up, h, M, N, P, stream);
    if (M <= kGemvRowsMax) return launch_gated_rows<4>(x, w_gate, w_up, h, M, N, P, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_m1(int fmt, const float *x, const uint8_t *w, float *y, int M,
                          int N, int K, hipStream_t stream)
{
    return fmt == FMT_Q4_0 ? launch_rows<FMT_Q4_0>(x, w, y, M, N, K, stream)
                           : launch_rows<FMT_Q8_0>(x, w, y, M, N, K, stream);
}

}  // namespace qmm
