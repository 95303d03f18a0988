// Decode GEMV over Q4_K super-blocks, 1 to 4 activation rows:
// y[m][n] = sum_k x[m][k] * w[n][k], f32 arithmetic.
//
// Q4_K is the k-quant 4-bit format the pages keep for their CLIP/CLAP path
// (named without a layout; GGUF's is read here). A super-block of 256
// weights takes 144 bytes: fp16 d and dmin (bytes 0-3), eight 6-bit
// sub-block scales sc[j] and minimums mn[j] packed in bytes 4-15, and 128
// nibble bytes. Weight 64c + i (c < 4, i < 32) is the low nibble of nibble
// byte 32c + i and weight 64c + 32 + i its high nibble; weight e belongs to
// sub-block e / 32 and is w = d sc q - dmin mn. For a sub-block j < 4, sc is
// the low 6 bits of scale byte j and mn of byte 4 + j; for j >= 4, byte
// 8 + (j - 4) holds the low 4 bits of sc (low nibble) and mn (high nibble)
// and the top 2 bits of bytes j - 4 and j hold their top 2 bits.
//
// A row of K weights is K / 64 "chunks" of 64 weights (a quarter of a
// super-block: sub-blocks 2c and 2c + 1). A thread owns one chunk of one
// row per pass; T threads cover a row, a workgroup WG / T rows. A thread
// loads the super-block's 16-byte header and the chunk's 32 nibble bytes
// (three aligned 16-byte loads), and the activations of a pass are staged
// once per workgroup in LDS (coalesced 16-byte loads, one barrier that
// waits for LDS only, so each wave reads its activations while its weights
// arrive). Per weight: one conversion of the nibble, one FMA forming
// w = d sc q - dmin mn (d sc and dmin mn are exact in f32, so w is rounded
// once), one FMA into the sub-block's sum. The T threads of a row reduce
// with DPP row operations (and through LDS when a row spans two waves) in a
// fixed order.
//
// With MR activation rows (2 or 4; M = 3 runs four, the fourth repeating
// the third and not stored) each weight is formed once and applied to every
// row, and each row's operations run in the one-row order, so a row of the
// result equals the one-row result bit for bit when both use the same T.
#include "qmm_internal.h"

namespace qmm {
namespace {

constexpr int kQKBytes = 144;       // bytes per super-block of 256 weights
constexpr int XS = 68;              // padded LDS row of one chunk's activations

// Scale and minimum of sub-block 2c + h from the scale bytes held in the
// header's dwords 1-3 (b0: bytes 0-3, b1: bytes 4-7, b2: bytes 8-11). The
// byte index inside b0, b1 and b2 is 2 (c % 2) + h in both halves of the
// sub-block range.
__device__ __forceinline__ void sub_block(uint32_t b0, uint32_t b1, uint32_t b2, int c, int h,
                                          uint32_t &sc, uint32_t &mn)
{
    const int sh = 8 * (2 * (c & 1) + h);
    const uint32_t x0 = (b0 >> sh) & 0xFFu, x1 = (b1 >> sh) & 0xFFu, x2 = (b2 >> sh) & 0xFFu;
    if (c < 2) {
        sc = x0 & 63u;
        mn = x1 & 63u;
    } else {
        sc = (x2 & 15u) | ((x0 >> 6) << 4);
        mn = (x2 >> 4) | ((x1 >> 6) << 4);
    }
}

template <int T, int WG, int MR>
__global__ __launch_bounds__(WG) void gemv_q4_k_kernel(const float *__restrict__ x,
                                                       const uint8_t *__restrict__ w,
                                                       float *__restrict__ y, int M, int N,
                                                       int C)
{
    constexpr int RPAR = WG / T;                // rows per workgroup
    constexpr int TW = T < 64 ? T : 64;         // chunks per wave per row
    constexpr int WPR = T / TW;                 // waves per row
    constexpr int XU = (16 * T + WG - 1) / WG;  // staged float4 per thread, row and pass
    static_assert(MR == 1 || WPR == 1, "several activation rows: a weight row within a wave");
    __shared__ __attribute__((aligned(16))) float xs[MR * T * XS];
    __shared__ float red[WPR > 1 ? WG / 64 : 1];

    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int t = tid % T, r = tid / T;
    const int n = blockIdx.x * RPAR + r;
    const int64_t row_bytes = (int64_t)(C / 4) * kQKBytes;
    const uint8_t *wrow = w + (int64_t)min(n, N - 1) * row_bytes;

    float acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = 0.f;
    for (int c0 = 0; c0 < C; c0 += T) {
        // 1. this pass's activations: float4 i of a row is chunk i / 16,
        //    part i % 16 (four scalar arrays: an array of float4 is kept in
        //    scratch)
        float xvx[MR * XU], xvy[MR * XU], xvz[MR * XU], xvw[MR * XU];
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const float *xr = x + (int64_t)min(r, M - 1) * (64 * (int64_t)C);
#pragma unroll
            for (int u = 0; u < XU; ++u) {
                const int i = tid + WG * u;
                const int ch = min(c0 + min(i / 16, T - 1), C - 1);
                const float4 v = *reinterpret_cast<const float4 *>(xr + 64 * ch + 4 * (i % 16));
                xvx[r * XU + u] = v.x; xvy[r * XU + u] = v.y;
                xvz[r * XU + u] = v.z; xvw[r * XU + u] = v.w;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // 2. the super-block header and the chunk's nibbles
        const int ch = min(c0 + t, C - 1);
        const uint8_t *sb = wrow + (int64_t)(ch / 4) * kQKBytes;
        const int c = ch % 4;
        const u32x4_a4 hdr = *reinterpret_cast<const u32x4_a4 *>(sb);
        const u32x4_a4 q0 = *reinterpret_cast<const u32x4_a4 *>(sb + 16 + 32 * c);
        const u32x4_a4 q1 = *reinterpret_cast<const u32x4_a4 *>(sb + 32 + 32 * c);
        __builtin_amdgcn_sched_barrier(0);
        // 3. activations to LDS (from the second pass on, after the
        //    previous pass's readers)
        if (c0 != 0) __syncthreads();
#pragma unroll
        for (int r = 0; r < MR; ++r) {
#pragma unroll
            for (int u = 0; u < XU; ++u) {
                const int i = tid + WG * u;
                if (16 * T % WG == 0 || i < 16 * T)
                    *reinterpret_cast<float4 *>(&xs[(r * T + i / 16) * XS + 4 * (i % 16)]) =
                        make_float4(xvx[r * XU + u], xvy[r * XU + u], xvz[r * XU + u],
                                    xvw[r * XU + u]);
            }
        }
        lds_only_barrier();
        // 4. the chunk's 64 weights against its activations
        const float d = half_lo(hdr.x), dmin = half_hi(hdr.x);
        const uint32_t nb[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        float part[MR];
#pragma unroll
        for (int r = 0; r < MR; ++r) part[r] = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t sc, mn;
            sub_block(hdr.y, hdr.z, hdr.w, c, h, sc, mn);
            const float dsc = d * (float)sc, dmn = dmin * (float)mn;
            float s[MR];
#pragma unroll
            for (int r = 0; r < MR; ++r) s[r] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t v = h ? (nb[i] >> 4) & 0x0F0F0F0Fu : nb[i] & 0x0F0F0F0Fu;
                // hide the nibble range from the compiler, which would
                // otherwise extract each nibble with a bit-field op before
                // converting it; this way each byte converts in one
                // v_cvt_f32_ubyteN
                asm("" : "+v"(v));
                const float w0 = fmaf(dsc, (float)(v & 0xFFu), -dmn);
                const float w1 = fmaf(dsc, (float)((v >> 8) & 0xFFu), -dmn);
                const float w2 = fmaf(dsc, (float)((v >> 16) & 0xFFu), -dmn);
                const float w3 = fmaf(dsc, (float)(v >> 24), -dmn);
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    const float4 xa = *reinterpret_cast<const float4 *>(
                        &xs[(r * T + t) * XS + 32 * h + 4 * i]);
                    s[r] = fmaf(w0, xa.x, s[r]);
                    s[r] = fmaf(w1, xa.y, s[r]);
                    s[r] = fmaf(w2, xa.z, s[r]);
                    s[r] = fmaf(w3, xa.w, s[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < MR; ++r) part[r] += s[r];
        }
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[r] += c0 + t < C ? part[r] : 0.f;
    }

#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = group_sum<TW>(acc[r]);
    if constexpr (WPR == 1) {
        if (t == T - 1 && n < N) {
#pragma unroll
            for (int r = 0; r < MR; ++r)
                if (r < M) y[(int64_t)r * N + n] = acc[r];
        }
    } else {
        if (lane == 63) red[wave] = acc[0];
        __syncthreads();
        if (tid < RPAR) {
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < WPR; ++q) s += red[tid * WPR + q];
            const int nn = blockIdx.x * RPAR + tid;
            if (nn < N) y[nn] = s;
        }
    }
}

// The same with two weight rows per thread (rows n0 and n0 + WG / T of the
// workgroup's block), each staged activation float4 read once for both;
// every row keeps the one-row order of operations. A separate kernel, so
// that the one-row-per-thread instances keep their own schedule (folded
// into one template, they were compiled to read LDS one float4 at a time).
template <int T, int WG, int MR>
__global__ __launch_bounds__(WG) void gemv_q4_k_pair_kernel(const float *__restrict__ x,
                                                            const uint8_t *__restrict__ w,
                                                            float *__restrict__ y, int M,
                                                            int N, int C)
{
    constexpr int RPT = 2;                      // weight rows per thread
    constexpr int RPAR = WG / T;                // rows in flight per workgroup
    constexpr int TW = T < 64 ? T : 64;         // chunks per wave per row
    constexpr int WPR = T / TW;                 // waves per row
    constexpr int XU = (16 * T + WG - 1) / WG;  // staged float4 per thread, row and pass
    static_assert(MR == 1 || WPR == 1, "several activation rows: a weight row within a wave");
    static_assert(WPR == 1, "several weight rows per thread: a row within a wave");
    __shared__ __attribute__((aligned(16))) float xs[MR * T * XS];

    const int tid = threadIdx.x;
    const int t = tid % T, r = tid / T;
    // this thread's weight rows: n0 + RPAR j (j < RPT)
    const int n0 = blockIdx.x * (RPAR * RPT) + r;
    const int64_t row_bytes = (int64_t)(C / 4) * kQKBytes;
    const uint8_t *wrow[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) wrow[j] = w + (int64_t)min(n0 + RPAR * j, N - 1) * row_bytes;

    float acc[RPT][MR];
#pragma unroll
    for (int j = 0; j < RPT; ++j)
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[j][r] = 0.f;
    for (int c0 = 0; c0 < C; c0 += T) {
        // 1. this pass's activations: float4 i of a row is chunk i / 16,
        //    part i % 16 (four scalar arrays: an array of float4 is kept in
        //    scratch)
        float xvx[MR * XU], xvy[MR * XU], xvz[MR * XU], xvw[MR * XU];
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const float *xr = x + (int64_t)min(r, M - 1) * (64 * (int64_t)C);
#pragma unroll
            for (int u = 0; u < XU; ++u) {
                const int i = tid + WG * u;
                const int ch = min(c0 + min(i / 16, T - 1), C - 1);
                const float4 v = *reinterpret_cast<const float4 *>(xr + 64 * ch + 4 * (i % 16));
                xvx[r * XU + u] = v.x; xvy[r * XU + u] = v.y;
                xvz[r * XU + u] = v.z; xvw[r * XU + u] = v.w;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // 2. each row's super-block header and the chunk's nibbles
        const int ch = min(c0 + t, C - 1);
        const int c = ch % 4;
        u32x4_a4 hdr[RPT], q0[RPT], q1[RPT];
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const uint8_t *sb = wrow[j] + (int64_t)(ch / 4) * kQKBytes;
            hdr[j] = *reinterpret_cast<const u32x4_a4 *>(sb);
            q0[j] = *reinterpret_cast<const u32x4_a4 *>(sb + 16 + 32 * c);
            q1[j] = *reinterpret_cast<const u32x4_a4 *>(sb + 32 + 32 * c);
        }
        __builtin_amdgcn_sched_barrier(0);
        // 3. activations to LDS (from the second pass on, after the
        //    previous pass's readers)
        if (c0 != 0) __syncthreads();
#pragma unroll
        for (int r = 0; r < MR; ++r) {
#pragma unroll
            for (int u = 0; u < XU; ++u) {
                const int i = tid + WG * u;
                if (16 * T % WG == 0 || i < 16 * T)
                    *reinterpret_cast<float4 *>(&xs[(r * T + i / 16) * XS + 4 * (i % 16)]) =
                        make_float4(xvx[r * XU + u], xvy[r * XU + u], xvz[r * XU + u],
                                    xvw[r * XU + u]);
            }
        }
        lds_only_barrier();
        // 4. the chunk's 64 weights of each row against its activations;
        //    every activation float4 is read once for the thread's rows
        float d[RPT], dmin[RPT];
        uint32_t nb[RPT][8];
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            d[j] = half_lo(hdr[j].x);
            dmin[j] = half_hi(hdr[j].x);
            nb[j][0] = q0[j].x; nb[j][1] = q0[j].y; nb[j][2] = q0[j].z; nb[j][3] = q0[j].w;
            nb[j][4] = q1[j].x; nb[j][5] = q1[j].y; nb[j][6] = q1[j].z; nb[j][7] = q1[j].w;
        }
        float part[RPT][MR];
#pragma unroll
        for (int j = 0; j < RPT; ++j)
#pragma unroll
            for (int r = 0; r < MR; ++r) part[j][r] = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float dsc[RPT], dmn[RPT];
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                uint32_t sc, mn;
                sub_block(hdr[j].y, hdr[j].z, hdr[j].w, c, h, sc, mn);
                dsc[j] = d[j] * (float)sc;
                dmn[j] = dmin[j] * (float)mn;
            }
            float s[RPT][MR];
#pragma unroll
            for (int j = 0; j < RPT; ++j)
#pragma unroll
                for (int r = 0; r < MR; ++r) s[j][r] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float wv[RPT][4];
#pragma unroll
                for (int j = 0; j < RPT; ++j) {
                    uint32_t v = h ? (nb[j][i] >> 4) & 0x0F0F0F0Fu : nb[j][i] & 0x0F0F0F0Fu;
                    // hide the nibble range from the compiler, which would
                    // otherwise extract each nibble with a bit-field op
                    // before converting it; this way each byte converts in
                    // one v_cvt_f32_ubyteN
                    asm("" : "+v"(v));
                    wv[j][0] = fmaf(dsc[j], (float)(v & 0xFFu), -dmn[j]);
                    wv[j][1] = fmaf(dsc[j], (float)((v >> 8) & 0xFFu), -dmn[j]);
                    wv[j][2] = fmaf(dsc[j], (float)((v >> 16) & 0xFFu), -dmn[j]);
                    wv[j][3] = fmaf(dsc[j], (float)(v >> 24), -dmn[j]);
                }
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    const float4 xa = *reinterpret_cast<const float4 *>(
                        &xs[(r * T + t) * XS + 32 * h + 4 * i]);
#pragma unroll
                    for (int j = 0; j < RPT; ++j) {
                        s[j][r] = fmaf(wv[j][0], xa.x, s[j][r]);
                        s[j][r] = fmaf(wv[j][1], xa.y, s[j][r]);
                        s[j][r] = fmaf(wv[j][2], xa.z, s[j][r]);
                        s[j][r] = fmaf(wv[j][3], xa.w, s[j][r]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < RPT; ++j)
#pragma unroll
                for (int r = 0; r < MR; ++r) part[j][r] += s[j][r];
        }
#pragma unroll
        for (int j = 0; j < RPT; ++j)
#pragma unroll
            for (int r = 0; r < MR; ++r) acc[j][r] += c0 + t < C ? part[j][r] : 0.f;
    }

#pragma unroll
    for (int j = 0; j < RPT; ++j)
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[j][r] = group_sum<TW>(acc[j][r]);
    if (t == T - 1) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int n = n0 + RPAR * j;
            if (n < N) {
#pragma unroll
                for (int r = 0; r < MR; ++r)
                    if (r < M) y[(int64_t)r * N + n] = acc[j][r];
            }
        }
    }
}

template <int T, int WG, int MR, int RPT = 1>
hipError_t launch(const float *x, const uint8_t *w, float *y, int M, int N, int C,
                  hipStream_t stream)
{
    static_assert(RPT == 1 || RPT == 2, "one or two weight rows per thread");
    constexpr int rows = WG / T * RPT;
    if constexpr (RPT == 1)
        hipLaunchKernelGGL((gemv_q4_k_kernel<T, WG, MR>), dim3((N + rows - 1) / rows), dim3(WG),
                           0, stream, x, w, y, M, N, C);
    else
        hipLaunchKernelGGL((gemv_q4_k_pair_kernel<T, WG, MR>), dim3((N + rows - 1) / rows),
                           dim3(WG), 0, stream, x, w, y, M, N, C);
    return hipGetLastError();
}

// Several activation rows: T up to 64 (rows longer than 64 chunks take
// several passes), so that a weight row stays within one wave and the
// staged rows fit twice per compute unit's LDS. From timing sweeps on random
// weights over matrix shapes from N = 2048 to 65536 and K = 2048 to 28672:
//  * two rows past 32 chunks above N = 4096 loop over T = 32 in 256 threads
//    (N = 13824, K = 5120: 25.2 -> 19.0 us; N = 28672, K = 8192: 51.6 ->
//    45.4 us; at N = 4096, T = 64 in 512 threads stays faster);
//  * four rows take two weight rows per thread (the pair kernel: each
//    staged activation float4 read once for both, since at four rows those
//    LDS reads set the pace) with T = 16 and 512 threads above N = 8192
//    where a row has 17-128 chunks (N = 14336, K = 4096: 26.8 -> 16.1 us;
//    N = 13824, K = 5120: 43.5 -> 19.3 us; N = 28672, K = 8192: 89.5 ->
//    57.6 us; N = 16384, K = 2048: 11.4 -> 9.9 us; N = 11008, K = 2048:
//    11.2 -> 9.4 us), else past 32 chunks T = 32 in 256 threads above N = 4096 (N =
//    8192, K = 8192: 27.3 -> 18.5 us; K = 28672: 81.1 -> 59.2 us; N = 6144,
//    K = 4096: 12.6 -> 10.1 us) and T = 64 in 512 threads at N = 4096
//    (exactly one 16-row workgroup per compute unit: K = 4096 8.9 -> 7.3 us;
//    K = 14336 25.5 -> 19.1 us); 17-32 chunks at N = 8192-12287 keep one
//    row per thread with T = 16 (FFN up shape 8.4 -> 6.7 us against T = 32).
// Rows of a multi-row call round differently from a one-row call wherever
// the two take different T.
template <int MR>
hipError_t launch_rows(const float *x, const uint8_t *w, float *y, int M, int N, int C,
                       hipStream_t stream)
{
    if constexpr (MR == 4) {
        if (N > 8192 && C > 16 && C <= 128)
            return launch<16, 512, MR, 2>(x, w, y, M, N, C, stream);
        if (N >= 8192 && C > 16 && C <= 32) return launch<16, 512, MR>(x, w, y, M, N, C, stream);
        if (N > 4096 && C > 32) return launch<32, 256, MR, 2>(x, w, y, M, N, C, stream);
        if (N == 4096 && C > 32) return launch<64, 512, MR, 2>(x, w, y, M, N, C, stream);
    } else {
        if (N > 4096 && C > 32) return launch<32, 256, MR>(x, w, y, M, N, C, stream);
    }
    if (C <= 4) return launch<4, 256, MR>(x, w, y, M, N, C, stream);
    if (C <= 8) return launch<8, 256, MR>(x, w, y, M, N, C, stream);
    if (C <= 16) return launch<16, 256, MR>(x, w, y, M, N, C, stream);
    if (C <= 32) return launch<32, 256, MR>(x, w, y, M, N, C, stream);
    return launch<64, 512, MR>(x, w, y, M, N, C, stream);
}

}  // namespace

// C = K / 64 chunks per row (a multiple of 4). With one activation row, T
// is the smallest of 4, 8, 16, 32, 64 and 128 that covers a row in one pass
// (rows longer than 128 chunks take several passes), except that from
// N = 4096 rows of more than 64 chunks loop over T = 32 in 256 threads
// (N = 13824, K = 5120: 17.4 -> 14.7 us; N = 8192, K = 28672: 40.7 -> 36.9
// us; at the FFN down shape, N = 2048, T = 128 stays faster); otherwise the
// shapes of the Q4_0 GEMV, whose chunks (pairs of blocks) hold as many
// weights and bytes. Two to four rows: launch_rows.
hipError_t launch_gemv_q4_k(const float *x, const uint8_t *w, float *y, int M, int N, int K,
                            hipStream_t stream)
{
    const int C = K / 64;
    if (M == 2) return launch_rows<2>(x, w, y, M, N, C, stream);
    if (M > 2) return launch_rows<4>(x, w, y, M, N, C, stream);
    if (C <= 4) return launch<4, 256, 1>(x, w, y, M, N, C, stream);
    if (C <= 8) return launch<8, 256, 1>(x, w, y, M, N, C, stream);
    if (C <= 16) return launch<16, 256, 1>(x, w, y, M, N, C, stream);
    if (C <= 32) return launch<32, 256, 1>(x, w, y, M, N, C, stream);
    if (C <= 64) return launch<64, 512, 1>(x, w, y, M, N, C, stream);
    if (N >= 4096) return launch<32, 256, 1>(x, w, y, M, N, C, stream);
    return launch<128, 512, 1>(x, w, y, M, N, C, stream);
}

}  // namespace qmm
