// Matrix-core kernels over GGUF Q4_0 / Q8_0 weights: the prefill GEMM's
// tile kernel (described here), the medium-M GEMM (5-128 rows, and few-tile shapes above) and the
// weight-slice GEMV to the f32 bound (9-16 rows), each introduced where it starts.
//
// Prefill GEMM over GGUF Q4_0 or Q8_0 weights on the bf16 matrix cores:
// y[m][n] = sum_k bf16(x[m][k]) * bf16(w[n][k]) with f32 accumulation, where
// w = d * (q - 8) (Q4_0) or d * q (Q8_0) is exact in f32 before its one
// rounding to bf16.
//
// Workgroup tile BM x BN = 256 x 256, K step 64 (one pair of Q4_0 blocks per
// weight row), 8 waves each owning a 128 x 64 sub-tile as 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 (f32 accumulators, 128 per lane).
//
// Per K step every thread
//  * converts 32 activations (a float4 in each of 8 rows) from f32 to bf16
//    (round to nearest even, v_cvt_pk_bf16_f32) on their way into LDS, and
//  * dequantizes one block of one weight row: d * (q - 8) (Q4_0) or d * q
//    (Q8_0) is exact in f32 and is rounded once to bf16 (nearest even) into
//    LDS.
// LDS is double buffered. During step s the registers hold step s+1, which
// is converted into the other buffer a quarter per 16-wide substep (a
// quarter of the activations and a quarter of the weight block each),
// interleaved with that substep's matrix-core instructions. Each activation
// quarter is reloaded with step s+2 as soon as it is written; the weight
// window is double buffered in registers and loads step s+2 at the top of
// step s. So every global load has most of a K step to land. LDS fragments
// are prefetched one substep ahead. One barrier per step.
//
// Global traffic goes through buffer resources based at the tile's first
// row, with the whole byte offset in the lane's offset register (the part
// the hardware range-checks): rows past M or N fall outside the resource,
// so they load zeros and their stores are dropped. 32-bit offsets replace
// the 64-bit pointers a thread would otherwise keep per activation row.
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the
// eight XCDs, and consecutive tiles in band-major order (one 256-row band
// of x with all its column tiles) are given to the same XCD, so each XCD's
// L2 holds the activation band its compute units share.
#include "qmm_internal.h"

#include <type_traits>

namespace qmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;                            // padded LDS row (bf16)
constexpr int kXcds = 8;
// word 3 of a raw (stride 0) buffer resource on gfx9: 32-bit data format
constexpr int kBufferWord3 = 0x00020000;

// Workgroup shapes: the 256 x 256 tile with 8 waves of 128 x 64, and a
// 128 x 128 tile with 4 waves of 64 x 64 for problems with fewer 256 x 256
// tiles than compute units (then the smaller tiles fill more of the chip).
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_> struct Tile {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // per wave
    static constexpr int TM = WTM / 32, TN = WTN / 32;            // MFMA tiles per wave
    static constexpr int A_F4 = BM * BK / 4 / kThreads;           // float4 per thread
    static constexpr int A_ROW_STRIDE = kThreads / 16;            // rows between them
    static_assert(BN * 2 == kThreads, "one weight block per thread per K step");
    static_assert(A_F4 == 8, "activation float4s split into four quarters of two");
};
using TileLarge = Tile<256, 256, 2, 4>;
using TileSmall = Tile<128, 128, 2, 2>;

// f rounded to bf16 (nearest even), back in f32
__device__ __forceinline__ float bf16_round(float f)
{
    return (float)(__bf16)f;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Weight staging per format. A thread owns block blk (0 or 1) of one pair
// of a weight row per K step and loads the dword-aligned window of the pair
// that holds it: the block's scale is the low (blk 0) or high (blk 1) half
// of the window's first dword, and its codes start 2 bytes (blk 0) or 4
// bytes (blk 1) into the window.
template <int FMT> struct BFmt;

template <> struct BFmt<FMT_Q4_0> {
    static constexpr int kPairBytes = 36;
    static constexpr int kWin = 5;          // window dwords at pair byte 16 blk
    static constexpr int kWinStride = 16;

    // the window of block blk of K step p, for a weight row at byte row_off
    __device__ static void load_step(__amdgpu_buffer_rsrc_t r, int row_off, int blk, int p,
                                     uint32_t (&b)[kWin])
    {
        load(r, row_off + kWinStride * blk, p * kPairBytes, b);
    }

    __device__ static void load(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                uint32_t (&b)[kWin])
    {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
        b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
        b[4] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 16, soff, 0);
    }

    // Quarter q of the block: the low (q = 0, 1) or high (q = 2, 3) nibbles
    // of qs dwords 2h, 2h+1 with h = q % 2, i.e. elements 16 (q / 2) + 8h ..
    // +7 -> bf16(d * (q - 8)), one 16-byte LDS store at dst.
    __device__ static void convert_quarter(const uint32_t (&b)[kWin], int blk, int q,
                                           __bf16 *dst)
    {
        const float dq = half_lo(b[0] >> (16 * blk)) * (1.0f / 16.0f);
        const int h = q % 2, nib = q / 2;
        uint4 v;
        uint32_t *o = &v.x;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int i = 2 * h + t;
            const uint32_t realigned = __builtin_amdgcn_alignbyte(b[i + 1], b[i], 2);
            const uint32_t qs = blk ? b[i + 1] : realigned;
            const uint32_t s = nib ? hi16(qs) : lo16(qs);
            o[2 * t] = pack_bf16x2(sbyte(s, 0) * dq, sbyte(s, 1) * dq);
            o[2 * t + 1] = pack_bf16x2(sbyte(s, 2) * dq, sbyte(s, 3) * dq);
        }
        *reinterpret_cast<uint4 *>(dst + 16 * nib + 8 * h) = v;
    }

    // The same quarter as integer codes 16 (q - 8), exact in bf16, for
    // products kept exact; the block's scale is applied afterwards.
    static constexpr float kCodeScale = 1.0f / 16.0f;
    __device__ static void codes_quarter(const uint32_t (&b)[kWin], int blk, int q, __bf16 *dst)
    {
        const int h = q % 2, nib = q / 2;
        uint4 v;
        uint32_t *o = &v.x;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int i = 2 * h + t;
            const uint32_t realigned = __builtin_amdgcn_alignbyte(b[i + 1], b[i], 2);
            const uint32_t qs = blk ? b[i + 1] : realigned;
            const uint32_t s = nib ? hi16(qs) : lo16(qs);
            o[2 * t] = pack_bf16x2(sbyte(s, 0), sbyte(s, 1));
            o[2 * t + 1] = pack_bf16x2(sbyte(s, 2), sbyte(s, 3));
        }
        *reinterpret_cast<uint4 *>(dst + 16 * nib + 8 * h) = v;
    }
    __device__ static float scale(const uint32_t (&b)[kWin], int blk)
    {
        return half_lo(b[0] >> (16 * blk));
    }
    static constexpr bool kHasMin = false;
};

template <> struct BFmt<FMT_Q8_0> {
    static constexpr int kPairBytes = 68;
    static constexpr int kWin = 9;          // window dwords at pair byte 32 blk
    static constexpr int kWinStride = 32;

    __device__ static void load_step(__amdgpu_buffer_rsrc_t r, int row_off, int blk, int p,
                                     uint32_t (&b)[kWin])
    {
        load(r, row_off + kWinStride * blk, p * kPairBytes, b);
    }

    __device__ static void load(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                uint32_t (&b)[kWin])
    {
        const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
        const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, 0);
        b[0] = v0.x; b[1] = v0.y; b[2] = v0.z; b[3] = v0.w;
        b[4] = v1.x; b[5] = v1.y; b[6] = v1.z; b[7] = v1.w;
        b[8] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 32, soff, 0);
    }

    // Quarter h of the block (q dwords 2h, 2h+1: elements 8h..8h+7, element
    // j is byte j) -> bf16(d * q), one 16-byte LDS store at dst.
    __device__ static void convert_quarter(const uint32_t (&b)[kWin], int blk, int h,
                                           __bf16 *dst)
    {
        const float d = half_lo(b[0] >> (16 * blk));
        uint4 v;
        uint32_t *o = &v.x;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int i = 2 * h + t;
            const uint32_t realigned = __builtin_amdgcn_alignbyte(b[i + 1], b[i], 2);
            const uint32_t q = blk ? b[i + 1] : realigned;
            o[2 * t] = pack_bf16x2(sbyte(q, 0) * d, sbyte(q, 1) * d);
            o[2 * t + 1] = pack_bf16x2(sbyte(q, 2) * d, sbyte(q, 3) * d);
        }
        *reinterpret_cast<uint4 *>(dst + 8 * h) = v;
    }

    // the quarter as integer codes q, exact in bf16
    static constexpr float kCodeScale = 1.0f;
    __device__ static void codes_quarter(const uint32_t (&b)[kWin], int blk, int h, __bf16 *dst)
    {
        uint4 v;
        uint32_t *o = &v.x;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int i = 2 * h + t;
            const uint32_t realigned = __builtin_amdgcn_alignbyte(b[i + 1], b[i], 2);
            const uint32_t q = blk ? b[i + 1] : realigned;
            o[2 * t] = pack_bf16x2(sbyte(q, 0), sbyte(q, 1));
            o[2 * t + 1] = pack_bf16x2(sbyte(q, 2), sbyte(q, 3));
        }
        *reinterpret_cast<uint4 *>(dst + 8 * h) = v;
    }
    __device__ static float scale(const uint32_t (&b)[kWin], int blk)
    {
        return half_lo(b[0] >> (16 * blk));
    }
    static constexpr bool kHasMin = false;
};

// Q4_K super-blocks (256 weights in 144 bytes: fp16 d and dmin, 6-bit
// sub-block scales and minimums, 128 nibble bytes; see gemv_q4_k.hip). A K
// step of 64 is a quarter c of a super-block: sub-block 2c takes the low
// nibbles of its 32 nibble bytes, sub-block 2c + 1 the high nibbles. The
// thread with blk holds the super-block's 16-byte header and nibble bytes
// 16 blk .. 16 blk + 15 of the quarter, i.e. elements 16 blk .. +15 of both
// sub-blocks; b[8] keeps c. Each weight is formed in f32 with one FMA,
// d sc q - dmin mn (both products exact), and rounded to bf16 (nearest even).
template <> struct BFmt<FMT_Q4_K> {
    static constexpr int kPairBytes = 36;   // per K step, on average (144 per 4 steps)
    static constexpr int kWin = 11;         // + d sc and dmin mn of the current sub-block

    __device__ static void load_step(__amdgpu_buffer_rsrc_t r, int row_off, int blk, int p,
                                     uint32_t (&b)[kWin])
    {
        const int sb = (p / 4) * 144, c = p % 4;
        const u32x4 h = __builtin_amdgcn_raw_buffer_load_b128(r, row_off, sb, 0);
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(r, row_off + 16 * blk,
                                                              sb + 16 + 32 * c, 0);
        b[0] = h.x; b[1] = h.y; b[2] = h.z; b[3] = h.w;
        b[4] = q.x; b[5] = q.y; b[6] = q.z; b[7] = q.w;
        b[8] = c;
    }

    // quarter q: sub-block 2c + q / 2 (low or high nibbles), nibble bytes
    // 16 blk + 8 (q % 2) .. +7 -> elements 32 (q / 2) + 16 blk + 8 (q % 2) ..
    // +7 of the K step; dst is the row's base plus 32 blk (as for the block
    // formats), one 16-byte LDS store. Callers convert a window's quarters in
    // order 0..3: the even quarter unpacks its sub-block's scale and minimum
    // into b[9], b[10] and the odd one reuses them.
    // d sc and dmin mn of sub-block 2c + h of the window's quarter c (both
    // products exact in f32)
    __device__ static void sub_scales(const uint32_t (&b)[kWin], int h, float &dsc, float &dmn)
    {
        // c is the same across the wave; hidden from the compiler, the
        // choices below stay per-lane selects instead of becoming
        // branches that would split the K step into many basic blocks
        int c = (int)b[8];
        asm("" : "+v"(c));
        const int sh = 8 * (2 * (c & 1) + h);
        const uint32_t x0 = (b[1] >> sh) & 0xFFu, x1 = (b[2] >> sh) & 0xFFu;
        const uint32_t x2 = (b[3] >> sh) & 0xFFu;
        const uint32_t sc = c < 2 ? (x0 & 63u) : ((x2 & 15u) | ((x0 >> 6) << 4));
        const uint32_t mn = c < 2 ? (x1 & 63u) : ((x2 >> 4) | ((x1 >> 6) << 4));
        dsc = half_lo(b[0]) * (float)sc;
        dmn = half_hi(b[0]) * (float)mn;
    }

    __device__ static void convert_quarter(uint32_t (&b)[kWin], int blk, int q, __bf16 *dst)
    {
        const int h = q / 2, qq = q % 2;
        float dsc, dmn;
        if (qq == 0) {
            sub_scales(b, h, dsc, dmn);
            b[9] = __float_as_uint(dsc);
            b[10] = __float_as_uint(dmn);
        } else {
            dsc = __uint_as_float(b[9]);
            dmn = __uint_as_float(b[10]);
        }
        uint4 v;
        uint32_t *o = &v.x;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t raw = b[4 + 2 * qq + t];
            uint32_t nib = h ? (raw >> 4) & 0x0F0F0F0Fu : raw & 0x0F0F0F0Fu;
            // hidden range: each byte converts in one v_cvt_f32_ubyteN
            // instead of a bit-field extract and a conversion
            asm("" : "+v"(nib));
            o[2 * t] = pack_bf16x2(fmaf(dsc, (float)(nib & 0xFFu), -dmn),
                                   fmaf(dsc, (float)((nib >> 8) & 0xFFu), -dmn));
            o[2 * t + 1] = pack_bf16x2(fmaf(dsc, (float)((nib >> 16) & 0xFFu), -dmn),
                                       fmaf(dsc, (float)(nib >> 24), -dmn));
        }
        *reinterpret_cast<uint4 *>(dst - 32 * blk + 32 * h + 16 * blk + 8 * qq) = v;
    }

    // The same quarter as the nibbles q (0..15, exact in bf16), for products
    // kept exact; the sub-block's d sc and dmin mn are applied afterwards.
    static constexpr float kCodeScale = 1.0f;
    static constexpr bool kHasMin = true;
    __device__ static void codes_quarter(const uint32_t (&b)[kWin], int blk, int q, __bf16 *dst)
    {
        const int h = q / 2, qq = q % 2;
        uint4 v;
        uint32_t *o = &v.x;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t raw = b[4 + 2 * qq + t];
            uint32_t nib = h ? (raw >> 4) & 0x0F0F0F0Fu : raw & 0x0F0F0F0Fu;
            asm("" : "+v"(nib));
            o[2 * t] = pack_bf16x2((float)(nib & 0xFFu), (float)((nib >> 8) & 0xFFu));
            o[2 * t + 1] = pack_bf16x2((float)((nib >> 16) & 0xFFu), (float)(nib >> 24));
        }
        *reinterpret_cast<uint4 *>(dst - 32 * blk + 32 * h + 16 * blk + 8 * qq) = v;
    }
};

template <int FMT, class TL>
__global__ __launch_bounds__(TL::kThreads) void gemm_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ w,
    float *__restrict__ y, int M, int N, int K, int tiles_m, int tiles_n,
    int per_xcd)
{
    constexpr int BM = TL::BM, BN = TL::BN, WAVES_N = TL::WAVES_N;
    constexpr int WTM = TL::WTM, WTN = TL::WTN, TM = TL::TM, TN = TL::TN;
    constexpr int A_F4 = TL::A_F4, A_ROW_STRIDE = TL::A_ROW_STRIDE;
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
    using BF = BFmt<FMT>;
    const int P = K / 64;
    const int row_bytes = P * BF::kPairBytes;

    // Resources over the tile's rows (all sizes fit 32 bits: K <= 65536).
    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(x + (int64_t)m0 * K), 0, a_rows * K * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(w + (int64_t)n0 * row_bytes), 0, b_rows * row_bytes,
        kBufferWord3);

    // A staging: 16 threads per row (one float4 each), rows tid/16 + A_ROW_STRIDE u.
    // The row lives in the lane offset (the part of the address the
    // hardware range-checks, whether or not it includes the uniform
    // offset); the step's column offset goes into the uniform offset and
    // never carries a valid row past its end.
    const int a_col = (tid % 16) * 4;
    int a_voff[A_F4];
#pragma unroll
    for (int u = 0; u < A_F4; ++u) a_voff[u] = ((tid / 16 + A_ROW_STRIDE * u) * K + a_col) * 4;
    // B staging: thread -> (row tid / 2, block tid % 2) of the tile
    const int b_row = tid / 2, b_blk = tid % 2;
    const int b_roff = b_row * row_bytes;

    float4 a_reg[A_F4];
    uint32_t b_reg[2][BF::kWin];    // weight windows of two consecutive steps

    // global -> registers for K step p: activation quarter q (float4s 2q,
    // 2q+1), weight window
    auto load_a = [&](int p, int q) {
#pragma unroll
        for (int u = 2 * q; u < 2 * q + 2; ++u) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_voff[u], p * 256, 0);
            a_reg[u] = __builtin_bit_cast(float4, v);
        }
    };
    auto load_b = [&](uint32_t (&b)[BF::kWin], int p) {
        BF::load_step(b_rsrc, b_roff, b_blk, p, b);
    };

    // Converts quarter q of a step into LDS buffer buf: activation float4s
    // 2q, 2q+1 (f32 -> bf16, RNE) and quarter q of weight block b_blk (->
    // bf16, RNE), so each of the four substeps' matrix-core work hides the
    // same share of the conversion.
    auto convert = [&](int buf, int q, uint32_t (&b)[BF::kWin]) {
#pragma unroll
        for (int u = 2 * q; u < 2 * q + 2; ++u) {
            const float4 v = a_reg[u];
            uint2 pk;
            pk.x = pack_bf16x2(v.x, v.y);
            pk.y = pack_bf16x2(v.z, v.w);
            *reinterpret_cast<uint2 *>(&As[buf][(tid / 16 + A_ROW_STRIDE * u) * LDK + a_col]) = pk;
        }
        BF::convert_quarter(b, b_blk, q, &Bs[buf][b_row * LDK + 32 * b_blk]);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int frow = lane % 32, fk = 8 * (lane / 32);

    // Prologue: step 0 is converted into buffer 0. Step 1's weight window is
    // requested together with step 0, and each of its activation quarters
    // as soon as step 0's quarter has been written, so that step 1 lands
    // while step 0 is converted rather than one memory latency later.
    // Steps past the last one reload (and convert) the last step, into the
    // buffer nobody reads any more: the loop body has no branches, so the
    // waits for the registers' loads stay exact.
#pragma unroll
    for (int q = 0; q < 4; ++q) load_a(0, q);
    load_b(b_reg[0], 0);
    load_b(b_reg[1], min(1, P - 1));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        convert(0, q, b_reg[0]);
        load_a(min(1, P - 1), q);
    }
    __syncthreads();

    // K step p out of LDS buffer PAR = p % 2. On entry the registers hold
    // step p+1 (weights in b_reg[PAR ^ 1]); b_reg[PAR] is free and takes
    // step p+2 at once, and each activation quarter is refilled with step
    // p+2 right after it is converted.
    auto step = [&](int p, auto par) {
        constexpr int PAR = decltype(par)::value;
        const int p2 = min(p + 2, P - 1);
        load_b(b_reg[PAR], p2);
        const __bf16 *as = &As[PAR][(wm * WTM + frow) * LDK + fk];
        const __bf16 *bs = &Bs[PAR][(wn * WTN + frow) * LDK + fk];
        // fragments double-buffered across the four 16-wide substeps
        bf16x8 a[2][TM], b[2][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            a[0][i] = *reinterpret_cast<const bf16x8 *>(as + 32 * i * LDK);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            b[0][j] = *reinterpret_cast<const bf16x8 *>(bs + 32 * j * LDK);
        __builtin_amdgcn_sched_barrier(0);
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
            convert(PAR ^ 1, s, b_reg[PAR ^ 1]);
            load_a(p2, s);
            // interleave: each matrix-core instruction is followed by a few
            // VALU instructions of the conversion and one LDS access
#pragma unroll
            for (int k = 0; k < TM * TN; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // VALU
                __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);   // LDS
            }
            __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);       // VMEM reads
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    };
    // two steps per iteration (the weight registers and the LDS buffers
    // alternate with the step's parity), then an odd last step: it reads
    // buffer 0, written during the step before, and its own conversion goes
    // to buffer 1, which nobody reads any more
    int p = 0;
    for (; p + 1 < P; p += 2) {
        step(p, std::integral_constant<int, 0>());
        step(p + 1, std::integral_constant<int, 1>());
    }
    if (p < P) step(p, std::integral_constant<int, 0>());

    // ---- epilogue: acc[i][j][e] = C[32i + 8(e/4) + 4(lane/32) + e%4][32j + lane%32]
    // Columns past N get bit 31 set in their offset, which puts them outside
    // the resource (its size, BM * N * 4 at most, is below 2^31 by the
    // entry point's bound on N); rows past M lie outside it already. The
    // hardware drops stores outside the resource.
    const __amdgpu_buffer_rsrc_t y_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        y + (int64_t)m0 * N, 0, a_rows * N * 4, kBufferWord3);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * WTN + 32 * j + lane % 32;
            const int r0 = wm * WTM + 32 * i + 4 * (lane / 32);
            const uint32_t outside = n < N ? 0u : 0x80000000u;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = r0 + 8 * (e / 4) + e % 4;
                const float v = acc[i][j][e];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), y_rsrc,
                                                      int(uint32_t((r * N + n) * 4) | outside),
                                                      0, 0);
            }
        }
    }
}

// Medium M: few output tiles, so instead of one tile's K loop per compute
// unit, a workgroup owns a 32 NT-column slice of y for a band of 32 MT rows
// (grid: column slices x row bands) and its WAVES waves take interleaved K
// steps of 64 in parallel (wave w: steps w, w + WAVES, ...), each with its
// own accumulators, meeting in LDS at the end (summed in wave order). Same
// arithmetic as the tile kernel: x and w rounded once to bf16 (RNE), f32
// accumulation.
//
// The waves never share LDS during the K loop: each wave's region holds its
// own step, so the only synchronization inside the loop is the wave's own
// ordering of its LDS writes before its reads (wave_lds_sync).
//
// Per step a wave loads its activation rows (16 lanes per row, a float4
// each) and NT weight blocks per lane (rows lane / 2 + 32 j of the slice,
// block lane % 2 of the pair), converts both into its own LDS region, then
// runs MT x NT 32x32x16 MFMAs per 16-wide substep; the next step's loads are
// issued before this step's matrix-core work. Rows past M and columns past
// N load zeros through the buffer resources' range checks and are not
// stored. Every workgroup reads all of its activation band, so the band is
// re-read once per column slice: wider slices (NT = 2) halve that L2
// traffic where there are enough of them to fill the chip.
template <int FMT, int MT, int NT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemm_mid_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ w, float *__restrict__ y,
    int M, int N, int K)
{
    constexpr int BM = 32 * MT, BN = 32 * NT;
    constexpr int AF4 = BM / 4;                         // activation float4 per lane
    constexpr int REGION = (BM + BN) * LDK;             // bf16 per wave
    static_assert(MT * NT * 1024 * 4 <= REGION * 2, "wave partials fit the wave's region");
    __shared__ __attribute__((aligned(16))) __bf16 lds[WAVES * REGION];

    using BF = BFmt<FMT>;
    // the wave index is the same on every lane; read from one lane, the
    // compiler knows it (and the K steps derived from it) to be uniform, so
    // the buffer loads' scalar offsets need no per-lane loop
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int rows = min(BM, M - m0);
    const int P = K / 64;
    const int row_bytes = P * BF::kPairBytes;
    __bf16 *As = lds + wave * REGION;
    __bf16 *Bs = As + BM * LDK;

    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(x + (int64_t)m0 * K), 0, rows * K * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(w + (int64_t)n0 * row_bytes), 0, min(BN, N - n0) * row_bytes,
        kBufferWord3);
    // activation row lane / 16 + 4 u, columns 4 (lane % 16) .. +3 of the step
    const int a_col = 4 * (lane % 16);
    const int a_voff0 = ((lane / 16) * K + a_col) * 4;
    // weight rows lane / 2 + 32 j of the slice, block lane % 2 of the step's pair
    const int b_row = lane / 2, b_blk = lane % 2;
    const int b_roff = b_row * row_bytes;

    float4 a_reg[AF4];
    uint32_t b_reg[NT][BF::kWin];
    auto load = [&](int p) {
#pragma unroll
        for (int u = 0; u < AF4; ++u) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                a_rsrc, a_voff0 + 16 * K * u, p * 256, 0);
            a_reg[u] = __builtin_bit_cast(float4, v);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
            BF::load_step(b_rsrc, b_roff + 32 * j * row_bytes, b_blk, p, b_reg[j]);
    };

    f32x16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int frow = lane % 32, fk = 8 * (lane / 32);
    // a wave without steps (P < WAVES) loads the last step and never uses it
    load(min(wave, P - 1));
    for (int p = wave; p < P; p += WAVES) {
#pragma unroll
        for (int u = 0; u < AF4; ++u) {
            const float4 v = a_reg[u];
            uint2 pk;
            pk.x = pack_bf16x2(v.x, v.y);
            pk.y = pack_bf16x2(v.z, v.w);
            *reinterpret_cast<uint2 *>(&As[(lane / 16 + 4 * u) * LDK + a_col]) = pk;
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                BF::convert_quarter(b_reg[j], b_blk, q, &Bs[(b_row + 32 * j) * LDK + 32 * b_blk]);
        load(min(p + WAVES, P - 1));            // registers are free again
        wave_lds_sync();
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            bf16x8 b[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j)
                b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[(32 * j + frow) * LDK + fk + 16 * s]);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                    &As[(32 * i + frow) * LDK + fk + 16 * s]);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[j], acc[i][j], 0, 0, 0);
            }
        }
        wave_lds_sync();                        // fragments read before the next writes
    }

    // partials: red[wave][i][j][e][lane] = C[32 i + 8 (e / 4) + 4 (lane / 32) + e % 4][32 j + lane % 32]
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                red[(((wave * MT + i) * NT + j) * 16 + e) * 64 + lane] = acc[i][j][e];
    __syncthreads();
    for (int o = threadIdx.x; o < MT * NT * 16 * 64; o += 64 * WAVES) {
        const int l = o % 64, e = (o / 64) % 16, j = (o / 1024) % NT, i = o / (1024 * NT);
        const int r = 32 * i + 8 * (e / 4) + 4 * (l / 32) + e % 4;
        const int n = n0 + 32 * j + l % 32;
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < WAVES; ++q) s += red[(((q * MT + i) * NT + j) * 16 + e) * 64 + l];
        if (r < rows && n < N) y[(int64_t)(m0 + r) * N + n] = s;
    }
}

template <int FMT, int MT, int NT, int WAVES>
hipError_t launch_mid(const float *x, const uint8_t *w, float *y, int M, int N, int K,
                      hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_mid_kernel<FMT, MT, NT, WAVES>),
                       dim3((N + 32 * NT - 1) / (32 * NT), (M + 32 * MT - 1) / (32 * MT)),
                       dim3(64 * WAVES), 0, stream, x, w, y, M, N, K);
    return hipGetLastError();
}

// Variant to the f32 bound for 5 .. 16 activation rows (the GEMV entry points'
// accuracy): the same slices and interleaved K steps, but the 32 A rows
// hold hi = bf16(x) of the (up to 16) activation rows in rows 0-15 and
// lo = bf16(x - hi) in rows 16-31, the weight operand holds the integer
// codes (exact in bf16), and each block's two MFMAs run into a fresh f32
// tile that is scaled by the block's fp16 d in f32 before it is added to
// the accumulators. The split represents x to within 2^-17 |x| and each
// code-term product is exact; y[m] = (C[m] + C[m + 16]) x the codes' scale.
// Q4_K: a block is a 32-weight sub-block, the codes are its nibbles, the
// scale is d sc, and dmin mn times the sum of the block's activations (two
// more MFMAs of the same A operand against a B operand of ones) is
// subtracted in f32.
// GATED (Q4_0): the gated FFN front half. Weight rows 0-15 of the slice are
// rows n0 .. n0 + 15 of the gate matrix w, rows 16-31 the same rows of the
// up matrix w2, and the output is y[m][n] = gelu_tanh(gate) * up in f32.
// Each lane issues its window loads against both matrices' buffer
// resources, the one it does not own at an offset past the resource's end,
// which the hardware's range check answers with zeros: the loads stay
// branch-free and the two results are merged with an OR. Grid: ceil(N / 16).
template <int FMT, int WAVES, bool GATED = false>
__global__ __launch_bounds__(64 * WAVES) void gemv_slice_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ w, float *__restrict__ y,
    int M, int N, int K, const uint8_t *__restrict__ w2 = nullptr)
{
    using BF = BFmt<FMT>;
    constexpr int BM = 32, BN = 32;
    constexpr int SC = BF::kHasMin ? 4 : 2;                 // f32 scales per weight row
    constexpr int REGION = (BM + BN) * LDK + 2 * BN * SC;   // bf16: A, B, then the scales
    static_assert(1024 * 4 <= REGION * 2, "wave partials fit the wave's region");
    __shared__ __attribute__((aligned(16))) __bf16 lds[WAVES * REGION];

    // the wave index is the same on every lane; read from one lane, the
    // compiler knows it (and the K steps derived from it) to be uniform, so
    // the buffer loads' scalar offsets need no per-lane loop
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
    const int n0 = blockIdx.x * (GATED ? BN / 2 : BN);
    const int P = K / 64;
    const int row_bytes = P * BF::kPairBytes;
    __bf16 *As = lds + wave * REGION;
    __bf16 *Bs = As + BM * LDK;
    float *ds = reinterpret_cast<float *>(Bs + BN * LDK);  // [BN][SC]: scales, then offsets

    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(x), 0, M * K * 4, kBufferWord3);
    const int b_len = min(GATED ? BN / 2 : BN, N - n0) * row_bytes;
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(w + (int64_t)n0 * row_bytes), 0, b_len, kBufferWord3);
    // activation row lane / 16 + 4 u (u < 4), columns 4 (lane % 16) .. +3
    const int a_col = 4 * (lane % 16);
    const int a_voff0 = ((lane / 16) * K + a_col) * 4;
    const int b_row = lane / 2, b_blk = lane % 2;
    const int b_roff = (GATED ? b_row % 16 : b_row) * row_bytes;

    float4 a_reg[4];
    uint32_t b_reg[BF::kWin];
    auto load = [&](int p) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                a_rsrc, a_voff0 + 16 * K * u, p * 256, 0);
            a_reg[u] = __builtin_bit_cast(float4, v);
        }
        if constexpr (GATED) {
            // gate rows from w, up rows from w2; the other load lands past
            // its resource's end and reads zeros
            const __amdgpu_buffer_rsrc_t u_rsrc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t *>(w2 + (int64_t)n0 * row_bytes), 0, b_len, kBufferWord3);
            uint32_t u_reg[BF::kWin];
            BF::load_step(b_rsrc, b_row < 16 ? b_roff : b_len, b_blk, p, b_reg);
            BF::load_step(u_rsrc, b_row < 16 ? b_len : b_roff, b_blk, p, u_reg);
#pragma unroll
            for (int i = 0; i < BF::kWin; ++i) b_reg[i] |= u_reg[i];
        } else {
            BF::load_step(b_rsrc, b_roff, b_blk, p, b_reg);
        }
    };

    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    const f32x16 zero = acc;
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

    const int frow = lane % 32, fk = 8 * (lane / 32);
    load(min(wave, P - 1));
    for (int p = wave; p < P; p += WAVES) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float4 v = a_reg[u];
            uint2 hi, lo;
            hi.x = pack_bf16x2(v.x, v.y);
            hi.y = pack_bf16x2(v.z, v.w);
            lo.x = pack_bf16x2(v.x - bf16_round(v.x), v.y - bf16_round(v.y));
            lo.y = pack_bf16x2(v.z - bf16_round(v.z), v.w - bf16_round(v.w));
            const int r = lane / 16 + 4 * u;
            *reinterpret_cast<uint2 *>(&As[r * LDK + a_col]) = hi;
            *reinterpret_cast<uint2 *>(&As[(r + 16) * LDK + a_col]) = lo;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            BF::codes_quarter(b_reg, b_blk, q, &Bs[b_row * LDK + 32 * b_blk]);
        if constexpr (BF::kHasMin) {
            // the lane with b_blk holds the header: sub-block 2c + b_blk
            float dsc, dmn;
            BF::sub_scales(b_reg, b_blk, dsc, dmn);
            ds[SC * b_row + b_blk] = dsc;
            ds[SC * b_row + 2 + b_blk] = dmn;
        } else {
            ds[SC * b_row + b_blk] = BF::scale(b_reg, b_blk);
        }
        load(min(p + WAVES, P - 1));            // registers are free again
        wave_lds_sync();
        const float d0 = ds[SC * frow], d1 = ds[SC * frow + 1];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x16 c = zero, xs = zero;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int s = 2 * blk + s2;
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&As[frow * LDK + fk + 16 * s]);
                const bf16x8 b = *reinterpret_cast<const bf16x8 *>(&Bs[frow * LDK + fk + 16 * s]);
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
                if constexpr (BF::kHasMin)
                    xs = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ones, xs, 0, 0, 0);
            }
            const float d = blk ? d1 : d0;
            if constexpr (BF::kHasMin) {
                const float dm = ds[SC * frow + 2 + blk];
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] = fmaf(-dm, xs[e], acc[e]);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = fmaf(d, c[e], acc[e]);
        }
        wave_lds_sync();                        // operands read before the next writes
    }

    // partials red[wave][e][lane] = C[8 (e / 4) + 4 (lane / 32) + e % 4][lane % 32];
    // activation row m = that row for e < 8, its lo part at e + 8
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int e = 0; e < 16; ++e) red[(wave * 16 + e) * 64 + lane] = acc[e];
    __syncthreads();
    if constexpr (GATED) {
        // column c < 16 of the tile is gate row n0 + c, column c + 16 the
        // same up row
        for (int o = threadIdx.x; o < 8 * 64; o += 64 * WAVES) {
            const int l = o % 64, e = o / 64;
            if (l % 32 >= 16) continue;
            const int m = 8 * (e / 4) + 4 * (l / 32) + e % 4;
            const int n = n0 + l % 32;
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int q = 0; q < WAVES; ++q) {
                g += red[(q * 16 + e) * 64 + l];
                u += red[(q * 16 + e) * 64 + l + 16];
            }
            float g_lo = 0.f, u_lo = 0.f;
#pragma unroll
            for (int q = 0; q < WAVES; ++q) {
                g_lo += red[(q * 16 + e + 8) * 64 + l];
                u_lo += red[(q * 16 + e + 8) * 64 + l + 16];
            }
            if (m < M && n < N)
                y[(int64_t)m * N + n] =
                    gelu_tanh((g + g_lo) * BF::kCodeScale) * ((u + u_lo) * BF::kCodeScale);
        }
        return;
    }
    for (int o = threadIdx.x; o < 8 * 64; o += 64 * WAVES) {
        const int l = o % 64, e = o / 64;
        const int m = 8 * (e / 4) + 4 * (l / 32) + e % 4;
        const int n = n0 + l % 32;
        float hi = 0.f, lo = 0.f;
#pragma unroll
        for (int q = 0; q < WAVES; ++q) {
            hi += red[(q * 16 + e) * 64 + l];
            lo += red[(q * 16 + e + 8) * 64 + l];
        }
        if (m < M && n < N) y[(int64_t)m * N + n] = (hi + lo) * BF::kCodeScale;
    }
}

template <int FMT, class TL>
hipError_t launch_tiles(const float *x, const uint8_t *w, float *y, int M, int N, int K,
                        hipStream_t stream)
{
    // the kernel runs whole K steps of 64
    if (K % BK != 0) return hipErrorInvalidValue;
    const int tiles_m = (M + TL::BM - 1) / TL::BM;
    const int tiles_n = (N + TL::BN - 1) / TL::BN;
    const int tiles = tiles_m * tiles_n;
    const int per_xcd = (tiles + kXcds - 1) / kXcds;
    hipLaunchKernelGGL((gemm_kernel<FMT, TL>), dim3(per_xcd * kXcds), dim3(TL::kThreads), 0,
                       stream, x, w, y, M, N, K, tiles_m, tiles_n, per_xcd);
    return hipGetLastError();
}

// MI355X has 256 compute units: with fewer 256 x 256 tiles than that, the
// 128 x 128 tile (4 x as many workgroups) keeps more of the chip busy.
constexpr int64_t kComputeUnits = 256;

// Up to kMidRowsMax rows the medium-M kernel (timing sweeps at K = 1024 ..
// 8192: M = 16, N = 8192 7.3 us and M = 128, N = 2048, K = 8192 22.5 us,
// against 23 and 88 us on tiles). Each workgroup's K loop is short and
// latency-bound, so the shape that runs best is the one whose workgroups
// all fit the chip at once: from N = 4096 the launch takes, among 32- or
// 64-row bands and 32- or 64-column slices, the one with the most
// workgroups not above the compute unit count (on a tie the wider slices,
// which re-read the activation band fewer times, then the narrower bands,
// which compute fewer rows past M), and when every shape has more, 64 x 64
// tiles with 4 waves (two workgroups per compute unit).
// Against the former 64 x 32 / 32 x 32 choice: M = 128, N = 8192 20.4 ->
// 16.3 us; M = 40, N = 4096 11.1 -> 7.2 us; M = 128, N = 16384 39.9 -> 24.6
// us; M = 64, N = 8192 12.4 -> 11.8 us.
constexpr int kMidRowsMax = 128;

template <int FMT>
hipError_t launch_mid_auto(const float *x, const uint8_t *w, float *y, int M, int N, int K,
                           hipStream_t stream)
{
    // few column slices: 16 waves keep more K steps in flight per slice
    // (N = 2048, K = 8192: M = 16 17.0 against 17.9 us, M = 64 18.3 against
    // 19.4); more rows than kMidRowsMax give enough bands for the rule below
    if (N < 4096 && M <= kMidRowsMax) return launch_mid<FMT, 1, 1, 16>(x, w, y, M, N, K, stream);
    int best = -1;
    int64_t best_wg = 0;
    for (int c = 0; c < 4; ++c) {
        const int mt = 1 + (c & 1), nt = 1 + (c >> 1);
        const int64_t wg = (int64_t)((N + 32 * nt - 1) / (32 * nt)) * ((M + 32 * mt - 1) / (32 * mt));
        if (wg > kComputeUnits) continue;
        const int bnt = 1 + (best >> 1), bmt = 1 + (best & 1);
        if (best < 0 || wg > best_wg ||
            (wg == best_wg && (nt > bnt || (nt == bnt && mt < bmt)))) {
            best = c;
            best_wg = wg;
        }
    }
    switch (best) {
    case 0: return launch_mid<FMT, 1, 1, 8>(x, w, y, M, N, K, stream);
    case 1: return launch_mid<FMT, 2, 1, 8>(x, w, y, M, N, K, stream);
    case 2: return launch_mid<FMT, 1, 2, 8>(x, w, y, M, N, K, stream);
    case 3: return launch_mid<FMT, 2, 2, 8>(x, w, y, M, N, K, stream);
    default: return launch_mid<FMT, 2, 2, 4>(x, w, y, M, N, K, stream);
    }
}

// More rows take the tile kernels: 256 x 256 tiles when they fill at least
// three quarters of the compute units in one round (M = 1024, N = 14336,
// K = 4096, 224 tiles: 169.6 -> 117.4 us against 128 x 128 tiles; M = 512,
// N = 28672, K = 8192: 325.7 -> 229.6 us; at 112 tiles the two are level,
// at 96 the smaller tiles are faster), else 128 x 128 ones. With at most 128 of those
// (half the chip, each running the whole K loop; below N = 4096 fewer than
// 128) the medium-M kernel's smaller tiles are faster (sweep at M =
// 160-768: N = 8192, K = 2048, M = 160 26.0 -> 21.2 us; N = 4096, K = 4096,
// M = 256 46.9 -> 25.3 us, M = 512 47.7 -> 42.2 us; N = 1024, K = 4096, M =
// 160 42.7 -> 10.3 us, M = 512 43.1 -> 17.5 us; N = 2048, K = 8192, M = 512
// 82.1 -> 42.8 us; the tile kernel wins from 192 small tiles on, e.g. N =
// 8192, M = 384 27.0 against 35.4 us, and below N = 4096 from 128: N = 1024,
// M = 2048 43.9 against 53.2 us).
template <int FMT>
hipError_t launch_fmt(const float *x, const uint8_t *w, float *y, int M, int N, int K,
                      hipStream_t stream)
{
    if (M <= kMidRowsMax) return launch_mid_auto<FMT>(x, w, y, M, N, K, stream);
    const int64_t large_tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
    if (large_tiles >= kComputeUnits * 3 / 4)
        return launch_tiles<FMT, TileLarge>(x, w, y, M, N, K, stream);
    const int64_t small_tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
    if (small_tiles < kComputeUnits / 2 || (N >= 4096 && small_tiles == kComputeUnits / 2))
        return launch_mid_auto<FMT>(x, w, y, M, N, K, stream);
    return launch_tiles<FMT, TileSmall>(x, w, y, M, N, K, stream);
}

}  // namespace

hipError_t launch_gemv_slices(int fmt, const float *x, const uint8_t *w, float *y, int M,
                              int N, int K, hipStream_t stream)
{
    if (M > 16) return hipErrorInvalidValue;
    const dim3 grid((N + 31) / 32);
    // Q4_0 and Q4_K: 8 waves from N = 8192 (a sweep of 4, 8 and 16 at M =
    // 12 and 16: FFN up shape 8.3 -> 7.6 us, N = 28672, K = 8192 76.1 ->
    // 68.3 us, N = 65536, K = 2048 53.0 -> 40.0 us, N = 262144 204.5 ->
    // 150.0 us for Q4_0, M = 16), 16 on narrower matrices, which keep more
    // K steps in flight per slice (M = 16, N = 2048, K = 8192 20.3 us
    // against 22.0 with 8); Q8_0: 8 (its wider windows; level with 4)
    const bool wide = N >= 8192;
    if (fmt == FMT_Q4_0) {
        if (wide)
            hipLaunchKernelGGL((gemv_slice_kernel<FMT_Q4_0, 8>), grid, dim3(512), 0, stream, x, w,
                               y, M, N, K);
        else
            hipLaunchKernelGGL((gemv_slice_kernel<FMT_Q4_0, 16>), grid, dim3(1024), 0, stream, x,
                               w, y, M, N, K);
    } else if (fmt == FMT_Q4_K) {
        if (wide)
            hipLaunchKernelGGL((gemv_slice_kernel<FMT_Q4_K, 8>), grid, dim3(512), 0, stream, x, w,
                               y, M, N, K);
        else
            hipLaunchKernelGGL((gemv_slice_kernel<FMT_Q4_K, 16>), grid, dim3(1024), 0, stream, x,
                               w, y, M, N, K);
    } else
        hipLaunchKernelGGL((gemv_slice_kernel<FMT_Q8_0, 8>), grid, dim3(512), 0, stream, x, w, y,
                           M, N, K);
    return hipGetLastError();
}

hipError_t launch_ffn_gate_up_slices(const float *x, const uint8_t *w_gate,
                                     const uint8_t *w_up, float *h, int M, int N, int K,
                                     hipStream_t stream)
{
    if (M > 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemv_slice_kernel<FMT_Q4_0, 8, true>), dim3((N + 15) / 16), dim3(512), 0,
                       stream, x, w_gate, h, M, N, K, w_up);
    return hipGetLastError();
}

hipError_t launch_gemm(int fmt, const float *x, const uint8_t *w, float *y, int M, int N,
                       int K, hipStream_t stream)
{
    if (fmt == FMT_Q4_K) return launch_fmt<FMT_Q4_K>(x, w, y, M, N, K, stream);
    return fmt == FMT_Q4_0 ? launch_fmt<FMT_Q4_0>(x, w, y, M, N, K, stream)
                           : launch_fmt<FMT_Q8_0>(x, w, y, M, N, K, stream);
}

}  // namespace qmm
