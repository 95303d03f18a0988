// Small-M GEMV (2 <= M <= 16 activation rows: batched or speculative
// decode) over GGUF Q4_0 / Q8_0 weights, and 5 <= M <= 16 over Q4_K
// super-blocks, on the bf16 matrix cores. The C-ABI sends 5 <= M <= 8, and
// 9 <= M <= 16 up to N = 4096 (below N = 3072 at K <= 2048), here when
// K % 256 == 0 (each wave takes K in slices of 256; always so for Q4_K),
// and 3-4 rows at the shapes where this kernel beats the f32 FMA kernels
// that stream the weights for one row (they decode each weight once for
// all rows); for 9 rows and more elsewhere the 32-row weight-slice kernel
// is faster.
//
// With several activation rows the f32 FMA count (M per weight) outgrows
// the weight stream, so the contraction moves to v_mfma_f32_16x16x32_bf16:
// one instruction covers 16 A rows x 16 weight rows x one 32-wide block.
// Accuracy is kept to the f32 bound:
//  * B operand (weights): the integer codes 16*(q-8) (Q4_0), q (Q8_0) or
//    the nibble q in 0..15 (Q4_K), exact in bf16. The fp16 scale d (Q4_0,
//    Q8_0) or the sub-block scale d*sc (Q4_K) is applied in f32 to the
//    block's result, so no weight is rounded. A Q4_K sub-block's offset
//    dmin*mn multiplies the sum of its 32 activations, which one more MFMA
//    per block forms from the same A operand against a B operand of ones:
//    per block, acc += d*sc * sum(q x) - dmin*mn * sum(x), in f32.
//  * A operand (activations): x = hi + lo with hi = bf16(x) and
//    lo = bf16(x - hi), both round-to-nearest-even; hi + lo represents x to
//    within 2^-17 |x| (about 16 of its 24 significand bits), each product
//    of a code and a term is exact, and the products accumulate in f32:
//    far inside the 1e-4 relative bound. For M <= 8 (PACK) the hi
//    rows and lo rows share one instruction (A rows m and M + m); for M > 8
//    they take one instruction each.
// Within a block the k order is permuted identically in A and B so that
// each lane's eight weights come from one qs dword (Q4_0: bytes 4g..4g+3,
// i.e. elements 4g..4g+3 and 4g+16..4g+19) or two (Q8_0: elements
// 8g..8g+7; Q4_K: the nibbles of bytes 8g..8g+7 of the sub-block's 32).
//
// Work split: a workgroup of WAVES waves owns NT x 16 weight rows; each wave
// takes a 256-wide slice of K (8 blocks, or one Q4_K super-block) per pass.
// A wave
//  1. loads its activation slice (M rows x 256, one float4 per lane and
//     row, coalesced) and its weight bytes (whole 36/68-byte pairs of
//     blocks with 16-byte loads; a 144-byte Q4_K super-block is four
//     36-byte pieces);
//  2. writes both to its own LDS region: activations already split into
//     hi/lo bf16 and laid out as MFMA A fragments, weight pairs re-aligned
//     so that every qs dword is dword-aligned;
//  3. runs, per block, one A-fragment read, one B dword and scale read per
//     weight tile, the MFMA(s), and the f32 scale-and-accumulate.
// No workgroup barrier is needed until the final reduction, where the
// waves' partial sums meet in LDS in a fixed order (bitwise reproducible).
#include "qmm_internal.h"

namespace qmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int KW = 256;             // K per wave per pass
constexpr int BPW = KW / 32;        // blocks per wave per pass (8)
constexpr int PPW = KW / 64;        // pairs per wave per pass (4)

template <int FMT> struct Fmt;

template <> struct Fmt<FMT_Q4_0> {
    static constexpr int kPairBytes = 36;
    static constexpr int kPairDwords = 9;     // global and LDS
    static constexpr float kOutScale = 1.0f / 16.0f;

    // global pair (9 dwords: d0 at byte 0, qs0 at 2..17, d1 at 18, qs1 at
    // 20..35) -> LDS pair: qs0[4], qs1[4], (d0 | d1 << 16)
    __device__ static void relayout(const uint32_t *D, uint32_t *o)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_alignbyte(D[i + 1], D[i], 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[4 + i] = D[5 + i];
        o[8] = (D[0] & 0xFFFFu) | (D[4] & 0xFFFF0000u);
    }

    static constexpr bool kHasMin = false;

    // lane group g's eight codes of block b of an LDS weight row, and the scale
    __device__ static void b_operand(const uint32_t *row, int b, int g, bf16x8 &bq, float &d)
    {
        const uint32_t *pair = row + (b / 2) * kPairDwords;
        const int h = b & 1;
        const uint32_t q = pair[4 * h + g];
        const uint32_t dd = pair[8];
        d = h ? half_hi(dd) : half_lo(dd);
        const uint32_t lo = lo16(q), hi = hi16(q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bq[e] = (__bf16)sbyte(lo, e);
            bq[4 + e] = (__bf16)sbyte(hi, e);
        }
    }

    // A-fragment position of block element kk (a multiple of 4): lane
    // group and first of the four slots
    __device__ static void slot(int kk, int &g, int &e0)
    {
        g = (kk & 15) >> 2;
        e0 = kk < 16 ? 0 : 4;
    }
};

template <> struct Fmt<FMT_Q8_0> {
    static constexpr int kPairBytes = 68;
    static constexpr int kPairDwords = 17;
    static constexpr float kOutScale = 1.0f;

    // global pair (17 dwords: d0 at 0, q0 at 2..33, d1 at 34, q1 at 36..67)
    // -> LDS pair: q0[8], q1[8], (d0 | d1 << 16)
    __device__ static void relayout(const uint32_t *D, uint32_t *o)
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = __builtin_amdgcn_alignbyte(D[i + 1], D[i], 2);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[8 + i] = D[9 + i];
        o[16] = (D[0] & 0xFFFFu) | (D[8] & 0xFFFF0000u);
    }

    static constexpr bool kHasMin = false;

    __device__ static void b_operand(const uint32_t *row, int b, int g, bf16x8 &bq, float &d)
    {
        const uint32_t *pair = row + (b / 2) * kPairDwords;
        const int h = b & 1;
        // two dword reads: an LDS pair of 17 dwords is only dword aligned
        const uint32_t q0 = pair[8 * h + 2 * g], q1 = pair[8 * h + 2 * g + 1];
        const uint32_t dd = pair[16];
        d = h ? half_hi(dd) : half_lo(dd);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bq[e] = (__bf16)sbyte(q0, e);
            bq[4 + e] = (__bf16)sbyte(q1, e);
        }
    }

    __device__ static void slot(int kk, int &g, int &e0)
    {
        g = kk >> 3;
        e0 = kk & 7;
    }
};

// Q4_K: one 144-byte super-block (256 weights, eight sub-blocks of 32) per
// weight row and pass, staged as four 36-byte pieces so that the loads are
// those of a Q4_0 row of the same K. LDS keeps the global order: dword 0 is
// d | dmin << 16, dwords 1-3 the twelve 6-bit scale/minimum bytes, dwords
// 4-35 the nibbles (weight 64c + i, i < 32, low nibble of qs byte 32c + i;
// weight 64c + 32 + i its high nibble).
template <> struct Fmt<FMT_Q4_K> {
    static constexpr int kPairBytes = 36;
    static constexpr int kPairDwords = 9;
    static constexpr float kOutScale = 1.0f;
    static constexpr bool kHasMin = true;

    __device__ static void relayout(const uint32_t *D, uint32_t *o)
    {
#pragma unroll
        for (int i = 0; i < 9; ++i) o[i] = D[i];
    }

    // sub-block b's 6-bit scale and minimum from the twelve scale bytes
    // (s0, s1, s2 = bytes 0-3, 4-7, 8-11): for b < 4 the low 6 bits of bytes
    // b and 4 + b; for b >= 4 the two nibbles of byte 4 + b below the top 2
    // bits of bytes b - 4 (scale) and b (minimum)
    __device__ static void scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int b, int &sc,
                                     int &mn)
    {
        if (b < 4) {
            sc = (s0 >> (8 * b)) & 63;
            mn = (s1 >> (8 * b)) & 63;
        } else {
            const uint32_t lo = s2 >> (8 * (b - 4));
            sc = (lo & 15) | (((s0 >> (8 * (b - 4) + 6)) & 3) << 4);
            mn = ((lo >> 4) & 15) | (((s1 >> (8 * (b - 4) + 6)) & 3) << 4);
        }
    }

    // lane group g's eight codes of sub-block b: the low (even b) or high
    // (odd b) nibbles of bytes 8g..8g+7 of the sub-block pair's 32 qs bytes,
    // i.e. elements 8g..8g+7 of the sub-block; its scale d*sc and offset
    // dmin*mn
    __device__ static void b_operand(const uint32_t *row, int b, int g, bf16x8 &bq, float &ds,
                                     float &dm)
    {
        const uint32_t *qs = row + 4 + 8 * (b / 2) + 2 * g;
        const int sh = 4 * (b & 1);
        const uint32_t c0 = (qs[0] >> sh) & 0x0F0F0F0Fu, c1 = (qs[1] >> sh) & 0x0F0F0F0Fu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bq[e] = (__bf16)(float)((c0 >> (8 * e)) & 0xFFu);
            bq[4 + e] = (__bf16)(float)((c1 >> (8 * e)) & 0xFFu);
        }
        int sc, mn;
        scale_min(row[1], row[2], row[3], b, sc, mn);
        ds = half_lo(row[0]) * (float)sc;
        dm = half_hi(row[0]) * (float)mn;
    }

    __device__ static void slot(int kk, int &g, int &e0)
    {
        g = kk >> 3;
        e0 = kk & 7;
    }
};

// hi = bf16(v), lo = bf16(v - hi), both round to nearest even
__device__ __forceinline__ void split4(const float4 v, bf16x4 &hi, bf16x4 &lo)
{
    const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 h = (__bf16)f[i];
        hi[i] = h;
        lo[i] = (__bf16)(f[i] - (float)h);
    }
}

// LDS dword address of A-fragment slot s (one lane's 16 bytes of one block's
// operand). Slot group G = s / 16 starts 4 (G + G / 8) dwords further on, so
// the staging writes, in which the lanes of one instruction hold the same
// activation row in slots 16 apart (different blocks and lane groups), fall
// in different banks, while each group's 16 slots (read by 16 lanes) stay
// contiguous.
__device__ __forceinline__ int afrag(int s)
{
    const int g = s >> 4;
    return 4 * s + 4 * (g + (g >> 3));
}

// GATED (NT = 2): the gated FFN front half. Weight tile 0 is rows n0 ..
// n0 + 15 of the gate matrix w, tile 1 the same rows of the up matrix w2,
// and the output is y[m][n] = gelu_tanh(gate) * up, formed in f32 once the
// waves' sums are complete. Grid: ceil(N / 16) workgroups.
template <int FMT, bool PACK, int NT, int WAVES, bool PF, bool GATED = false>
__global__ __launch_bounds__(64 * WAVES) void gemv_small_m_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ w,
    float *__restrict__ y, int M, int N, int K, const uint8_t *__restrict__ w2 = nullptr)
{
    using L = Fmt<FMT>;
    constexpr int TERMS = PACK ? 1 : 2;             // A operands per block
    constexpr int MMAX = PACK ? 8 : 16;
    constexpr int NG = BPW * TERMS * 4;             // A-fragment slot groups per wave
    constexpr int AF = NG * 64 + 4 * (NG + NG / 8); // A-fragment dwords per wave, with shifts
    constexpr int WROWS = 16 * NT;                  // weight rows per workgroup
    constexpr int PPL = WROWS * PPW / 64;           // pairs loaded per lane
    // a weight row's PPW pairs plus one dword, so that the rows (and the
    // lanes staging them) start in different banks
    constexpr int WROW = PPW * L::kPairDwords + 1;
    constexpr int WD = WROWS * WROW;                // weight dwords per wave
    constexpr int REGION = AF + WD;
    static_assert(PPL * 64 == WROWS * PPW, "pairs must tile the wave");
    static_assert(PPW % PPL == 0, "a lane's pairs lie in one weight row");
    static_assert(WAVES * NT * 64 * 4 <= WAVES * REGION, "reduction fits in LDS");
    static_assert(!GATED || NT == 2, "a gated tile is 16 gate rows and 16 up rows");
    __shared__ __attribute__((aligned(16))) uint32_t lds[WAVES * REGION];

    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    uint32_t *af = lds + wave * REGION;
    uint32_t *wl = af + AF;
    const int P = K / 64;
    const int64_t row_bytes = (int64_t)P * L::kPairBytes;
    const int n0 = blockIdx.x * (GATED ? 16 : WROWS);

    // A rows without an activation row stay zero for the whole kernel
    for (int i = lane; i < AF; i += 64) af[i] = 0u;

    // this lane's weight pairs: row lrow of the tile, local pairs lp0 + u
    const int lrow = lane / (PPW / PPL);
    const int lp0 = (lane % (PPW / PPL)) * PPL;
    const uint8_t *wsrc;
    if constexpr (GATED)
        wsrc = (lrow < 16 ? w : w2) + (int64_t)min(n0 + lrow % 16, N - 1) * row_bytes;
    else
        wsrc = w + (int64_t)min(n0 + lrow, N - 1) * row_bytes;

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // ---- 1. loads of the slice at k0 into registers
    float4 xv[MMAX];
    uint32_t D[PPL][L::kPairDwords];
    auto load = [&](int k0) {
#pragma unroll
        for (int m = 0; m < MMAX; ++m)
            if (m < M) xv[m] = *reinterpret_cast<const float4 *>(x + (int64_t)m * K + k0 + 4 * lane);
#pragma unroll
        for (int u = 0; u < PPL; ++u) {
            const uint8_t *src = wsrc + (int64_t)(k0 / 64 + lp0 + u) * L::kPairBytes;
#pragma unroll
            for (int i = 0; i + 4 <= L::kPairDwords; i += 4) {
                const u32x4_a4 v = *reinterpret_cast<const u32x4_a4 *>(src + 4 * i);
                D[u][i] = v.x; D[u][i + 1] = v.y; D[u][i + 2] = v.z; D[u][i + 3] = v.w;
            }
            D[u][L::kPairDwords - 1] =
                *reinterpret_cast<const uint32_t *>(src + 4 * (L::kPairDwords - 1));
        }
    };
    // PF: a wave's next slice is loaded while its matrix cores work on this
    // one (the registers are free once this slice sits in LDS)
    if constexpr (PF)
        if (wave * KW < K) load(wave * KW);
    for (int k0 = wave * KW; k0 < K; k0 += WAVES * KW) {
        if constexpr (!PF) load(k0);
        // ---- 2. to LDS
        wave_lds_sync();            // previous pass's reads done
        {
            const int b = lane / 8, kk = 4 * (lane % 8);
            int g, e0;
            L::slot(kk, g, e0);
            // slots of A row 0 for the hi and lo parts; row r (< 16) of the
            // same fragment is 4 r dwords further on (same slot group)
            const int tl = PACK ? 0 : 1;              // A operand of the lo part
            uint32_t *ahi = &af[afrag((b * TERMS + 0) * 64 + 16 * g) + e0 / 2];
            uint32_t *alo = &af[afrag((b * TERMS + tl) * 64 + 16 * g) + e0 / 2];
#pragma unroll
            for (int m = 0; m < MMAX; ++m) {
                if (m < M) {
                    bf16x4 hi, lo;
                    split4(xv[m], hi, lo);
                    const int rl = PACK ? M + m : m;  // A row of the lo part
                    *reinterpret_cast<bf16x4 *>(ahi + 4 * m) = hi;
                    *reinterpret_cast<bf16x4 *>(alo + 4 * rl) = lo;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < PPL; ++u)
            L::relayout(D[u], wl + lrow * WROW + (lp0 + u) * L::kPairDwords);
        if constexpr (PF)
            if (k0 + WAVES * KW < K) load(k0 + WAVES * KW);
        wave_lds_sync();
        // ---- 3. matrix cores
        const int col = lane % 16, g = lane / 16;
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            bf16x8 a[TERMS];
#pragma unroll
            for (int tt = 0; tt < TERMS; ++tt)
                a[tt] = *reinterpret_cast<const bf16x8 *>(&af[afrag((b * TERMS + tt) * 64 + lane)]);
            // Q4_K: sum of block b's activations for each A row, in every column
            f32x4 xsum = zero;
            if constexpr (L::kHasMin) {
                bf16x8 ones;
#pragma unroll
                for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
                xsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], ones, zero, 0, 0, 0);
                if constexpr (!PACK)
                    xsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[TERMS - 1], ones, xsum, 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t *row = wl + (16 * t + col) * WROW;
                bf16x8 bq;
                float d, dm = 0.f;
                if constexpr (L::kHasMin)
                    L::b_operand(row, b, g, bq, d, dm);
                else
                    L::b_operand(row, b, g, bq, d);
                f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], bq, zero, 0, 0, 0);
                if constexpr (!PACK)
                    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[TERMS - 1], bq, c, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (L::kHasMin) acc[t][e] = fmaf(-dm, xsum[e], acc[t][e]);
                    acc[t][e] = fmaf(d, c[e], acc[t][e]);
                }
            }
        }
    }

    // acc[t][e] is C[A row 4g + e][weight row 16 t + col] of this wave; sum
    // the waves (and, packed, A rows m and M + m) in a fixed order.
    __syncthreads();
    f32x4 *red = reinterpret_cast<f32x4 *>(lds);    // [WAVES][NT][64]
#pragma unroll
    for (int t = 0; t < NT; ++t) red[(wave * NT + t) * 64 + lane] = acc[t];
    __syncthreads();
    if constexpr (GATED) {
        for (int o = threadIdx.x; o < 16 * 16; o += 64 * WAVES) {
            const int m = o / 16, c = o % 16;
            const int n = n0 + c;
            if (m >= M || n >= N) continue;
            float s[2] = {0.f, 0.f};
            for (int q = 0; q < WAVES; ++q) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    s[t] += red[(q * NT + t) * 64 + 16 * (m / 4) + c][m % 4];
                    if constexpr (PACK)
                        s[t] += red[(q * NT + t) * 64 + 16 * ((M + m) / 4) + c][(M + m) % 4];
                }
            }
            y[(int64_t)m * N + n] = gelu_tanh(s[0] * L::kOutScale) * (s[1] * L::kOutScale);
        }
        return;
    }
    for (int o = threadIdx.x; o < 16 * WROWS; o += 64 * WAVES) {
        const int m = o / WROWS, nl = o % WROWS;
        const int t = nl / 16, c = nl % 16;
        const int n = n0 + nl;
        if (m >= M || n >= N) continue;
        float s = 0.f;
        for (int q = 0; q < WAVES; ++q) {
            s += red[(q * NT + t) * 64 + 16 * (m / 4) + c][m % 4];
            if constexpr (PACK) s += red[(q * NT + t) * 64 + 16 * ((M + m) / 4) + c][(M + m) % 4];
        }
        y[(int64_t)m * N + n] = s * L::kOutScale;
    }
}

template <int FMT, bool PACK, int NT, int WAVES, bool PF>
void launch_shape(const float *x, const uint8_t *w, float *y, int M, int N, int K,
                  hipStream_t stream)
{
    const int grid = (N + 16 * NT - 1) / (16 * NT);
    hipLaunchKernelGGL((gemv_small_m_kernel<FMT, PACK, NT, WAVES, PF>), dim3(grid),
                       dim3(64 * WAVES), 0, stream, x, w, y, M, N, K);
}

// Launch shapes from timing sweeps on MI355X (random weights, cold copies;
// NT x 16 weight rows and WAVES waves per workgroup, PF = next-slice
// prefetch). Prefetch measured faster wherever a workgroup holds 16 weight
// rows (Q4_0, M = 8, N = 2048, K = 16384: 18.6 -> 17.1 us; Q4_K, M = 8,
// N = 4096, K = 14336: 20.1 -> 18.0 us) and with one slice per wave (its
// loads then issue before the LDS clearing: FFN up shape, M = 8, 7.18 ->
// 6.89 us), slightly slower with 32 rows and 8 waves over deeper K (N =
// 28672, K = 8192: 57.9 -> 58.9 us).
// For 5-8 rows over wide matrices the fastest shape is, in the sweeps, the
// one with the most waves resident whose workgroups all fit the chip at
// once: 32 rows and 8 waves (one workgroup per CU) up to N = 8192; 16 rows
// and 4 waves (three per CU, 768 in all) up to N = 12288 (Q4_0, N = 10240,
// K = 4096: 18.0 -> 14.5 us; Q8_0 24.4 -> 18.6 us); 32 rows and 4 waves (two
// per CU) up to N = 16384 (Q4_0, N = 14336, K = 4096: 18.5 -> 16.6 us; Q4_K
// with the prefetch, N = 13824, K = 5120: 22.6 -> 21.3 us).
// Beyond that Q4_0 runs 32 rows in 2-wave workgroups (N = 28672, K = 8192:
// 58.0 -> 51.0 us; N = 128256, K = 4096: 116.2 -> 101.6 us), Q4_K 32 rows in
// 4-wave ones (N = 65536, K = 4096: 73.1 -> 66.2 us), and Q8_0, whose weight
// rows take more LDS, 16 rows in 4 waves below N = 65536 (N = 28672, K =
// 8192: 85.8 -> 73.9 us) and 32 rows in 4 waves above (N = 128256, K = 4096:
// 159.5 -> 154.1 us).
template <int FMT>
hipError_t launch_fmt(const float *x, const uint8_t *w, float *y, int M, int N, int K,
                      hipStream_t stream)
{
    if (N <= 4096) {
        // at most 128 workgroups of 32 rows: 16 rows per workgroup (one per
        // compute unit), eight waves over K (seven for M > 8, whose A
        // fragments take twice the LDS; Q4_0, M = 16, N = 4096, K = 14336:
        // 34.0 us on the 32-row weight slices, 28.8 with six waves, 24.4 with
        // seven and prefetch)
        if (M <= 8)
            launch_shape<FMT, true, 1, 8, true>(x, w, y, M, N, K, stream);
        else
            launch_shape<FMT, false, 1, 7, true>(x, w, y, M, N, K, stream);
    } else if (M > 8) {
        // 32 weight rows per workgroup, six waves over K (from a launch
        // sweep at M = 12 and 16, K = 2048, N = 8192). The entry points send
        // 9-16 rows over N > 4096 to the 32-row weight slices, which are
        // faster there, so this shape only backs the launcher's contract.
        launch_shape<FMT, false, 2, 6, false>(x, w, y, M, N, K, stream);
    } else if (FMT == FMT_Q8_0 && N < 8192) {
        // Q8_0 between N = 4096 and 8192: 16 rows in 4 waves (N = 6144,
        // K = 4096, M = 6: 13.7 -> 12.1 us)
        launch_shape<FMT, true, 1, 4, true>(x, w, y, M, N, K, stream);
    } else if (N <= 8192) {
        // 32 rows in 8 waves, one workgroup per compute unit in one round
        // (between N = 4096 and 8192 in place of 16 rows: Q4_0, N = 6144,
        // K = 4096, M = 6: 11.7 -> 9.4 us; Q4_K 13.1 -> 10.9 us)
        if (K <= 8 * KW)
            launch_shape<FMT, true, 2, 8, true>(x, w, y, M, N, K, stream);
        else
            launch_shape<FMT, true, 2, 8, false>(x, w, y, M, N, K, stream);
    } else if constexpr (FMT == FMT_Q8_0) {
        if (N < 65536)
            launch_shape<FMT, true, 1, 4, true>(x, w, y, M, N, K, stream);
        else
            launch_shape<FMT, true, 2, 4, true>(x, w, y, M, N, K, stream);
    } else {
        if (N <= 12288)
            launch_shape<FMT, true, 1, 4, true>(x, w, y, M, N, K, stream);
        else if (N <= 16384 && FMT != FMT_Q4_K)
            launch_shape<FMT, true, 2, 4, false>(x, w, y, M, N, K, stream);
        else if constexpr (FMT == FMT_Q4_K)
            launch_shape<FMT, true, 2, 4, true>(x, w, y, M, N, K, stream);
        else
            launch_shape<FMT, true, 2, 2, true>(x, w, y, M, N, K, stream);
    }
    return hipGetLastError();
}

// Gated FFN front half for 5-16 tokens: 16 gate and 16 up rows per
// workgroup.
template <bool PACK, int WAVES, bool PF>
void launch_gated_shape(const float *x, const uint8_t *wg, const uint8_t *wu, float *h, int M,
                        int N, int K, hipStream_t stream)
{
    hipLaunchKernelGGL((gemv_small_m_kernel<FMT_Q4_0, PACK, 2, WAVES, PF, true>),
                       dim3((N + 15) / 16), dim3(64 * WAVES), 0, stream, x, wg, h, M, N, K, wu);
}

}  // namespace

hipError_t launch_gemv_small_m(int fmt, const float *x, const uint8_t *w, float *y,
                               int M, int N, int K, hipStream_t stream)
{
    if (fmt == FMT_Q4_K) return launch_fmt<FMT_Q4_K>(x, w, y, M, N, K, stream);
    return fmt == FMT_Q4_0 ? launch_fmt<FMT_Q4_0>(x, w, y, M, N, K, stream)
                           : launch_fmt<FMT_Q8_0>(x, w, y, M, N, K, stream);
}

// Gated launch shapes from a timing sweep (random weights, cold copies; N =
// 2048-28672, M = 5, 8, 12, 16): as for the GEMV, the most waves whose
// workgroups (N / 16 of them) all fit the chip at once. Up to 8 rows (13.5
// KB of LDS per wave): 8 waves to N = 4096, 4 to N = 8192, 2 to N = 20480,
// then 4 again (N = 28672, K = 8192, M = 5: 81.2 us, against 98.4 with 2
// waves); 9-16 rows (22.3 KB per wave): 6 waves to N = 4096, else 3 (the
// entry point now sends 9-16 rows over N > 4096 to the gated weight
// slices, which are faster there). Against two GEMV launches for gate and
// up: N = 8192, K = 2048, M = 5 12.8 -> 9.9 us; N = 13824, K = 5120, M = 5
// 35.8 -> 31.2 us; N = 4096, K = 4096, M = 16 20.0 -> 13.1 us.
hipError_t launch_ffn_gate_up_small_m(const float *x, const uint8_t *w_gate,
                                      const uint8_t *w_up, float *h, int M, int N, int K,
                                      hipStream_t stream)
{
    if (M <= 8) {
        if (N <= 4096)
            launch_gated_shape<true, 8, true>(x, w_gate, w_up, h, M, N, K, stream);
        else if (N <= 8192)
            launch_gated_shape<true, 4, false>(x, w_gate, w_up, h, M, N, K, stream);
        else if (N <= 20480)
            launch_gated_shape<true, 2, true>(x, w_gate, w_up, h, M, N, K, stream);
        else
            launch_gated_shape<true, 4, true>(x, w_gate, w_up, h, M, N, K, stream);
    } else {
        if (N <= 4096)
            launch_gated_shape<false, 6, true>(x, w_gate, w_up, h, M, N, K, stream);
        else
            launch_gated_shape<false, 3, true>(x, w_gate, w_up, h, M, N, K, stream);
    }
    return hipGetLastError();
}

}  // namespace qmm
