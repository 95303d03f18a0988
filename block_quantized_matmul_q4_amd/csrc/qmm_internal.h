// Internal declarations shared by the C-ABI layer and the gfx950 kernels.
// Not installed; the public interface is include/qmm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

enum Format : int { FMT_Q4_0 = 0, FMT_Q8_0 = 1, FMT_Q4_K = 2 };

constexpr int kBlock = 32;           // weights per GGUF block
constexpr int kQ4Bytes = 18;         // fp16 d + 16 nibble bytes
constexpr int kQ8Bytes = 34;         // fp16 d + 32 int8

inline constexpr int block_bytes(int fmt) { return fmt == FMT_Q4_0 ? kQ4Bytes : kQ8Bytes; }

// Launchers. Arguments are already validated by the C-ABI layer:
// pointers non-null and aligned, 1 <= M, 1 <= N, 64 <= K <= 65536,
// K % 64 == 0 (whole pairs of blocks per row), N and M * N within int32
// range; launch_gemv_small_m also needs K % 256 == 0. Each returns the
// hipGetLastError() of its launch.
// GEMV with f32 FMAs for M <= kGemvRowsMax activation rows (the weights
// streamed once per launch); more rows, and for Q4_0 and Q8_0 three or four
// rows at the matrix shapes where the FMA kernel is the slower one (the
// entry points choose), take the matrix-core kernels.
constexpr int kGemvRowsMax = 4;
hipError_t launch_gemv_m1(int fmt, const float *x, const uint8_t *w, float *y, int M,
                          int N, int K, hipStream_t stream);
hipError_t launch_gemv_small_m(int fmt, const float *x, const uint8_t *w, float *y,
                               int M, int N, int K, hipStream_t stream);
// GEMV to the f32 bound on the matrix cores over 32-row weight slices (x as
// two bf16 terms, within 2^-17 |x|), M <= 16
// (taken for 9 <= M <= 16 above N = 4096 and, from N = 3072, at K <= 2048,
// and for Q4_0 and Q8_0 wherever K % 256 != 0: Q4_0 at M = 16, N = 8192,
// K = 2048 7.6 us against 10.6 us on the small-M kernel; Q8_0 at N = 65536
// 54 against 79 us)
hipError_t launch_gemv_slices(int fmt, const float *x, const uint8_t *w, float *y, int M,
                              int N, int K, hipStream_t stream);
// Gated FFN front half over Q4_0, M <= kGemvRowsMax activation rows (f32
// FMAs), and on the matrix cores for up to 16 rows (K % 256 == 0).
hipError_t launch_ffn_gate_up(const float *x, const uint8_t *w_gate, const uint8_t *w_up,
                              float *h, int M, int N, int K, hipStream_t stream);
hipError_t launch_ffn_gate_up_small_m(const float *x, const uint8_t *w_gate,
                                      const uint8_t *w_up, float *h, int M, int N, int K,
                                      hipStream_t stream);
// ... and on the 32-row weight slices (16 gate and 16 up rows), M <= 16.
hipError_t launch_ffn_gate_up_slices(const float *x, const uint8_t *w_gate,
                                     const uint8_t *w_up, float *h, int M, int N, int K,
                                     hipStream_t stream);
// Q4_K GEMV, 1 to 4 activation rows (K % 256 == 0).
hipError_t launch_gemv_q4_k(const float *x, const uint8_t *w, float *y, int M, int N, int K,
                            hipStream_t stream);
hipError_t launch_gemm(int fmt, const float *x, const uint8_t *w, float *y, int M, int N,
                       int K, hipStream_t stream);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// Vector types with 4-byte alignment: weight rows are only guaranteed to be
// dword aligned at pair granularity, and gfx950 vector memory instructions
// need dword alignment only.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

__device__ __forceinline__ float half_lo(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}

__device__ __forceinline__ float half_hi(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Q4_0 nibbles as signed bytes scaled by 16: byte b of the result holds
// 16 * (q - 8) for the low (lo16) or high (hi16) nibble of byte b of v.
// XOR with 8 maps q in 0..15 to the two's-complement nibble of q - 8.
__device__ __forceinline__ uint32_t lo16(uint32_t v)
{
    return ((v << 4) ^ 0x80808080u) & 0xF0F0F0F0u;
}

__device__ __forceinline__ uint32_t hi16(uint32_t v)
{
    return (v ^ 0x88888888u) & 0xF0F0F0F0u;
}

// Signed byte b of v as f32 (one v_cvt_f32_i32 with an SDWA byte select).
__device__ __forceinline__ float sbyte(uint32_t v, int b)
{
    return (float)(int8_t)(v >> (8 * b));
}

// Workgroup barrier that waits only for this wave's LDS operations, not for
// its global loads still in flight (__syncthreads() waits for every
// outstanding memory access first). The scheduling barriers keep the
// compiler from moving work across it.
__device__ __forceinline__ void lds_only_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// The gated FFN's activation, the tanh form of GELU, in f32:
// gelu_tanh(g) = g/2 (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))).
__device__ __forceinline__ float gelu_tanh(float g)
{
    const float c = 0.7978845608028654f;        // sqrt(2 / pi)
    return 0.5f * g * (1.0f + tanhf(c * (g + 0.044715f * g * g * g)));
}

// Orders this wave's LDS writes before its later LDS reads by other lanes
// of the same wave (and reads before later writes). The wave barrier alone
// carries no memory ordering for the compiler; the wavefront-scope fences
// keep it from moving LDS accesses across.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                           ROW_MASK, 0xF, false));
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64)
// with DPP row operations. The total is valid in lane G-1 of each group
// (in every lane of the group when G <= 16). Fixed order: deterministic.
template <int G>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "G must be 2^k <= 64");
    if constexpr (G >= 2) v += dpp_f<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v += dpp_f<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v += dpp_f<0x141, 0xF>(v);  // row_half_mirror
    if constexpr (G >= 16) v += dpp_f<0x140, 0xF>(v); // row_mirror
    if constexpr (G >= 32) v += dpp_f<0x142, 0xA>(v); // row_bcast15 -> rows 1, 3
    if constexpr (G >= 64) v += dpp_f<0x143, 0xC>(v); // row_bcast31 -> rows 2, 3
    return v;
}

}  // namespace qmm
