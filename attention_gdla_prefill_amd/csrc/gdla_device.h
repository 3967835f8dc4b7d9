// gdla_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core tile used throughout: v_mfma_f32_16x16x32_bf16.  For a wave of
// 64 lanes, lane l = 16*g + r (r = l % 16, g = l / 16):
//   A operand (16 x 32): lane holds A[r][8g .. 8g+7]
//   B operand (32 x 16): lane holds B[8g .. 8g+7][r]
//   C/D       (16 x 16): lane holds C[4g .. 4g+3][r]
// Scores are formed transposed, S^T = K * Q^T: A = a 16-key slice of K, B =
// the queries, so C holds 4 keys (rows 4g..4g+3) of one query (column r) per
// lane.  A query's scores are spread over the 4 lanes r, r+16, r+32, r+48;
// row reductions are an in-lane reduction plus two lane swaps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D_QK = 192;
constexpr int D_V = 128;
constexpr int GROUP = 4;
constexpr int HEADS = GROUP + 1;      // signal heads of a group + its noise head
constexpr float LOG2E = 1.4426950408889634f;
// Lazy rescale threshold (in log2 units): the running maximum used as the
// softmax reference is only raised when a new score exceeds it by more than
// this, so unnormalised weights stay below 2^8 and fp32 cannot overflow.
constexpr float RESCALE_LOG2 = 8.0f;
// Prefill keeps each row's reference fixed (the row's first visible maximum).
// If one lane's part of a row sum ends a query tile above 2^62 (weights that
// grew far past the reference) or not finite, the workgroup redoes that query
// tile with exact row maxima as references, found by a scores-only pass; then
// every weight is <= 1.  Below the bound, row sums stay under 2^64 and fp32
// (max 2^128) cannot overflow for any realistic V.
constexpr float RESTART_PART_SUM = 0x1p62f;

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max / sum over the 4 lanes that share r (lanes r, r^16, r^32, r^48)
__device__ __forceinline__ float group4_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group4_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// acc + lo + hi of a packed bf16 pair, in fp32 (one v_dot2c_f32_bf16 against (1, 1))
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Transpose a 4 (keys) x 8 (columns) block of bf16: rows[k] holds columns
// 0..7 of key k as 4 packed words; cols[c] receives keys 0..3 of column c as
// 2 packed words.
__device__ __forceinline__ void transpose4x8(const u32x4 rows[4], u32x2 cols[8]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // word w of each row holds columns 2w (low half) and 2w+1 (high half)
        const uint32_t r0 = rows[0][w], r1 = rows[1][w], r2 = rows[2][w], r3 = rows[3][w];
        cols[2 * w][0] = (r0 & 0xffffu) | (r1 << 16);
        cols[2 * w][1] = (r2 & 0xffffu) | (r3 << 16);
        cols[2 * w + 1][0] = (r0 >> 16) | (r1 & 0xffff0000u);
        cols[2 * w + 1][1] = (r2 >> 16) | (r3 & 0xffff0000u);
    }
}

// Position of key r (0..31 within a 32-key slice) in the transposed V rows,
// chosen so that the 8 keys one lane feeds to the B operand of P*V are
// contiguous: lane group g owns keys {4g..4g+3} and {16+4g..16+4g+3}, and
// MFMA k-index 8g+e takes key 16*(e/4) + 4g + e%4.
__device__ __forceinline__ int vt_pos(int r) {
    return 8 * ((r >> 2) & 3) + 4 * (r >> 4) + (r & 3);
}

__device__ __forceinline__ u32x4 ldg16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

}  // namespace gdla
