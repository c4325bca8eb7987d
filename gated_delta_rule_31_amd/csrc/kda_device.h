// Device-side helpers shared by the KDA kernels (gfx950 only).
//
// Matrix-core wrappers: every product in the chunk kernel is a 16x16 output
// tile accumulated in float32 from two operands staged in LDS with the
// reduction index contiguous ("A rows x k" and "B columns x k").  Lane layouts
// (wave64) of the instructions used:
//   16x16x32 (bf16 / f16): lane l holds A[l%16][8*(l/16) .. +8] and B^T likewise
//                          (a 16-wide reduction uses it with the upper four zero, so
//                          accumulation chains never mix instruction shapes);
//   16x16x4  (f32):        lane l holds A[l%16][l/16];
//   result: lane l holds D[4*(l/16) + e][l%16], e = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }

// Sum over the 16 lanes that share lane >> 4 (one DPP row): row rotations by 8, 4, 2
// and 1 stay inside the row, and every lane ends with the row's sum.
template <int ROR>
__device__ __forceinline__ float row_ror(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + ROR, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += row_ror<8>(x);
    x += row_ror<4>(x);
    x += row_ror<2>(x);
    x += row_ror<1>(x);
    return x;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }

// acc += A[16 x kdim] * B[kdim x 16], A stored row-major with stride lda (k contiguous),
// B stored as B^T: 16 rows (output columns) with stride ldb (k contiguous).
// kdim is a multiple of 16 (of 4 for float).  Every lane of the wave must call it.
template <typename T>
__device__ __forceinline__ void mma_tile(f4 &acc, const T *A, int lda, const T *B, int ldb, int kdim,
                                         int lane);

template <>
__device__ __forceinline__ void mma_tile<__bf16>(f4 &acc, const __bf16 *A, int lda, const __bf16 *B,
                                                 int ldb, int kdim, int lane) {
    const __bf16 *a = A + (lane & 15) * lda;
    const __bf16 *b = B + (lane & 15) * ldb;
    int k0 = 0;
    for (; k0 + 32 <= kdim; k0 += 32) {
        bf16x8 av = *reinterpret_cast<const bf16x8 *>(a + k0 + 8 * (lane >> 4));
        bf16x8 bv = *reinterpret_cast<const bf16x8 *>(b + k0 + 8 * (lane >> 4));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
    if (k0 < kdim) {
        // a 16-wide tail uses the same instruction with the upper half of each operand zero
        const __bf16 *pa = a + k0 + 4 * (lane >> 4), *pb = b + k0 + 4 * (lane >> 4);
        const __bf16 z = (__bf16)0.f;
        bf16x8 av = {pa[0], pa[1], pa[2], pa[3], z, z, z, z};
        bf16x8 bv = {pb[0], pb[1], pb[2], pb[3], z, z, z, z};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
}

template <>
__device__ __forceinline__ void mma_tile<_Float16>(f4 &acc, const _Float16 *A, int lda,
                                                   const _Float16 *B, int ldb, int kdim, int lane) {
    const _Float16 *a = A + (lane & 15) * lda;
    const _Float16 *b = B + (lane & 15) * ldb;
    int k0 = 0;
    for (; k0 + 32 <= kdim; k0 += 32) {
        f16x8 av = *reinterpret_cast<const f16x8 *>(a + k0 + 8 * (lane >> 4));
        f16x8 bv = *reinterpret_cast<const f16x8 *>(b + k0 + 8 * (lane >> 4));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
    }
    if (k0 < kdim) {
        const f16x4 pa = *reinterpret_cast<const f16x4 *>(a + k0 + 4 * (lane >> 4));
        const f16x4 pb = *reinterpret_cast<const f16x4 *>(b + k0 + 4 * (lane >> 4));
        f16x8 av = {pa[0], pa[1], pa[2], pa[3], 0, 0, 0, 0};
        f16x8 bv = {pb[0], pb[1], pb[2], pb[3], 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
    }
}

template <>
__device__ __forceinline__ void mma_tile<float>(f4 &acc, const float *A, int lda, const float *B,
                                                int ldb, int kdim, int lane) {
    const float *a = A + (lane & 15) * lda + (lane >> 4);
    const float *b = B + (lane & 15) * ldb + (lane >> 4);
    for (int k0 = 0; k0 < kdim; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k0], b[k0], acc, 0, 0, 0);
}

// The bounded gate applied on the fly: alpha = exp(lower * sigmoid(scale * x)), with
// s2 = scale * log2(e) and l2 = lower * log2(e), on the hardware base-2 exponential and
// reciprocal (a few ulp).  sigmoid(u) = 1 / (1 + 2^(-u log2 e)) needs no sign split: for
// very negative u the exponential overflows to +inf and its reciprocal is the exact limit
// 0; otherwise 1 + 2^(...) >= 1 and the reciprocal keeps its relative accuracy.  alpha
// stays in [e^lower, 1].
__device__ __forceinline__ float fast_bounded_alpha(float x, float s2, float l2) {
    const float r = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-(s2 * x)));
    return __builtin_amdgcn_exp2f(l2 * r);
}

// Load one element of an input tensor as float.
__device__ __forceinline__ float ld_f32(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_f32(const __bf16 *p, int64_t i) { return (float)p[i]; }

__device__ __forceinline__ void st_out(void *out, int is_bf16, int64_t i, float x) {
    if (is_bf16)
        static_cast<__bf16 *>(out)[i] = (__bf16)x;
    else
        static_cast<float *>(out)[i] = x;
}

}  // namespace kda
