// sa_device.hpp -- device-side building blocks shared by the HIP kernels of
// the sparse-attention prefill (gfx950 / CDNA4 only).
//
// Matrix-core convention used throughout (v_mfma_f32_32x32x16_bf16,
// wave64): for D = A(32x16) * B(16x32) + C, lane l supplies row (l % 32) of
// A and column (l % 32) of B, each as 8 consecutive contraction elements
// starting at 8 * (l / 32); it receives D[8*(v/4) + 4*(l/32) + v%4][l % 32]
// in accumulator register v (v = 0..15).
//
// Attention is computed transposed, S^T = K * Q^T, so that a lane owns one
// query column: row statistics of the softmax stay in the lane (plus its
// partner lane l ^ 32), and the probabilities it holds are already laid out
// as the B operand of O^T = V^T * P^T.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_f16(const f16x8& a, const f16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// fp32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 to_bf16x8(const float* p) {
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = (__bf16)p[t];
    return r;
}

// fp32 -> fp16 with round-to-nearest-even (v_cvt_pk_f16_f32).
__device__ __forceinline__ f16x8 to_f16x8(const float* p) {
    f16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = (_Float16)p[t];
    return r;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

// OCP E4M3 (bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN) ->
// bf16 bits, exactly: normal values 2^-6 .. 448 and subnormals m * 2^-9 are
// all bf16 values.
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t b) {
    const uint32_t s = (b & 0x80u) << 8;
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 15u && m == 7u) return s | 0x7fc0u;                 // NaN
    if (e != 0u) return s | ((e + 120u) << 7) | (m << 4);         // 2^(e-7) (1 + m/8)
    if (m == 0u) return s;                                        // signed zero
    // subnormal m * 2^-9: leading bit p of m, value 2^(p-9) (1 + rest / 2^p)
    const uint32_t p = m >= 4u ? 2u : (m >= 2u ? 1u : 0u);
    return s | ((p + 118u) << 7) | (((m - (1u << p)) << (7u - p)) & 0x7fu);
}

}  // namespace sa
