// Matrix instructions on 16-bit inputs.  The BF16 kernels carry their operand fragments as
// eight 16-bit patterns (bf16x8); the same kernels serve IEEE fp16 inputs, the other
// 16-bit input type of the matrix cores ("Matrix cores: MFMA and Tensor Cores"; same
// layouts, same copies, another instruction), by choosing the instruction here: F16 reads the patterns as fp16 (v_mfma_f32_32x32x16_f16,
// v_mfma_f32_16x16x32_f16), otherwise as bf16.  Products and sums are FP32 either way.
#pragma once

namespace gemm {

typedef __bf16 mma_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 mma_f16x8 __attribute__((ext_vector_type(8)));
typedef float mma_f32x16 __attribute__((ext_vector_type(16)));
typedef float mma_f32x4 __attribute__((ext_vector_type(4)));

template <bool F16>
__device__ __forceinline__ mma_f32x16 mma_32x32x16(mma_bf16x8 a, mma_bf16x8 b, mma_f32x16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(mma_f16x8, a),
                                                       __builtin_bit_cast(mma_f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ mma_f32x4 mma_16x16x32(mma_bf16x8 a, mma_bf16x8 b, mma_f32x4 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mma_f16x8, a),
                                                       __builtin_bit_cast(mma_f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace gemm
