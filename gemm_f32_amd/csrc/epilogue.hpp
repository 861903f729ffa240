// Fused epilogue: C = act(alpha * acc + beta * C + bias), applied to each accumulator before it
// leaves the registers, with C stored as FP32 or as bf16 ("How a Matrix Multiply Runs on a GPU",
// section "Level 2", the epilogue line of its block-tile loop, and section "Operational guidance
// and trade-offs": bias, activation and casts belong in the epilogue; "A06 - Tiled Matrix
// Multiply (GEMM)", section "6. Challenges, Drawbacks & Tradeoffs": fusion is what a hand-written
// kernel adds).
#pragma once

#include "common.hpp"

namespace gemm {

constexpr int kActNone = 0, kActRelu = 1, kActGelu = 2;

struct Epilogue {
    float alpha, beta;
    const float* bias;   // nullptr: no bias
    int bias_rows;       // bias indexed by row of the normalised C (a column-major C's columns)
    int act;             // kActNone, kActRelu, kActGelu
    int out_bf16;        // C holds bf16 bit patterns (2 bytes per element, ldc in elements)
};

// The kernel argument of an epilogue launch: the problem (C as raw memory) plus the epilogue.
struct EpiProblem : Problem {
    Epilogue e;
};
template <> struct ModeArgT<kEpilogue> { using type = EpiProblem; };

// C's previous value at element offset off, as FP32.
__device__ __forceinline__ float epi_load(const Epilogue& e, const void* C, int64_t off) {
    return e.out_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(C)[off] << 16)
                      : static_cast<const float*>(C)[off];
}

// x * Phi(x), Phi the standard normal distribution function written through erf.
__device__ __forceinline__ float gelu(float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); }

// One output value.  beta == 0 does not read C (it may hold anything, NaN included).
__device__ __forceinline__ float epi_value(const Epilogue& e, float acc, const void* C, int64_t off, int row,
                                           int col) {
    float y = e.alpha * acc;
    if (e.beta != 0.f) y += e.beta * epi_load(e, C, off);
    if (e.bias != nullptr) y += e.bias[e.bias_rows ? row : col];
    if (e.act == kActRelu) y = fmaxf(y, 0.f);
    else if (e.act == kActGelu) y = gelu(y);
    return y;
}

// FP32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t to_bf16(float y) {
    const uint32_t u = __float_as_uint(y);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Store one output value at element offset off of C.
__device__ __forceinline__ void epi_store(const Epilogue& e, void* C, int64_t off, float y) {
    if (e.out_bf16) static_cast<uint16_t*>(C)[off] = to_bf16(y);
    else static_cast<float*>(C)[off] = y;
}

// Four consecutive values of a row (16-byte aligned FP32 / 8-byte aligned bf16 C).
__device__ __forceinline__ void epi_store4(const Epilogue& e, void* C, int64_t off, const float (&y)[4]) {
    if (e.out_bf16) {
        const uint32_t lo = to_bf16(y[0]) | ((uint32_t)to_bf16(y[1]) << 16);
        const uint32_t hi = to_bf16(y[2]) | ((uint32_t)to_bf16(y[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + off) = make_uint2(lo, hi);
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(C) + off) = make_float4(y[0], y[1], y[2], y[3]);
    }
}

}  // namespace gemm
