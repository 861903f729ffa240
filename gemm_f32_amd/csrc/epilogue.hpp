// Fused epilogue: C = act(alpha * acc + beta * C + bias), applied to each value on its way from the
// accumulators to C (after the kernel's staging through LDS), with C stored as FP32 or as bf16 ("How a Matrix Multiply Runs on a GPU",
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

// x * Phi(x), Phi the standard normal distribution function written through erf:
// Phi(x) = (1 + erf(x / sqrt 2)) / 2.  erf by Abramowitz and Stegun, Handbook of Mathematical
// Functions, formula 7.1.26: for z >= 0, erf z = 1 - (a1 t + a2 t^2 + ... + a5 t^5) exp(-z^2) with
// t = 1 / (1 + p z), absolute error at most 1.5e-7; erf is odd.  With the hardware's exp2 and
// reciprocal (about 1 ulp each) the result stays within 5e-7 |x| of x Phi(x), far below the
// rounding of a bf16 output and of an FP32 sum of K products; about a third of the
// instructions of the general-purpose erff.
__device__ __forceinline__ float gelu(float x) {
    constexpr float p = 0.3275911f, a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f,
                    a4 = -1.453152027f, a5 = 1.061405429f;
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(p, z, 1.f));
    const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
    const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);   // exp(-z^2)
    const float erf_abs = fmaf(-poly, e, 1.f);
    const float phi2 = x >= 0.f ? 1.f + erf_abs : 1.f - erf_abs;          // 2 Phi(x)
    return 0.5f * x * phi2;
}

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

// Four consecutive previous values of a row of C (off 16-byte aligned for FP32 C, 8-byte for bf16 C).
__device__ __forceinline__ void epi_load4(const Epilogue& e, const void* C, int64_t off, float (&old)[4]) {
    if (e.out_bf16) {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(C) + off);
        old[0] = __uint_as_float(u.x << 16);
        old[1] = __uint_as_float(u.x & 0xffff0000u);
        old[2] = __uint_as_float(u.y << 16);
        old[3] = __uint_as_float(u.y & 0xffff0000u);
    } else {
        const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(C) + off);
        old[0] = f.x;
        old[1] = f.y;
        old[2] = f.z;
        old[3] = f.w;
    }
}

// One output value from its accumulator, C's previous value (read only when beta != 0) and its bias
// (0 without one): the arithmetic of epi_value with the loads done by the caller.
__device__ __forceinline__ float epi_apply(const Epilogue& e, float acc, float old, float bias) {
    float y = e.alpha * acc;
    if (e.beta != 0.f) y += e.beta * old;
    y += bias;
    if (e.act == kActRelu) y = fmaxf(y, 0.f);
    else if (e.act == kActGelu) y = gelu(y);
    return y;
}

// FP32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays a (quiet) NaN (gfx950's
// conversion instruction).
__device__ __forceinline__ uint16_t to_bf16(float y) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(y));
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
