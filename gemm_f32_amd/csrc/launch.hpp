// Kernel launchers, one per kernel family.  Each takes a normalised Problem (row-major C)
// and enqueues on l.stream; the host has already validated shapes and chosen options.
#pragma once

#include "common.hpp"
#include "epilogue.hpp"

namespace gemm {

// FP32 ladder (f32_ladder.hip)
hipError_t launch_naive(const Problem& p, const Launch& l, bool coalesced);
hipError_t launch_tiled(const Problem& p, const Launch& l);
// FP32 register-blocked VALU kernel (f32_regblock.hip)
hipError_t launch_regblock(const Problem& p, const Launch& l);
// FP32 matrix-core kernel (f32_mfma.hip); tile is 128x128 or 64x64 (bm == bn)
hipError_t launch_f32_mfma(const Problem& p, const Launch& l, int bm);
// FP32 matrix-core kernel with direct global->LDS copies (f32_dma.hip); tile 256x256 or
// 128x128.
// Needs aligned operands, K a multiple of 32 and whole tiles (M, N multiples of the tile);
// f32_dma_applies says whether the whole-tile part of a problem may run there.
bool f32_dma_applies(const Problem& p, const Launch& l, int bm, int bn);
hipError_t launch_f32_dma(const Problem& p, const Launch& l, int bm, int bn);
// Split-K on the FP32 direct-copy kernel's whole 256 x 256 tiles (M, N multiples of 256, the
// f32_dma_applies conditions, every slice K >= 32 deep): as launch_bf16_dma_split.
hipError_t launch_f32_dma_split(const SplitProblem& s, int slices, const Launch& l);
// The FP32 direct-copy kernel with the fused epilogue (epilogue.hpp): row-major A, column-major
// B, any M, N, K >= 32, tiles 256x256 or 128x128 overhanging both edges.
hipError_t launch_f32_dma_epi(const EpiProblem& p, const Launch& l, int bm, int bn);
// Input element types of the kernels that take more than one
constexpr int kElemF32 = 0, kElemBf16 = 1, kElemF16 = 2, kElemFp8 = 3;
// BF16 direct-copy kernel (bf16_dma.hip): row-major A, column-major B, any M, N, K >= 64,
// 256x256 or 256x128 tiles; bf16_dma_applies checks the layouts and offset ranges.  With
// f16 the same kernel on IEEE fp16 inputs.
bool bf16_dma_applies(const Problem& p, const Launch& l, int bm, int bn);
hipError_t launch_bf16_dma(const Problem& p, const Launch& l, int bm, int bn, bool f16 = false);
// The same kernel on 8-bit inputs (OCP formats, fmt 0 E4M3, 1 E5M2 per operand): row-major A,
// column-major B, any M, N and K >= 1, 256x256 or 256x128 tiles; fp8_dma_applies checks the
// layouts and offset ranges.
bool fp8_dma_applies(const Problem& p);
hipError_t launch_fp8_dma(const Problem& p, const Launch& l, int bm, int bn, int fmt_a, int fmt_b);
// BF16 matrix-core kernel (bf16_mfma.hip); tile is one of 256x128, 128x128, 64x64;
// f16: fp16 inputs
hipError_t launch_bf16_mfma(const Problem& p, const Launch& l, int bm, int bn, bool f16 = false);
// Small-problem kernel (skinny.hip): 64 x 16 blocks of C with K split over the workgroup;
// row-major A, B column-major for BF16 or either order for FP32.  AUTO uses it for
// M <= kSkinnyMaxM or when 64 x 64 tiles would not fill half the chip.
constexpr int kSkinnyMaxM = 64;
#ifndef GEMM_SKINNY_WAVES
#define GEMM_SKINNY_WAVES 8
#endif
constexpr int kSkinnyWaves = GEMM_SKINNY_WAVES;   // wavefronts splitting K in a workgroup
bool skinny_applies(const Problem& p, bool bf16);
// column blocks of 16 per workgroup (1 or 4) and row strips of 16 per workgroup (1 .. 4)
// for a problem on `cus` CUs
int skinny_blocks(const Problem& p, int cus);
int skinny_strips(const Problem& p, int fn, int cus);
// Split-K across workgroups for the small-problem kernel: `slices` K ranges of `kslice`,
// partial products in a workspace of `bytes` (slices dense M x N FP32 slices), summed in
// slice order by a second kernel.  slices == 1: no split (the problem fills the CUs, or K is
// too short).
struct SkinnySplit {
    int fn = 1, fm = 1, kslice = 0, slices = 1;
    size_t bytes = 0;
};
SkinnySplit skinny_split(const Problem& p, bool bf16, int cus);
// `et`: kElemF32, kElemBf16 or kElemF16.  `sp` and `part` (16-byte aligned, sp->bytes) select
// the split; nullptr: one pass into C
hipError_t launch_skinny(const Problem& p, const Launch& l, int et, int fn, int fm,
                         const SkinnySplit* sp = nullptr, float* part = nullptr);
// Few rows of an FP32 product with row-major A and B (M <= 16, N and ldb even, B 8-byte
// aligned): 32-column blocks over two K halves, C zeroed first and each half's sum added into
// it atomically (exactly two contributions per output, so the result does not depend on their
// order).  _applies: where the host prefers it to the 16-column blocks (K >= kSkinnyHalvesMinK).
constexpr int kSkinnyHalvesMinK = 4096;
bool skinny_halves_ok(const Problem& p);
bool skinny_halves_applies(const Problem& p, int cus);
hipError_t launch_skinny_halves(const Problem& p, const Launch& l);
// The same 32-column blocks over the whole of K with plain stores (no fill, no atomics), where
// the 16-column blocks would take more than one round (N > 16 CUs) and K >= kSkinnyPairsMinK.
constexpr int kSkinnyPairsMinK = 512;
// Also for a column-major B of any input type `et` (two plain 16-column blocks per workgroup).
bool skinny_pairs_applies(const Problem& p, int et, int cus);
hipError_t launch_skinny_pairs(const Problem& p, const Launch& l, int et);
// C = 0 for K == 0 (fill.hip)
hipError_t launch_zero_c(const Problem& p, const Launch& l);
// Fused epilogue (epilogue.hpp): the 16-bit direct-copy kernel with the epilogue in its stores
// (same requirements as launch_bf16_dma; l.vec_c for 16-byte FP32 or 8-byte bf16 row groups),
// and the epilogue of an empty sum for K == 0 (fill.hip)
hipError_t launch_bf16_dma_epi(const EpiProblem& p, const Launch& l, int bm, int bn, bool f16);
hipError_t launch_epi_fill(const EpiProblem& p, const Launch& l);
// Split-K on the 16-bit direct-copy kernel (same requirements as launch_bf16_dma, every slice
// K >= 64): `slices` K slices of s.kslice as a second grid dimension, slices 1 .. S-1 into the
// slabs at s.part, then launch_add_slabs (fill.hip) adds them to C in slice order.
hipError_t launch_bf16_dma_split(const SplitProblem& s, int slices, const Launch& l, int bm, int bn, bool f16);
hipError_t launch_add_slabs(float* C, int64_t ldc, int M, int N, const float* part, int slabs, const Launch& l);

// Block-tile sizes, exported for the host's scheduler choices.
constexpr int kRegblockBM = 128, kRegblockBN = 128;

}  // namespace gemm
