// FP32 ladder, first rungs: one output of C per thread.
//
//  * naive_uncoalesced: the direct kernel of "GEMM" (Part 4 of How to make your models
//    fast), whose thread index walks rows of C, so neighbouring lanes read A and write C
//    one full row apart.
//  * naive: the same arithmetic with the fast thread index along columns of C, so a
//    wavefront reads one broadcast A value and a contiguous run of B per k ("How a Matrix
//    Multiply Runs on a GPU", "Level 0: one thread per output"; "GEMM", "Cost after
//    coalescing").  0.25 flop per byte requested.
//  * tiled: T x T tiles of A and B staged in LDS, T = 32, one output per thread, two
//    barriers per K step, out-of-range tile slots filled with zero and the store guarded
//    ("Level 1: shared-memory tiling"; "A06 - Tiled Matrix Multiply (GEMM)", "The tiled
//    kernel, and what each line is protecting").  T/4 = 8 flop per byte from global
//    memory.
//
// These rungs exist to be measured against each other; the production paths are the
// register-blocked and matrix-core kernels.  All accept either order for A and B; C is
// row-major (the host normalises a column-major C).
#include "common.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

__device__ __forceinline__ float load_a(const Problem& p, int64_t i, int64_t k) {
    return static_cast<const float*>(p.A)[elem_offset(i, k, p.lda, p.oa)];
}
__device__ __forceinline__ float load_b(const Problem& p, int64_t k, int64_t j) {
    return static_cast<const float*>(p.B)[elem_offset(k, j, p.ldb, p.ob)];
}

// 64 x 4 threads.  Uncoalesced: x -> row, y -> column.  Coalesced: x -> column, y -> row.
template <bool COALESCED>
__global__ __launch_bounds__(256) void k_naive(Problem p, int blocks_x) {
    const int bx = blockIdx.x % blocks_x;
    const int by = blockIdx.x / blocks_x;
    int row, col;
    if (COALESCED) {
        col = bx * 64 + threadIdx.x;
        row = by * 4 + threadIdx.y;
    } else {
        row = bx * 64 + threadIdx.x;
        col = by * 4 + threadIdx.y;
    }
    if (row >= p.M || col >= p.N) return;
    float acc = 0.f;
    for (int k = 0; k < p.K; ++k) acc += load_a(p, row, k) * load_b(p, k, col);
    p.C[(int64_t)row * p.ldc + col] = acc;
}

constexpr int T = 32;

// 32 x 32 threads; thread (ty, tx) owns C[row0 + ty][col0 + tx].  Each tile load lets the
// fast thread index run along the operand's contiguous dimension, so a column-major
// operand is read coalesced too and written transposed into the (padded) LDS tile.
template <int OA, int OB>
__global__ __launch_bounds__(1024) void k_tiled(Problem p, int blocks_x) {
    __shared__ float As[T][T + 1];   // As[m][k]
    __shared__ float Bs[T][T + 1];   // Bs[k][n]
    const int tx = threadIdx.x, ty = threadIdx.y;
    const int row0 = (blockIdx.x / blocks_x) * T;
    const int col0 = (blockIdx.x % blocks_x) * T;
    const float* A = static_cast<const float*>(p.A);
    const float* B = static_cast<const float*>(p.B);
    float acc = 0.f;
    for (int k0 = 0; k0 < p.K; k0 += T) {
        if (OA == kRow) {   // contiguous along k
            const int m = row0 + ty, k = k0 + tx;
            As[ty][tx] = (m < p.M && k < p.K) ? A[(int64_t)m * p.lda + k] : 0.f;
        } else {            // contiguous along m
            const int m = row0 + tx, k = k0 + ty;
            As[tx][ty] = (m < p.M && k < p.K) ? A[m + (int64_t)k * p.lda] : 0.f;
        }
        if (OB == kRow) {   // contiguous along n
            const int k = k0 + ty, n = col0 + tx;
            Bs[ty][tx] = (k < p.K && n < p.N) ? B[(int64_t)k * p.ldb + n] : 0.f;
        } else {            // contiguous along k
            const int k = k0 + tx, n = col0 + ty;
            Bs[tx][ty] = (k < p.K && n < p.N) ? B[k + (int64_t)n * p.ldb] : 0.f;
        }
        __syncthreads();    // tile complete before anyone reads it
#pragma unroll
        for (int k = 0; k < T; ++k) acc += As[ty][k] * Bs[k][tx];
        __syncthreads();    // tile consumed before the next K step overwrites it
    }
    const int row = row0 + ty, col = col0 + tx;
    if (row < p.M && col < p.N) p.C[(int64_t)row * p.ldc + col] = acc;
}

}  // namespace

hipError_t launch_naive(const Problem& p, const Launch& l, bool coalesced) {
    const dim3 block(64, 4);
    if (coalesced) {
        const int bx = (p.N + 63) / 64, by = (p.M + 3) / 4;
        hipLaunchKernelGGL(k_naive<true>, dim3((unsigned)bx * by), block, 0, l.stream, p, bx);
    } else {
        const int bx = (p.M + 63) / 64, by = (p.N + 3) / 4;
        hipLaunchKernelGGL(k_naive<false>, dim3((unsigned)bx * by), block, 0, l.stream, p, bx);
    }
    return hipGetLastError();
}

hipError_t launch_tiled(const Problem& p, const Launch& l) {
    const int bx = (p.N + T - 1) / T, by = (p.M + T - 1) / T;
    const dim3 grid((unsigned)bx * by), block(T, T);
    if (p.oa == kRow && p.ob == kRow)
        hipLaunchKernelGGL((k_tiled<kRow, kRow>), grid, block, 0, l.stream, p, bx);
    else if (p.oa == kRow)
        hipLaunchKernelGGL((k_tiled<kRow, kCol>), grid, block, 0, l.stream, p, bx);
    else if (p.ob == kRow)
        hipLaunchKernelGGL((k_tiled<kCol, kRow>), grid, block, 0, l.stream, p, bx);
    else
        hipLaunchKernelGGL((k_tiled<kCol, kCol>), grid, block, 0, l.stream, p, bx);
    return hipGetLastError();
}

}  // namespace gemm
