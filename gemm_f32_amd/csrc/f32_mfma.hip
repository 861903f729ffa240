// FP32 GEMM on the matrix cores: v_mfma_f32_32x32x2_f32.
//
// A wavefront of 64 lanes issues one matrix instruction for a 32 x 32 x 2 product with
// FP32 inputs and FP32 accumulation ("A06 - Tiled Matrix Multiply (GEMM)", "Matrix
// cores: MFMA and Tensor Cores").  On MI355X this instruction runs at the same 256
// FLOP/clk/CU as packed FP32 FMA on the vector ALUs, so it reaches the chip's full FP32
// roof (157.3 TFLOP/s) without packed vector math; the register-blocked VALU kernel is
// capped at half of that with unpacked FMAs.
//
// Structure (the same block-tile hierarchy as the pages' register-blocked kernel, with
// the thread's 8 x 8 patch replaced by the wavefront's matrix fragments):
//  * block tile 128 x 128, BK = 16, 256 threads = 4 wavefronts in a 2 x 2 grid, each
//    owning 64 x 64 of C as 2 x 2 fragments of 32 x 32 (64 accumulator registers);
//  * LDS tiles k-major, As[k][m] and Bs[k][n], pitch 132 floats, double-buffered with
//    register-staged prefetch and one barrier per k-tile;
//  * operand fragment for one instruction: lane l supplies A[i = l % 32][k = l / 32] and
//    B[k = l / 32][j = l % 32]; both read consecutive LDS words across lanes;
//  * accumulator layout: lane l, register r holds C[i][j] with j = l % 32 and
//    i = 8 (r / 4) + 4 (l / 32) + r % 4.
#include "common.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

constexpr int BM = kF32MfmaBM, BN = kF32MfmaBN, BK = 16;
constexpr int PITCH = BM + 4;
constexpr int THREADS = 256;
constexpr int LOADS = BM * BK / 4 / THREADS;   // float4 per thread per operand (2)

typedef float f32x16 __attribute__((ext_vector_type(16)));

// float4 number s of this thread's share of the A tile.
//   row-major A: idx -> m = idx / 4, k = 4 * (idx % 4)
//   col-major A: idx -> k = idx / 32, m = 4 * (idx % 32)
template <int OA>
__device__ __forceinline__ float4 load_a(const Problem& p, int m0, int k0, int idx, bool fast) {
    const float* A = static_cast<const float*>(p.A);
    const int m = OA == kRow ? idx >> 2 : (idx & 31) * 4;
    const int k = OA == kRow ? (idx & 3) * 4 : idx >> 5;
    if (fast) return *reinterpret_cast<const float4*>(A + elem_offset(m0 + m, k0 + k, p.lda, OA));
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int mm = m0 + m + (OA == kCol ? e : 0), kk = k0 + k + (OA == kRow ? e : 0);
        v[e] = (mm < p.M && kk < p.K) ? A[elem_offset(mm, kk, p.lda, OA)] : 0.f;
    }
    return make_float4(v[0], v[1], v[2], v[3]);
}

template <int OA>
__device__ __forceinline__ void store_a(float (*As)[PITCH], int idx, float4 v) {
    if (OA == kRow) {
        const int m = idx >> 2, k = (idx & 3) * 4;
        As[k + 0][m] = v.x;
        As[k + 1][m] = v.y;
        As[k + 2][m] = v.z;
        As[k + 3][m] = v.w;
    } else {
        *reinterpret_cast<float4*>(&As[idx >> 5][(idx & 31) * 4]) = v;
    }
}

//   row-major B: idx -> k = idx / 32, n = 4 * (idx % 32)
//   col-major B: idx -> n = idx / 4, k = 4 * (idx % 4)
template <int OB>
__device__ __forceinline__ float4 load_b(const Problem& p, int n0, int k0, int idx, bool fast) {
    const float* B = static_cast<const float*>(p.B);
    const int n = OB == kRow ? (idx & 31) * 4 : idx >> 2;
    const int k = OB == kRow ? idx >> 5 : (idx & 3) * 4;
    if (fast) return *reinterpret_cast<const float4*>(B + elem_offset(k0 + k, n0 + n, p.ldb, OB));
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int nn = n0 + n + (OB == kRow ? e : 0), kk = k0 + k + (OB == kCol ? e : 0);
        v[e] = (nn < p.N && kk < p.K) ? B[elem_offset(kk, nn, p.ldb, OB)] : 0.f;
    }
    return make_float4(v[0], v[1], v[2], v[3]);
}

template <int OB>
__device__ __forceinline__ void store_b(float (*Bs)[PITCH], int idx, float4 v) {
    if (OB == kRow) {
        *reinterpret_cast<float4*>(&Bs[idx >> 5][(idx & 31) * 4]) = v;
    } else {
        const int n = idx >> 2, k = (idx & 3) * 4;
        Bs[k + 0][n] = v.x;
        Bs[k + 1][n] = v.y;
        Bs[k + 2][n] = v.z;
        Bs[k + 3][n] = v.w;
    }
}

template <int OA, int OB>
__global__ __launch_bounds__(THREADS) void k_f32_mfma(Problem p, int tiles_m, int tiles_n,
                                                      int group_m, int vec_a, int vec_b) {
    __shared__ __align__(16) float As[2][BK][PITCH];
    __shared__ __align__(16) float Bs[2][BK][PITCH];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const bool interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);
    const bool fast_a = interior && vec_a, fast_b = interior && vec_b;
    const int nk = (p.K + BK - 1) / BK;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    float4 ra[LOADS], rb[LOADS];
    {
        const bool full = BK <= p.K;
#pragma unroll
        for (int s = 0; s < LOADS; ++s) {
            ra[s] = load_a<OA>(p, m0, 0, t + s * THREADS, fast_a && full);
            rb[s] = load_b<OB>(p, n0, 0, t + s * THREADS, fast_b && full);
        }
#pragma unroll
        for (int s = 0; s < LOADS; ++s) {
            store_a<OA>(As[0], t + s * THREADS, ra[s]);
            store_b<OB>(Bs[0], t + s * THREADS, rb[s]);
        }
    }
    __syncthreads();

    const int li = lane & 31, lk = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int k0 = (kt + 1) * BK;
            const bool full = k0 + BK <= p.K;
#pragma unroll
            for (int s = 0; s < LOADS; ++s) {
                ra[s] = load_a<OA>(p, m0, k0, t + s * THREADS, fast_a && full);
                rb[s] = load_b<OB>(p, n0, k0, t + s * THREADS, fast_b && full);
            }
        }
#pragma unroll
        for (int kk = 0; kk < BK; kk += 2) {
            const float a0 = As[cur][kk + lk][wm + li];
            const float a1 = As[cur][kk + lk][wm + 32 + li];
            const float b0 = Bs[cur][kk + lk][wn + li];
            const float b1 = Bs[cur][kk + lk][wn + 32 + li];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (more) {
#pragma unroll
            for (int s = 0; s < LOADS; ++s) {
                store_a<OA>(As[cur ^ 1], t + s * THREADS, ra[s]);
                store_b<OB>(Bs[cur ^ 1], t + s * THREADS, rb[s]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn + j * 32 + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
                if (interior || (row < p.M && col < p.N))
                    p.C[(int64_t)row * p.ldc + col] = acc[i][j][r];
            }
        }
}

}  // namespace

hipError_t launch_f32_mfma(const Problem& p, const Launch& l) {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const dim3 grid((unsigned)tiles_m * tiles_n), block(THREADS);
    const int va = l.vec_a, vb = l.vec_b;
    if (p.oa == kRow && p.ob == kRow)
        hipLaunchKernelGGL((k_f32_mfma<kRow, kRow>), grid, block, 0, l.stream, p, tiles_m, tiles_n, l.group_m, va, vb);
    else if (p.oa == kRow)
        hipLaunchKernelGGL((k_f32_mfma<kRow, kCol>), grid, block, 0, l.stream, p, tiles_m, tiles_n, l.group_m, va, vb);
    else if (p.ob == kRow)
        hipLaunchKernelGGL((k_f32_mfma<kCol, kRow>), grid, block, 0, l.stream, p, tiles_m, tiles_n, l.group_m, va, vb);
    else
        hipLaunchKernelGGL((k_f32_mfma<kCol, kCol>), grid, block, 0, l.stream, p, tiles_m, tiles_n, l.group_m, va, vb);
    return hipGetLastError();
}

}  // namespace gemm
