// FP32 register-blocked GEMM on the vector ALUs.
//
// The "Level 2" design of "How a Matrix Multiply Runs on a GPU" (block tile BM x BN
// swept in BK-deep slices, each thread holding a TM x TN patch of C in registers) with
// BM = BN = 128, BK = 8, TM = TN = 8 and 256 threads, as in "GEMM Optimization" (V2:
// register-level tiling; V3: double buffering) and "GEMM" (Part 4, "Final kernel").
// Per k a thread reads 8 values of A and 8 of B from LDS and does 64 FMAs, which lifts
// the LDS intensity from 1/4 to 2 flop per byte ("GEMM, step by step", Maths).
//
// MI355X specifics:
//  * LDS tiles are k-major, As[k][m] and Bs[k][n], so a thread's operands for one k are
//    contiguous and are read with 16-byte LDS loads.  The A tile is stored transposed
//    from a row-major A, with the row pitch padded to BM + 4 floats: the 64 lanes of a
//    wavefront then write each LDS bank exactly twice, the minimum for 64 four-byte
//    stores ("A06 - Tiled Matrix Multiply (GEMM)", "Layout, padding, and the bank
//    conflicts that remain", and its float4 stretch goal).
//  * A thread's 8 rows are two groups of 4, 64 apart (likewise its 8 columns), so the 16
//    lanes that share a row of threads read 256 contiguous bytes of Bs: no conflicts.
//  * Double buffering: the next k-tile's global loads are issued into registers before
//    the current tile is consumed and written to the other LDS buffer afterwards, one
//    barrier per k-tile.
//  * Loads run along each operand's contiguous dimension (16 bytes per lane when the
//    pointer and leading dimension allow), whichever order the operand has.
//  * Edge tiles and the K tail load element by element with bounds checks and zero
//    fill; stores are guarded ("A06", "Pitfall 1 - The boundary guard that fails
//    silently").
#include "common.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

constexpr int BM = kRegblockBM, BN = kRegblockBN, BK = 8;
constexpr int PITCH = BM + 4;     // LDS row pitch in floats (BM == BN)
constexpr int THREADS = 256;

// One float4 of A per thread per k-tile.
//   row-major A (contiguous in k): thread t -> m = t / 2, k = 4 * (t % 2) .. +3
//   col-major A (contiguous in m): thread t -> k = t / 32, m = 4 * (t % 32) .. +3
template <int OA>
__device__ __forceinline__ float4 load_a(const Problem& p, int m0, int k0, int t, bool fast) {
    const float* A = static_cast<const float*>(p.A);
    const int m = OA == kRow ? t >> 1 : (t & 31) * 4;
    const int k = OA == kRow ? (t & 1) * 4 : t >> 5;
    if (fast) return load16f(A + elem_offset(m0 + m, k0 + k, p.lda, OA));
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int mm = m0 + m + (OA == kCol ? e : 0), kk = k0 + k + (OA == kRow ? e : 0);
        v[e] = (mm < p.M && kk < p.K) ? A[elem_offset(mm, kk, p.lda, OA)] : 0.f;
    }
    return make_float4(v[0], v[1], v[2], v[3]);
}

template <int OA>
__device__ __forceinline__ void store_a(float (*As)[PITCH], int t, float4 v) {
    if (OA == kRow) {
        const int m = t >> 1, k = (t & 1) * 4;
        As[k + 0][m] = v.x;
        As[k + 1][m] = v.y;
        As[k + 2][m] = v.z;
        As[k + 3][m] = v.w;
    } else {
        *reinterpret_cast<float4*>(&As[t >> 5][(t & 31) * 4]) = v;
    }
}

// One float4 of B per thread per k-tile.
//   row-major B (contiguous in n): thread t -> k = t / 32, n = 4 * (t % 32) .. +3
//   col-major B (contiguous in k): thread t -> n = t / 2, k = 4 * (t % 2) .. +3
template <int OB>
__device__ __forceinline__ float4 load_b(const Problem& p, int n0, int k0, int t, bool fast) {
    const float* B = static_cast<const float*>(p.B);
    const int n = OB == kRow ? (t & 31) * 4 : t >> 1;
    const int k = OB == kRow ? t >> 5 : (t & 1) * 4;
    if (fast) return load16f(B + elem_offset(k0 + k, n0 + n, p.ldb, OB));
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int nn = n0 + n + (OB == kRow ? e : 0), kk = k0 + k + (OB == kCol ? e : 0);
        v[e] = (nn < p.N && kk < p.K) ? B[elem_offset(kk, nn, p.ldb, OB)] : 0.f;
    }
    return make_float4(v[0], v[1], v[2], v[3]);
}

template <int OB>
__device__ __forceinline__ void store_b(float (*Bs)[PITCH], int t, float4 v) {
    if (OB == kRow) {
        *reinterpret_cast<float4*>(&Bs[t >> 5][(t & 31) * 4]) = v;
    } else {
        const int n = t >> 1, k = (t & 1) * 4;
        Bs[k + 0][n] = v.x;
        Bs[k + 1][n] = v.y;
        Bs[k + 2][n] = v.z;
        Bs[k + 3][n] = v.w;
    }
}

template <int OA, int OB>
__global__ __launch_bounds__(THREADS) void k_regblock(Problem p, int tiles_m, int tiles_n,
                                                      int group_m, int vec_a, int vec_b,
                                                      int vec_c) {
    __shared__ __align__(16) float As[2][BK][PITCH];
    __shared__ __align__(16) float Bs[2][BK][PITCH];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int t = threadIdx.x;
    const int tx = t & 15, ty = t >> 4;   // 16 x 16 threads, each an 8 x 8 patch
    const bool interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);
    const bool fast_a = interior && vec_a, fast_b = interior && vec_b;
    const int nk = (p.K + BK - 1) / BK;

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    float4 ra = load_a<OA>(p, m0, 0, t, fast_a && BK <= p.K);
    float4 rb = load_b<OB>(p, n0, 0, t, fast_b && BK <= p.K);
    store_a<OA>(As[0], t, ra);
    store_b<OB>(Bs[0], t, rb);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int k0 = (kt + 1) * BK;
            const bool full = k0 + BK <= p.K;
            ra = load_a<OA>(p, m0, k0, t, fast_a && full);
            rb = load_b<OB>(p, n0, k0, t, fast_b && full);
        }
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const float4 a0 = *reinterpret_cast<const float4*>(&As[cur][k][ty * 4]);
            const float4 a1 = *reinterpret_cast<const float4*>(&As[cur][k][64 + ty * 4]);
            const float4 b0 = *reinterpret_cast<const float4*>(&Bs[cur][k][tx * 4]);
            const float4 b1 = *reinterpret_cast<const float4*>(&Bs[cur][k][64 + tx * 4]);
            const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        if (more) {
            store_a<OA>(As[cur ^ 1], t, ra);
            store_b<OB>(Bs[cur ^ 1], t, rb);
        }
        __syncthreads();
    }

    // Epilogue: rows m0 + {ty*4 + i, 64 + ty*4 + i}, columns n0 + {tx*4 + j, 64 + tx*4 + j}.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + i - 4);
        float* crow = p.C + (int64_t)row * p.ldc;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = n0 + h * 64 + tx * 4;
            if (interior && vec_c) {
                *reinterpret_cast<float4*>(crow + col) =
                    make_float4(acc[i][4 * h], acc[i][4 * h + 1], acc[i][4 * h + 2], acc[i][4 * h + 3]);
            } else if (row < p.M) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (col + j < p.N) crow[col + j] = acc[i][4 * h + j];
            }
        }
    }
}

}  // namespace

hipError_t launch_regblock(const Problem& p, const Launch& l) {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const dim3 grid((unsigned)tiles_m * tiles_n), block(THREADS);
    const int va = l.vec_a, vb = l.vec_b, vc = l.vec_c;
    if (p.oa == kRow && p.ob == kRow)
        hipLaunchKernelGGL((k_regblock<kRow, kRow>), grid, block, 0, l.stream, p, tiles_m, tiles_n, l.group_m, va, vb, vc);
    else if (p.oa == kRow)
        hipLaunchKernelGGL((k_regblock<kRow, kCol>), grid, block, 0, l.stream, p, tiles_m, tiles_n, l.group_m, va, vb, vc);
    else if (p.ob == kRow)
        hipLaunchKernelGGL((k_regblock<kCol, kRow>), grid, block, 0, l.stream, p, tiles_m, tiles_n, l.group_m, va, vb, vc);
    else
        hipLaunchKernelGGL((k_regblock<kCol, kCol>), grid, block, 0, l.stream, p, tiles_m, tiles_n, l.group_m, va, vb, vc);
    return hipGetLastError();
}

}  // namespace gemm
