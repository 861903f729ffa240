// FP32 GEMM on the matrix cores: v_mfma_f32_32x32x2_f32.
//
// A wavefront of 64 lanes issues one matrix instruction for a 32 x 32 x 2 product with
// FP32 inputs and FP32 accumulation ("A06 - Tiled Matrix Multiply (GEMM)", "Matrix
// cores: MFMA and Tensor Cores").  On MI355X this instruction runs at the same 256
// FLOP/clk/CU as packed FP32 FMA on the vector ALUs, so it reaches the chip's full FP32
// roof (157.3 TFLOP/s) without packed vector math; the register-blocked VALU kernel is
// the pages' rung for the same arithmetic.
//
// Structure (the block-tile hierarchy of the pages' register-blocked kernel, with the
// thread's 8 x 8 patch replaced by the wavefront's matrix fragments):
//  * block tile BM x BN, k-tiles BK deep, WGM x WGN wavefronts each owning
//    (BM / WGM) x (BN / WGN) of C as 32 x 32 fragments;
//  * LDS tiles k-major, T[k][x] (x = m for A, n for B), one row of BM (or BN) floats per k
//    plus 28 floats of padding, double-buffered with register-staged prefetch and one
//    barrier per k-tile.  The pitch is 28 (mod 64) words: the two half-wavefronts of a
//    fragment read (rows k and k+1) land 28 banks apart (4 of 32 lanes share a bank), and
//    the transposing stores of a k-contiguous operand (64 lanes: 16 rows x 4 k-groups, the
//    groups 4 rows = 48 (mod 64) banks apart) hit all 64 banks once.  At 128 x 128 x 16 a
//    block then needs 39.9 KB of LDS and four blocks share a CU.  The pages pad by one word ("A06 - Tiled Matrix Multiply (GEMM)",
//    "Layout, padding, and the bank conflicts that remain"); a 64-bank LDS read 64 lanes at
//    a time needs the larger offset.  A plain pitch keeps every LDS address a lane constant
//    plus an immediate, so no registers go to addressing;
//  * optionally (PF) the fragments of k-step s + 1 are read while the matrix instructions
//    of step s run;
//  * operand fragment for one instruction: lane l supplies A[i = l % 32][k = l / 32] and
//    B[k = l / 32][j = l % 32]; accumulator layout: lane l, register r holds C[i][j] with
//    j = l % 32 and i = 8 (r / 4) + 4 (l / 32) + r % 4;
//  * loads along each operand's contiguous dimension, 16 bytes per lane (element alignment
//    suffices on gfx950);
//    edge tiles and the K tail load element by element with bounds checks and zero fill,
//    stores are guarded ("A06", "Pitfall 1 - The boundary guard that fails silently").
#include "common.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int PAD_ = 28>
struct F32Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
    static constexpr int THREADS = 64 * WGM * WGN;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int A_LOADS = BM * BK / 4 / THREADS;   // float4 per thread per k-tile
    static constexpr int B_LOADS = BN * BK / 4 / THREADS;
    static constexpr int PA = BM + PAD_, PB = BN + PAD_;      // LDS row pitches (floats)
    static_assert(A_LOADS >= 1 && B_LOADS >= 1 && FM >= 1 && FN >= 1, "bad tile");
};

// Element access of an operand viewed as R x K ("row" = m for A, n for B) with the
// contiguous dimension along k (KC) or along the row index.
struct Operand {
    const float* p;
    int64_t ld;
    int rows;
};

// float4 number idx of the operand's tile (x0 .. x0+X-1 by k0 .. k0+BK-1).
//   KC: idx -> x = idx / (BK / 4), k = 4 (idx % (BK / 4))   (4 consecutive k)
//   RC: idx -> k = idx / (X / 4),  x = 4 (idx % (X / 4))    (4 consecutive x)
template <int X, int BK, bool KC>
__device__ __forceinline__ float4 load4(const Operand& o, int x0, int k0, int K, int idx, bool fast) {
    const int x = KC ? idx / (BK / 4) : (idx % (X / 4)) * 4;
    const int k = KC ? (idx % (BK / 4)) * 4 : idx / (X / 4);
    if (fast)
        return load16f(o.p + (KC ? (int64_t)(x0 + x) * o.ld + k0 + k
                                                           : (int64_t)(k0 + k) * o.ld + x0 + x));
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int xx = x0 + x + (KC ? 0 : e), kk = k0 + k + (KC ? e : 0);
        v[e] = (xx < o.rows && kk < K) ? o.p[KC ? (int64_t)xx * o.ld + kk : (int64_t)kk * o.ld + xx] : 0.f;
    }
    return make_float4(v[0], v[1], v[2], v[3]);
}

template <int X, int P, int BK, bool KC>
__device__ __forceinline__ void store4(float* T, int idx, float4 v) {
    if (KC) {
        const int x = idx / (BK / 4), k = (idx % (BK / 4)) * 4;
        T[(k + 0) * P + x] = v.x;
        T[(k + 1) * P + x] = v.y;
        T[(k + 2) * P + x] = v.z;
        T[(k + 3) * P + x] = v.w;
    } else {
        const int k = idx / (X / 4), x = (idx % (X / 4)) * 4;
        *reinterpret_cast<float4*>(T + k * P + x) = v;
    }
}

template <int BM, int BN, int BK, int WGM, int WGN, bool PF, int PAD, bool A_KC, bool B_KC, bool BATCH = false>
__global__ __launch_bounds__(64 * WGM * WGN)
void k_f32_mfma(KArg<BATCH> p, int tiles_m, int tiles_n, int group_m, int vec_a, int vec_b) {
    using T = F32Tile<BM, BN, BK, WGM, WGN, PAD>;
    __shared__ __align__(16) float As[2][BK * T::PA];
    __shared__ __align__(16) float Bs[2][BK * T::PB];

    int tm, tn;
    if constexpr (BATCH) {
        int z;
        batch_tile_coords(blockIdx.x, blockIdx.z, gridDim.z, tiles_m, tiles_n, group_m, z, tm, tn);
        p.select(__builtin_amdgcn_readfirstlane(z));     // (uniform: keeps the pointers scalar)
        tm = __builtin_amdgcn_readfirstlane(tm);
        tn = __builtin_amdgcn_readfirstlane(tn);
    } else {
        tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = (wave / WGN) * T::WM, wn = (wave % WGN) * T::WN;
    const bool interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);
    const bool fast_a = interior && vec_a, fast_b = interior && vec_b;
    const int K = p.K;
    const int nk = (K + BK - 1) / BK;
    // A is M x K (KC when row-major); B is seen as N x K (KC when column-major)
    const Operand a{static_cast<const float*>(p.A), p.lda, p.M};
    const Operand b{static_cast<const float*>(p.B), p.ldb, p.N};

    float4 ra[T::A_LOADS], rb[T::B_LOADS];
    auto gload = [&](int k0) {
        const bool full = k0 + BK <= K;
        if (fast_a && full) {
#pragma unroll
            for (int s = 0; s < T::A_LOADS; ++s) ra[s] = load4<BM, BK, A_KC>(a, m0, k0, K, t + s * T::THREADS, true);
        } else {
#pragma unroll
            for (int s = 0; s < T::A_LOADS; ++s) ra[s] = load4<BM, BK, A_KC>(a, m0, k0, K, t + s * T::THREADS, false);
        }
        if (fast_b && full) {
#pragma unroll
            for (int s = 0; s < T::B_LOADS; ++s) rb[s] = load4<BN, BK, B_KC>(b, n0, k0, K, t + s * T::THREADS, true);
        } else {
#pragma unroll
            for (int s = 0; s < T::B_LOADS; ++s) rb[s] = load4<BN, BK, B_KC>(b, n0, k0, K, t + s * T::THREADS, false);
        }
    };
    auto lstore = [&](int stage) {
#pragma unroll
        for (int s = 0; s < T::A_LOADS; ++s) store4<BM, T::PA, BK, A_KC>(As[stage], t + s * T::THREADS, ra[s]);
#pragma unroll
        for (int s = 0; s < T::B_LOADS; ++s) store4<BN, T::PB, BK, B_KC>(Bs[stage], t + s * T::THREADS, rb[s]);
    };

    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int li = lane & 31, lk = lane >> 5;
    // fragments of k-step s (k = 2 s + lk) from one stage
    auto read_frags = [&](const float* as, const float* bs, int s, float (&fa)[T::FM], float (&fb)[T::FN]) {
        const int k = 2 * s + lk;
#pragma unroll
        for (int i = 0; i < T::FM; ++i) fa[i] = as[k * T::PA + wm + 32 * i + li];
#pragma unroll
        for (int j = 0; j < T::FN; ++j) fb[j] = bs[k * T::PB + wn + 32 * j + li];
    };
    // PF: read the fragments of k-step s + 1 before the matrix instructions of step s
    // (more registers, fewer waits); without it occupancy is higher.
    auto compute = [&](int stage) {
        const float* as = As[stage];
        const float* bs = Bs[stage];
        float fa[2][T::FM], fb[2][T::FN];
        if (PF) read_frags(as, bs, 0, fa[0], fb[0]);
#pragma unroll
        for (int s = 0; s < BK / 2; ++s) {
            const int cur = PF ? (s & 1) : 0;
            if (!PF) read_frags(as, bs, s, fa[0], fb[0]);
            else if (s + 1 < BK / 2) read_frags(as, bs, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) gload((kt + 1) * BK);
        compute(kt & 1);
        if (more) lstore((kt + 1) & 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const int col = n0 + wn + j * 32 + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
                if (interior || (row < p.M && col < p.N))
                    p.C[(int64_t)row * p.ldc + col] = acc[i][j][r];
            }
        }
}

template <int BM, int BN, int BK, int WGM, int WGN, bool PF, int PAD, bool BATCH>
hipError_t launch_cfg(const KArg<BATCH>& p, const Launch& l) {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const dim3 grid((unsigned)tiles_m * tiles_n, 1, BATCH ? l.batch : 1), block(64 * WGM * WGN);
    const bool akc = p.oa == kRow, bkc = p.ob == kCol;
    const int va = l.vec_a, vb = l.vec_b, g = l.group_m;
    if (akc && bkc)
        hipLaunchKernelGGL((k_f32_mfma<BM, BN, BK, WGM, WGN, PF, PAD, true, true, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb);
    else if (akc)
        hipLaunchKernelGGL((k_f32_mfma<BM, BN, BK, WGM, WGN, PF, PAD, true, false, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb);
    else if (bkc)
        hipLaunchKernelGGL((k_f32_mfma<BM, BN, BK, WGM, WGN, PF, PAD, false, true, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb);
    else
        hipLaunchKernelGGL((k_f32_mfma<BM, BN, BK, WGM, WGN, PF, PAD, false, false, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WGM, int WGN, bool PF, int PAD = 28>
hipError_t launch_any(const Problem& p, const Launch& l) {
    if (l.batch > 1) return launch_cfg<BM, BN, BK, WGM, WGN, PF, PAD, true>(batch_arg(p, l, 4), l);
    return launch_cfg<BM, BN, BK, WGM, WGN, PF, PAD, false>(p, l);
}

}  // namespace

hipError_t launch_f32_mfma(const Problem& p, const Launch& l, int bm) {
    if (bm == 64) return launch_any<64, 64, 16, 2, 2, false>(p, l);
    return launch_any<128, 128, 16, 2, 2, false>(p, l);
}

}  // namespace gemm
