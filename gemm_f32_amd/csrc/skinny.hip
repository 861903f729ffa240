// Small-problem GEMM: few rows (M <= 64 after the host's normalisation: the skinny,
// memory-bound regime) or too few 128 x 128 tiles to fill the chip.
//
// "How a Matrix Multiply Runs on a GPU", "Shapes that run slowly, and why": with few rows
// the product is bound by reading B once from HBM however well it is tiled, and a large
// block tile leaves most CUs idle.  "A06 - Tiled Matrix Multiply (GEMM)", "The next two
// rungs" (split-K): divide K among workers and combine the partial sums in a second step.
// Design for MI355X:
//
//  * a workgroup owns 16 columns n0 .. n0+15 and 64 rows m0 .. m0+63 of C (fewer when M is
//    smaller: 16 FM rows), so a 16 x 4096 problem spreads over 256 workgroups, one per CU,
//    and a 1000 x 1000 one over 16 x 63;
//  * its 8 wavefronts split K into 8 contiguous ranges (split-K inside the workgroup) and
//    each streams its range of those 16 columns of B and of the FM 16-row strips of A (A is
//    small and stays in L2) straight from global memory into registers -- no LDS staging in
//    the main loop, each lane loads 16 bytes per operand per step (4-byte loads from 4 rows
//    for a row-major FP32 B), a ring of load batches in flight ahead of the matrix
//    instructions (see Depth);
//  * matrix instructions with a 16-row granularity: v_mfma_f32_16x16x32_bf16 (BF16) and
//    v_mfma_f32_16x16x4_f32 (FP32).  Lane l supplies row / column l % 16; the k-assignment
//    of lanes is free as long as A and B use the same one, so lane l takes the 16-byte run
//    of k that starts at 8 (l / 16) (BF16) or 4 (l / 16) (FP32) within each k-step;
//  * the 8 partial products are summed through LDS in a fixed order (wave 0 + 1 + ... + 7):
//    deterministic, no atomics, no workspace;
//  * accumulator layout of a 16 x 16 result: lane l, register r holds row 4 (l / 16) + r,
//    column l % 16.
//
// Requirements (checked by the host): A row-major (k-contiguous); B column-major for BF16,
// either order for FP32.  Any M, N, K; A strips are re-read once per column slab, which is
// cheap only while the problem is small or M is.  Rows past M and columns past N are
// clamped to the last valid one (their products are never stored); the K tail uses
// element-wise loads with zero fill.
#include "common.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr int BN = 16;              // columns per workgroup

// Loads in flight: a wavefront keeps RING batches of CHUNK k-steps in registers, the loads
// of a batch issued RING - 1 batches before its matrix instructions.  Each wavefront has
// few k-steps, so the kernel waits on memory latency unless many loads are in flight:
// 16 k-steps with one 16-row strip of A (25% faster than 8 at 16 x 4096 x 4096; 24
// measured no faster), 8 with more strips (the registers of two wavefronts per SIMD).
template <int FM> struct Depth { static constexpr int RING = 2, CHUNK = 8; };
template <> struct Depth<2> { static constexpr int RING = 2, CHUNK = 4; };
template <> struct Depth<3> { static constexpr int RING = 2, CHUNK = 4; };
template <> struct Depth<4> { static constexpr int RING = 2, CHUNK = 4; };

// ---- per-dtype pieces -------------------------------------------------------------------
// One k-step: BF16 32 k (lane holds 8 consecutive k), FP32 16 k (lane holds 4).
struct Bf16 {
    using Elem = u16;
    using Frag = uint4;
    static constexpr int KSTEP = 32, KL = 8;        // k per step, k per lane
    __device__ static Frag load(const u16* row, int k, int K, bool fast) {
        if (fast) return load16(row + k);
        u16 v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (k + e < K) ? row[k + e] : (u16)0;
        return make_uint4(v[0] | (unsigned)v[1] << 16, v[2] | (unsigned)v[3] << 16,
                          v[4] | (unsigned)v[5] << 16, v[6] | (unsigned)v[7] << 16);
    }
    // B row-major is not handled by this kernel for BF16 (the host routes it elsewhere)
    __device__ static f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

struct F32 {
    using Elem = float;
    using Frag = float4;
    static constexpr int KSTEP = 16, KL = 4;
    __device__ static Frag load(const float* row, int k, int K, bool fast) {
        if (fast) return load16f(row + k);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (k + e < K) ? row[k + e] : 0.f;
        return make_float4(v[0], v[1], v[2], v[3]);
    }
    // B row-major: the 4 k of a lane are 4 rows of B (one column)
    __device__ static Frag load_strided(const float* col, int64_t ld, int k, int K) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (k + e < K) ? col[(int64_t)(k + e) * ld] : 0.f;
        return make_float4(v[0], v[1], v[2], v[3]);
    }
    __device__ static f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
        return c;
    }
};

template <typename D, int FM, int WAVES, bool B_KC>
__global__ __launch_bounds__(64 * WAVES) void k_skinny(Problem p, int klen, int vec_a, int vec_b) {
    using E = typename D::Elem;
    using Frag = typename D::Frag;
    __shared__ f32x4 red[WAVES - 1][FM][64];

    // (row block, column slab): the workgroups one XCD receives cover all row blocks of a
    // run of neighbouring slabs (which share 128-byte lines of a row-major B)
    const int slabs = (p.N + BN - 1) / BN, rblocks = (p.M + 63) / 64;
    int rb, slab;
    tile_coords(blockIdx.x, rblocks, slabs, rblocks, rb, slab);
    const int n0 = slab * BN, m0 = rb * 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int K = p.K;
    const int kbeg = wave * klen, kend = min(K, kbeg + klen);

    // this lane's rows of A (one per 16-row strip) and its column of B, clamped into range
    const E* arow[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f)
        arow[f] = static_cast<const E*>(p.A) + (int64_t)min(m0 + 16 * f + li, p.M - 1) * p.lda;
    const int n = min(n0 + li, p.N - 1);
    const E* bcol = static_cast<const E*>(p.B) + (B_KC ? (int64_t)n * p.ldb : (int64_t)n);

    f32x4 acc[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int CHUNK = Depth<FM>::CHUNK, RING = Depth<FM>::RING, CK = CHUNK * D::KSTEP;
    Frag fa[RING][CHUNK][FM], fb[RING][CHUNK];
    // one batch of CHUNK k-steps; `full` (wavefront-uniform): the whole batch lies inside
    // this wavefront's K range, so 16-byte loads need no bounds checks
    auto load_chunk = [&](int buf, int kc) {
        const bool full = kc + CK <= kend;
        const bool fa_fast = full && vec_a, fb_fast = full && vec_b;
#pragma unroll
        for (int s = 0; s < CHUNK; ++s) {
            const int k = kc + s * D::KSTEP + lq * D::KL;
#pragma unroll
            for (int f = 0; f < FM; ++f) fa[buf][s][f] = D::load(arow[f], k, kend, fa_fast);
            if constexpr (B_KC) fb[buf][s] = D::load(bcol, k, kend, fb_fast);
            else fb[buf][s] = F32::load_strided(reinterpret_cast<const float*>(bcol), p.ldb, k, kend);
        }
    };
    auto compute_chunk = [&](int buf) {
#pragma unroll
        for (int s = 0; s < CHUNK; ++s)
#pragma unroll
            for (int f = 0; f < FM; ++f) acc[f] = D::mma(fa[buf][s][f], fb[buf][s], acc[f]);
    };
    // ring of RING register buffers, unrolled by RING so that buffers are indexed by
    // constants: batch b lives in buffer b % RING
#pragma unroll
    for (int r = 0; r + 1 < RING; ++r)
        if (kbeg + r * CK < kend) load_chunk(r, kbeg + r * CK);
    for (int kc = kbeg; kc < kend; kc += RING * CK) {
#pragma unroll
        for (int r = 0; r < RING; ++r) {
            const int kl = kc + (r + RING - 1) * CK;       // the batch RING - 1 ahead
            if (kl < kend) load_chunk((r + RING - 1) % RING, kl);
            if (kc + r * CK < kend) compute_chunk(r);
        }
    }

    // ---- fixed-order sum of the wavefronts' partial products ----
    if (wave > 0)
#pragma unroll
        for (int f = 0; f < FM; ++f) red[wave - 1][f][lane] = acc[f];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            f32x4 s = acc[f];
#pragma unroll
            for (int w = 0; w < WAVES - 1; ++w) s += red[w][f][lane];
            const int col = n0 + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + 16 * f + 4 * lq + r;
                if (row < p.M && col < p.N) p.C[(int64_t)row * p.ldc + col] = s[r];
            }
        }
    }
}

template <typename D, int WAVES, bool B_KC>
hipError_t launch_d(const Problem& p, const Launch& l) {
    // per-wavefront K range, a multiple of the smallest load batch (4 k-steps)
    constexpr int CK = 4 * D::KSTEP;
    const int per = (p.K + WAVES - 1) / WAVES;
    const int klen = ((per + CK - 1) / CK) * CK;
    const int slabs = (p.N + BN - 1) / BN, rblocks = (p.M + 63) / 64;
    const dim3 grid((unsigned)(slabs * rblocks)), block(64 * WAVES);
    const int va = l.vec_a, vb = l.vec_b;
    const int fm = p.M >= 64 ? 4 : (p.M + 15) / 16;
    if (fm == 1) hipLaunchKernelGGL((k_skinny<D, 1, WAVES, B_KC>), grid, block, 0, l.stream, p, klen, va, vb);
    else if (fm == 2) hipLaunchKernelGGL((k_skinny<D, 2, WAVES, B_KC>), grid, block, 0, l.stream, p, klen, va, vb);
    else if (fm == 3) hipLaunchKernelGGL((k_skinny<D, 3, WAVES, B_KC>), grid, block, 0, l.stream, p, klen, va, vb);
    else hipLaunchKernelGGL((k_skinny<D, 4, WAVES, B_KC>), grid, block, 0, l.stream, p, klen, va, vb);
    return hipGetLastError();
}

}  // namespace

bool skinny_applies(const Problem& p, bool bf16) {
    return p.oa == kRow && (bf16 ? p.ob == kCol : true);
}

hipError_t launch_skinny(const Problem& p, const Launch& l, bool bf16) {
    constexpr int W = kSkinnyWaves;
    if (bf16) return launch_d<Bf16, W, true>(p, l);
    if (p.ob == kCol) return launch_d<F32, W, true>(p, l);
    return launch_d<F32, W, false>(p, l);
}

}  // namespace gemm
