// Small-problem GEMM: few rows (M <= 64 after the host's normalisation: the skinny,
// memory-bound regime) or too few 128 x 128 tiles to fill the chip.
//
// "How a Matrix Multiply Runs on a GPU", "Shapes that run slowly, and why": with few rows
// the product is bound by reading B once from HBM however well it is tiled, and a large
// block tile leaves most CUs idle.  "A06 - Tiled Matrix Multiply (GEMM)", "The next two
// rungs" (split-K): divide K among workers and combine the partial sums in a second step.
// Design for MI355X:
//
//  * a workgroup owns 16 FN columns n0 .. and 16 FM rows m0 .. of C: FN = 4 (64 columns)
//    when that still gives every CU a workgroup (1000 x 1000: 16 x 16), else FN = 1
//    (16 x 4096: 256 workgroups of 16 x 16); FN = 2 (32 columns, each lane two adjacent
//    columns of a row-major FP32 B) only in the two-halves mode below; FM = 4 (64 rows), or
//    fewer when M is smaller or when fewer rows per block are needed to give every CU one
//    (a 4095 x 1 column: 256 blocks of 16 rows);
//  * its 8 wavefronts split K among themselves (split-K inside the workgroup: batches of
//    k-steps dealt in turn) and each streams its batches of those columns of B and of the
//    FM 16-row strips of A (A stays in L2) straight from global memory into registers -- no LDS staging in
//    the main loop, each lane loads 16 bytes per operand per step (4-byte loads from 4 rows
//    for a row-major FP32 B), a ring of load batches in flight ahead of the matrix
//    instructions (see Depth);
//  * matrix instructions with a 16-row granularity: v_mfma_f32_16x16x32_bf16 (BF16) and
//    v_mfma_f32_16x16x4_f32 (FP32).  Lane l supplies row / column l % 16; the k-assignment
//    of lanes is free as long as A and B use the same one, so lane l takes the 16-byte run
//    of k that starts at 8 (l / 16) (BF16) or 4 (l / 16) (FP32) within each k-step;
//  * the 8 partial products are summed through LDS in a fixed order (wave 0 + 1 + ... + 7):
//    deterministic, no workspace; only the two-halves mode then adds each workgroup's sum
//    into a zeroed C with an atomic add (two contributions per output: still deterministic);
//  * accumulator layout of a 16 x 16 result: lane l, register r holds row 4 (l / 16) + r,
//    column l % 16.
//
// Requirements (checked by the host): A row-major (k-contiguous); B column-major for BF16,
// either order for FP32.  Any M, N, K; A strips are re-read once per column slab, which is
// cheap only while the problem is small or M is.  Rows past M and columns past N are
// clamped to the last valid one (their products are never stored); the K tail uses
// element-wise loads with zero fill.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "mma16.hpp"

namespace gemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;


// Loads in flight: a wavefront keeps RING batches of CHUNK k-steps in registers, the loads
// of a batch issued RING - 1 batches before its matrix instructions: 16 k-steps with one
// 16-row strip of A and one column block, fewer with more strips and blocks (the
// registers of two wavefronts per SIMD).  (At 16 x 4096 x 4096, 8, 16 and 24 k-steps in
// flight measured the same kernel time; at 1000^3 with four blocks, 2 batches of one
// k-step beat 2 of two by 9%.)
template <int FM, int FN> struct Depth {
    static constexpr int RING = 2, CHUNK = FN > 1 ? (FM > 1 ? 1 : 4) : (FM > 1 ? 4 : 8);
};

// ---- per-dtype pieces -------------------------------------------------------------------
// One k-step: BF16 32 k (lane holds 8 consecutive k), FP32 16 k (lane holds 4).
// 16-bit inputs: BF16, or IEEE fp16 with F16 (same loads, another matrix instruction)
template <bool F16>
struct In16 {
    using Elem = u16;
    using Frag = uint4;
    static constexpr int KSTEP = 32, KL = 8;        // k per step, k per lane
    // fast: the caller knows the lane's 8 elements lie inside K.  Otherwise each lane decides:
    // 16 bytes when its elements lie inside K, zero past K, element by element for the one
    // chunk that straddles K (a whole checked batch read element-wise doubled the time of a
    // 4095 x 1 x 1023 product, whose last batch straddles K).
    __device__ static Frag load(const u16* row, int k, int K, bool fast) {
        if (fast || k + 8 <= K) return load16(row + k);
        if (k >= K) return make_uint4(0u, 0u, 0u, 0u);
        u16 v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (k + e < K) ? row[k + e] : (u16)0;
        return make_uint4(v[0] | (unsigned)v[1] << 16, v[2] | (unsigned)v[3] << 16,
                          v[4] | (unsigned)v[5] << 16, v[6] | (unsigned)v[7] << 16);
    }
    // B row-major is not handled by this kernel for 16-bit inputs (the host routes it elsewhere)
    __device__ static f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
        return mma_16x16x32<F16>(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c);
    }
};
using Bf16 = In16<false>;
using F16 = In16<true>;

struct F32 {
    using Elem = float;
    using Frag = float4;
    static constexpr int KSTEP = 16, KL = 4;
    __device__ static Frag load(const float* row, int k, int K, bool fast) {
        if (fast || k + 4 <= K) return load16f(row + k);
        if (k >= K) return make_float4(0.f, 0.f, 0.f, 0.f);
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
    // B row-major, four column blocks: 4 consecutive columns col .. col+3 of row `row`
    __device__ static Frag load_row4(const float* B, int64_t ld, int row, int K, int col, int N, bool fast) {
        if (fast) return load16f(B + (int64_t)row * ld + col);
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (row < K && col + q < N) ? B[(int64_t)row * ld + col + q] : 0.f;
        return make_float4(v[0], v[1], v[2], v[3]);
    }
    // B row-major, whole batch inside the K range: 4 rows of one column through a buffer
    // resource, the row offsets of this lane fixed (voff), the k-step's offset scalar (soff)
    __device__ static Frag load_strided_buf(__amdgpu_buffer_rsrc_t r, const unsigned (&voff)[4], int soff) {
        return make_float4(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff[0], soff, 0)),
                           __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff[1], soff, 0)),
                           __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff[2], soff, 0)),
                           __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff[3], soff, 0)));
    }
    __device__ static f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
        return c;
    }
};

// FN column blocks of 16 per workgroup (1 or 4).  With FN = 4 and a row-major FP32 B, a
// lane's 16-byte load along N holds one k of 4 consecutive columns 4 c .. 4 c + 3, i.e. the
// B operand of 4 matrix instructions: block q's column c is column n0 + 4 c + q of C, and
// the epilogue writes the 4 columns of a lane with one 16-byte store.
template <typename D, int FM, int FN, int WAVES, bool B_KC, bool BATCH = false>
__global__ __launch_bounds__(64 * WAVES)
void k_skinny(KArg<BATCH> p, int vec_a, int vec_b, int vec_c, int bbuf, int kslice, float* part, int accum) {
    if constexpr (BATCH) p.select(blockIdx.z);
    using E = typename D::Elem;
    using Frag = typename D::Frag;
    constexpr bool RC4 = !B_KC && FN == 4;     // row-major FP32 B read 16 bytes along N
    constexpr bool RC2 = !B_KC && FN == 2;     // row-major FP32 B read 8 bytes along N
    constexpr int BNW = 16 * FN;               // columns per workgroup
    constexpr int NB = RC4 ? 4 : FN;           // B fragments per k-step
    static_assert(FN == 1 || FN == 2 || FN == 4, "one, two or four column blocks");
    static_assert(!(RC4 || RC2) || D::KL == 4, "column blocks read along a row-major B: FP32 only");
    __shared__ f32x4 red[WAVES - 1][FM][FN][64];

    // (row block, column slab): the workgroups one XCD receives cover all row blocks of a
    // run of neighbouring slabs (which share 128-byte lines of a row-major B)
    const int slabs = (p.N + BNW - 1) / BNW, rblocks = (p.M + 16 * FM - 1) / (16 * FM);
    int rb, slab;
    tile_coords(blockIdx.x, rblocks, slabs, rblocks, rb, slab);
    const int n0 = slab * BNW, m0 = rb * 16 * FM;
    // the wavefront index is the same in every lane: as a scalar it keeps the K loop bounds
    // and the batch offsets scalar too (uniform branches, no exec-mask loop)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lq = lane >> 4;
    const int K = p.K;
    const bool n_inside = n0 + BNW <= p.N;      // wavefront-uniform
    // Row-major FP32 B read 16 bytes along N (RC4) with N % 4 == 0: in the last column slab each
    // lane's four columns lie wholly inside N or wholly past it, and a lane past it reads the slab's
    // last four valid columns instead (its products reach only columns of C that are never stored),
    // so the slab takes the unchecked loads too.  (Checked loads in that one slab made the whole
    // launch wait on it: 1000^3 FP32 40.8 -> 31.5 us, 1000 x 1000 x 4000 129 -> 95 us.)
    const bool n_groups = RC4 && (p.N & 3) == 0 && p.N >= 4;     // uniform
    const int col4 = n_groups ? min(n0 + 4 * li, p.N - 4) : n0 + 4 * li;

    // this lane's rows of A (one per 16-row strip) and columns of B, clamped into range
    const E* arow[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f)
        arow[f] = static_cast<const E*>(p.A) + (int64_t)min(m0 + 16 * f + li, p.M - 1) * p.lda;
    // column of C that block q's lane li computes: n0 + 16 q + li, or n0 + 2 li + q for a
    // row-major FP32 B read 8 bytes along N (two interleaved blocks)
    auto col_of = [&](int q) { return RC2 ? n0 + 2 * li + q : n0 + 16 * q + li; };
    const E* bcol[FN];
#pragma unroll
    for (int q = 0; q < FN; ++q) {
        const int n = min(col_of(q), p.N - 1);
        bcol[q] = static_cast<const E*>(p.B) + (B_KC ? (int64_t)n * p.ldb : (int64_t)n);
    }
    const float* Bf = reinterpret_cast<const float*>(p.B);
    // row-major FP32 B, one column block: buffer loads for whole batches when byte offsets
    // fit in 31 bits (bbuf, host check), so that the four rows of a k-step cost no address
    // arithmetic (the per-element pointer path issued five times the VALU instructions of
    // the BF16 path at 16 x 4096 x 4096)
    unsigned bvoff[4] = {0, 0, 0, 0};
    const __amdgpu_buffer_rsrc_t rbuf = __builtin_amdgcn_make_buffer_rsrc((void*)Bf, (short)0, 0x7fffffff, 0x00020000);
    if constexpr (!B_KC && FN == 1) {
        const int n = min(n0 + li, p.N - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) bvoff[e] = (unsigned)(((lq * 4 + e) * p.ldb + n) * 4);
    }
    // two column blocks (RC2; the host guarantees an even N and ldb and an 8-byte aligned B):
    // byte offsets of the lane's column pair in its four rows of a k-step, the pair clamped to
    // the last one inside N (a lane past N reads it; its products reach no stored column)
    if constexpr (RC2) {
        const int n = min(n0 + 2 * li, p.N - 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) bvoff[e] = (unsigned)(((lq * 4 + e) * p.ldb + n) * 4);
    }

    f32x4 acc[FM][FN];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int q = 0; q < FN; ++q) acc[f][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int CHUNK = Depth<FM, FN>::CHUNK, RING = Depth<FM, FN>::RING, CK = CHUNK * D::KSTEP;
    // batches are dealt to the wavefronts in turn (wave w takes batches w, w + WAVES, ...), so
    // that the workgroup walks K as one front: at 16 x 4096 x 4096 this beat 8 contiguous
    // K ranges by 7% with one column block and by 2.3x with four (each workgroup's reads of
    // B stay within one contiguous band of rows)
    // split-K across workgroups (gridDim.y slices of `kslice`): this workgroup's slice is
    // k in [kz0, kend); its partial product goes to slice z of the workspace `part`
    const int z = blockIdx.y, kz0 = z * kslice, kend = min(K, kz0 + kslice);
    const int kbeg = kz0 + wave * CK;
    constexpr int SC = WAVES * CK;              // K distance between a wavefront's batches
    Frag fa[RING][CHUNK][FM], fb[RING][CHUNK][NB];
    // one batch of CHUNK k-steps; `full` (wavefront-uniform): the whole batch lies inside
    // K, so 16-byte loads need no bounds checks.  FAST: the caller knows the batch is full and
    // every operand takes its unchecked path (a branch-free batch, see the main loop)
    auto load_chunk = [&](int buf, int kc, auto fast) {
        constexpr bool FAST = decltype(fast)::value;
        const bool full = FAST || kc + CK <= kend;
        const bool fa_fast = FAST || (full && vec_a), fb_fast = FAST || (full && vec_b);
#pragma unroll
        for (int s = 0; s < CHUNK; ++s) {
            const int k = kc + s * D::KSTEP + lq * D::KL;
#pragma unroll
            for (int f = 0; f < FM; ++f) fa[buf][s][f] = D::load(arow[f], k, kend, fa_fast);
            if constexpr (B_KC) {
#pragma unroll
                for (int q = 0; q < FN; ++q) fb[buf][s][q] = D::load(bcol[q], k, kend, fb_fast);
            } else if constexpr (RC4) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    fb[buf][s][e] = F32::load_row4(Bf, p.ldb, k + e, kend, col4, p.N, FAST || (full && (n_inside || n_groups)));
            } else if constexpr (RC2) {
                if (FAST || (bbuf && full)) {
                    // 8-byte loads of the lane's two columns in its four rows: block 0 takes the
                    // first column of each pair, block 1 the second
                    const char* rowp = reinterpret_cast<const char*>(Bf) + (int64_t)(kc + s * D::KSTEP) * p.ldb * 4;
                    float2 v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = *reinterpret_cast<const float2*>(rowp + bvoff[e]);
                    fb[buf][s][0] = make_float4(v[0].x, v[1].x, v[2].x, v[3].x);
                    fb[buf][s][1] = make_float4(v[0].y, v[1].y, v[2].y, v[3].y);
                } else {
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        fb[buf][s][q] = F32::load_strided(reinterpret_cast<const float*>(bcol[q]), p.ldb, k, kend);
                }
            } else if (FAST || (bbuf && full)) {
                // kc is the same in every lane; saying so keeps the offset scalar (no waterfall)
                const int soff = __builtin_amdgcn_readfirstlane((int)((int64_t)(kc + s * D::KSTEP) * p.ldb * 4));
                fb[buf][s][0] = F32::load_strided_buf(rbuf, bvoff, soff);
            } else {
                fb[buf][s][0] = F32::load_strided(reinterpret_cast<const float*>(bcol[0]), p.ldb, k, kend);
            }
        }
    };
    auto compute_chunk = [&](int buf) {
#pragma unroll
        for (int s = 0; s < CHUNK; ++s) {
            if constexpr (RC4) {
                // step e: lane (g, c) holds A[row][k + e] and B[k + e][n0 + 4 c .. +3]
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int f = 0; f < FM; ++f)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[f][q] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[buf][s][f][e], fb[buf][s][e][q],
                                                                             acc[f][q], 0, 0, 0);
            } else {
#pragma unroll
                for (int f = 0; f < FM; ++f)
#pragma unroll
                    for (int q = 0; q < FN; ++q) acc[f][q] = D::mma(fa[buf][s][f], fb[buf][s][q], acc[f][q]);
            }
        }
    };
    // ring of RING register buffers, unrolled by RING so that buffers are indexed by
    // constants: batch b lives in buffer b % RING.  While every batch loaded in a round is
    // full and takes the unchecked loads, the round has no branch, and the wait before a
    // batch's matrix instructions leaves the loads of the batches after it in flight; with a
    // branch between checked and unchecked loads the compiler waits for all of them, the batch
    // ahead included, so each batch's memory latency was exposed in turn.  The rest of K (the
    // last rounds, or operands that need checked loads) runs the general round.
    const bool unchecked = vec_a && (B_KC ? vec_b : RC4 ? (n_inside || n_groups) : bbuf != 0);   // uniform
#pragma unroll
    for (int r = 0; r + 1 < RING; ++r)
        if (kbeg + r * SC < kend) load_chunk(r, kbeg + r * SC, std::false_type{});
    int kc = kbeg;
    if (unchecked) {
        for (; kc + (2 * RING - 2) * SC + CK <= kend; kc += RING * SC) {
#pragma unroll
            for (int r = 0; r < RING; ++r) {
                load_chunk((r + RING - 1) % RING, kc + (r + RING - 1) * SC, std::true_type{});
                compute_chunk(r);
            }
        }
    }
    for (; kc < kend; kc += RING * SC) {
#pragma unroll
        for (int r = 0; r < RING; ++r) {
            const int kl = kc + (r + RING - 1) * SC;       // the batch RING - 1 ahead
            if (kl < kend) load_chunk((r + RING - 1) % RING, kl, std::false_type{});
            if (kc + r * SC < kend) compute_chunk(r);
        }
    }

    // ---- fixed-order sum of the wavefronts' partial products ----
    // accum: C was zeroed and two workgroups (the two K halves) each add their sum into it.
    // Addition of two numbers is commutative, so 0 + x + y is the same whichever comes first:
    // deterministic, unlike three or more atomic contributions.
    auto put = [&](float* dst, float v) {
        if (accum) unsafeAtomicAdd(dst, v);
        else *dst = v;
    };
    if (wave > 0)
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int q = 0; q < FN; ++q) red[wave - 1][f][q][lane] = acc[f][q];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            f32x4 sum[FN];
#pragma unroll
            for (int q = 0; q < FN; ++q) {
                sum[q] = acc[f][q];
#pragma unroll
                for (int w = 0; w < WAVES - 1; ++w) sum[q] += red[w][f][q][lane];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + 16 * f + 4 * lq + r;
                if (row >= p.M) continue;
                float* crow = part ? part + ((int64_t)z * p.M + row) * p.N : p.C + (int64_t)row * p.ldc;
                if constexpr (RC4) {
                    // block q's column li is column n0 + 4 li + q
                    const int col = n0 + 4 * li;
                    if (!accum && (part ? (p.N & 3) == 0 : vec_c) && n_inside) {
                        *reinterpret_cast<f32x4*>(crow + col) = f32x4{sum[0][r], sum[1][r], sum[2][r], sum[3][r]};
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (col + q < p.N) put(crow + col + q, sum[q][r]);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < FN; ++q) {
                        const int col = col_of(q);
                        if (col < p.N) put(crow + col, sum[q][r]);
                    }
                }
            }
        }
    }
}

// K per batch of k-steps of the kernel instance (FM, FN) of dtype D
template <typename D> int batch_k(int fm, int fn) {
    const int chunk = fn > 1 ? (fm > 1 ? 1 : 4) : (fm > 1 ? 4 : 8);
    return chunk * D::KSTEP;
}

template <typename D, int FN, int WAVES, bool B_KC, bool BATCH>
hipError_t launch_d(const KArg<BATCH>& p, const Launch& l, int fm, int kslice, int slices, float* part) {
    const int slabs = (p.N + 16 * FN - 1) / (16 * FN), rblocks = (p.M + 16 * fm - 1) / (16 * fm);
    const dim3 grid((unsigned)(slabs * rblocks), (unsigned)slices, BATCH ? l.batch : 1), block(64 * WAVES);
    const int va = l.vec_a, vb = l.vec_b, vc = l.vec_c;
    // buffer offsets of a row-major B (rows up to K, plus 3 rows of one k-step's lane
    // spread) must fit in 31 bits
    const int bb = !B_KC && (int64_t)(p.K + 4) * p.ldb * 4 + (int64_t)p.N * 4 < ((int64_t)1 << 31);
    if (fm == 1) hipLaunchKernelGGL((k_skinny<D, 1, FN, WAVES, B_KC, BATCH>), grid, block, 0, l.stream, p, va, vb, vc, bb, kslice, part, 0);
    else if (fm == 2) hipLaunchKernelGGL((k_skinny<D, 2, FN, WAVES, B_KC, BATCH>), grid, block, 0, l.stream, p, va, vb, vc, bb, kslice, part, 0);
    else if (fm == 3) hipLaunchKernelGGL((k_skinny<D, 3, FN, WAVES, B_KC, BATCH>), grid, block, 0, l.stream, p, va, vb, vc, bb, kslice, part, 0);
    else hipLaunchKernelGGL((k_skinny<D, 4, FN, WAVES, B_KC, BATCH>), grid, block, 0, l.stream, p, va, vb, vc, bb, kslice, part, 0);
    return hipGetLastError();
}

// Second pass of split-K: C = part[0] + part[1] + ... + part[S-1], in slice order (the same
// sum for every call), four columns per thread.  part holds S dense M x N slices.
__global__ __launch_bounds__(256) void k_sum_slices(const float* part, int S, int M, int N, float* C,
                                                    int64_t ldc, int vec) {
    const int cq = (N + 3) / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * cq) return;
    const int row = (int)(i / cq), col = 4 * (int)(i % cq);
    const int64_t slice = (int64_t)M * N, off = (int64_t)row * N + col;
    float* crow = C + (int64_t)row * ldc;
    if (vec && col + 3 < N) {
        // loads in batches of 8 in flight, added in slice order
        constexpr int G = 8;
        f32x4 acc = *reinterpret_cast<const f32x4*>(part + off);
        int z = 1;
        for (; z + G <= S; z += G) {
            f32x4 v[G];
#pragma unroll
            for (int u = 0; u < G; ++u) v[u] = *reinterpret_cast<const f32x4*>(part + (z + u) * slice + off);
#pragma unroll
            for (int u = 0; u < G; ++u) acc += v[u];
        }
        for (; z < S; ++z) acc += *reinterpret_cast<const f32x4*>(part + z * slice + off);
        *reinterpret_cast<f32x4*>(crow + col) = acc;
    } else {
        for (int e = 0; e < 4 && col + e < N; ++e) {
            float acc = part[off + e];
            for (int z = 1; z < S; ++z) acc += part[z * slice + off + e];
            crow[col + e] = acc;
        }
    }
}

}  // namespace

bool skinny_applies(const Problem& p, bool bf16) {
    return p.oa == kRow && (bf16 ? p.ob == kCol : true);
}

int skinny_blocks(const Problem& p, int cus) {
    // four column blocks per workgroup when that still gives every CU a workgroup
    const int64_t wgs4 = (int64_t)((p.M + 63) / 64) * ((p.N + 63) / 64);
    return wgs4 >= (cus > 0 ? cus : 256) ? 4 : 1;
}

int skinny_strips(const Problem& p, int fn, int cus) {
    // 16-row strips of A per workgroup: as many as M has up to four (64 rows), fewer when
    // 64-row blocks would leave CUs without a workgroup (a 4095 x 1 column: 256 workgroups
    // of 16 rows instead of 64 of 64; B is re-read per block, which is cheap when it is)
    if (p.M < 64) return (p.M + 15) / 16;
    const int64_t slabs = (p.N + 16 * fn - 1) / (16 * fn), c = cus > 0 ? cus : 256;
    for (int fm = 4; fm > 1; fm /= 2)
        if (slabs * ((p.M + 16 * fm - 1) / (16 * fm)) >= c) return fm;
    return 1;
}

SkinnySplit skinny_split(const Problem& p, bool bf16, int cus) {
    SkinnySplit sp;
    // 64 columns per workgroup (four times fewer reads of A per column of C than 16) and as
    // many K slices as it takes to give every CU a workgroup, each slice at least one batch
    // of k-steps per wavefront
    const int64_t c = cus > 0 ? cus : 256;
    // not where the kernel's own blocks make exactly one round (at 16 x 4096 x 4096 its 256 blocks
    // of 16 columns fill the chip, and a split measured slower there: 24.6 us plus 4.7 for the slice
    // sum against 26.4).  Where they leave CUs without a workgroup, or need more than one round, the
    // split's one round of 64-column blocks wins (rocprofv3, operands from HBM: 16 x 8192 x 8192 FP32
    // 92.7 -> 63.7 us, 32 x 8192 x 4096 FP32 60.2 -> 37.4; their plain blocks take two rounds).
    const int fn0 = skinny_blocks(p, cus), fm0 = skinny_strips(p, fn0, cus);
    if ((int64_t)((p.M + 16 * fm0 - 1) / (16 * fm0)) * ((p.N + 16 * fn0 - 1) / (16 * fn0)) == c) return sp;
    const int fn = 4, fm = skinny_strips(p, fn, cus);
    const int64_t wgs = (int64_t)((p.M + 16 * fm - 1) / (16 * fm)) * ((p.N + 63) / 64);
    if (wgs >= c) return sp;
    const int bk = (bf16 ? batch_k<Bf16>(fm, fn) : batch_k<F32>(fm, fn)) * kSkinnyWaves;
    const int64_t want = (c + wgs - 1) / wgs, most = p.K / bk;
    const int s = (int)std::min<int64_t>(want, most);
    if (s < 2) return sp;
    const int kslice = ((p.K + s - 1) / s + bk - 1) / bk * bk;
    sp.fn = fn;
    sp.fm = fm;
    sp.kslice = kslice;
    sp.slices = (p.K + kslice - 1) / kslice;
    sp.bytes = (size_t)sp.slices * p.M * p.N * sizeof(float);
    return sp;
}

namespace {
// The kernel instance for input type, column blocks and B's order.
template <bool BATCH>
hipError_t launch_e(const KArg<BATCH>& p, const Launch& l, int et, int fn, int fm, int kslice, int slices,
                    float* out) {
    constexpr int W = kSkinnyWaves;
    if (fn == 4) {
        if (et == kElemBf16) return launch_d<Bf16, 4, W, true, BATCH>(p, l, fm, kslice, slices, out);
        if (et == kElemF16) return launch_d<F16, 4, W, true, BATCH>(p, l, fm, kslice, slices, out);
        if (p.ob == kCol) return launch_d<F32, 4, W, true, BATCH>(p, l, fm, kslice, slices, out);
        return launch_d<F32, 4, W, false, BATCH>(p, l, fm, kslice, slices, out);
    }
    if (et == kElemBf16) return launch_d<Bf16, 1, W, true, BATCH>(p, l, fm, kslice, slices, out);
    if (et == kElemF16) return launch_d<F16, 1, W, true, BATCH>(p, l, fm, kslice, slices, out);
    if (p.ob == kCol) return launch_d<F32, 1, W, true, BATCH>(p, l, fm, kslice, slices, out);
    return launch_d<F32, 1, W, false, BATCH>(p, l, fm, kslice, slices, out);
}
}  // namespace

// Two K halves of 32-column blocks added into a zeroed C (see launch.hpp).  The blocks of the
// plain kernel on a row-major FP32 B read 64 bytes of each row of B per workgroup and the
// whole of A; 32-column blocks read whole 128-byte lines of B and, over half of K, half of A,
// for the same number of workgroups.  Stand-alone read patterns of 16 x 4096 x 4096 on MI355X
// (B from HBM, A from L2): 16 columns with A 22.3 us, 32 columns over half of K with A 17.3.
int skinny_halves_kslice(const Problem& p) {
    const int bk = batch_k<F32>(1, 2) * kSkinnyWaves;
    return ((p.K + 1) / 2 + bk - 1) / bk * bk;
}

// What the kernel itself needs: one 16-row strip, row-major A and B, column pairs whose 8-byte
// loads are aligned, and a K that splits into exactly two slices (two partial sums per output).
bool skinny_halves_ok(const Problem& p) {
    const int kslice = skinny_halves_kslice(p);
    return p.oa == kRow && p.ob == kRow && p.M >= 1 && p.M <= 16 && p.N >= 2 && (p.N & 1) == 0 &&
           (p.ldb & 1) == 0 && (reinterpret_cast<uintptr_t>(p.B) & 7) == 0 && p.K > 0 &&
           (p.K + kslice - 1) / kslice == 2;
}

bool skinny_halves_applies(const Problem& p, int cus) {
    const int64_t c = cus > 0 ? cus : 256;
    if (!skinny_halves_ok(p) || p.K < kSkinnyHalvesMinK || skinny_blocks(p, cus) != 1) return false;
    // the unchecked loads address B with 32-bit offsets from the k-step's row
    if ((int64_t)(p.K + 4) * p.ldb * 4 + (int64_t)p.N * 4 >= ((int64_t)1 << 31)) return false;
    // as many workgroups as the plain kernel's 16-column blocks, and enough to occupy most CUs
    const int64_t wgs = 2 * ((p.N + 31) / 32);
    return 2 * wgs >= c && wgs <= c;
}

// 32-column blocks over the whole of K (no split, plain stores): where the 16-column blocks would
// take more than one round.  Operands from HBM, against those blocks: 16 x 8192 x 4096 51.5 ->
// 31.7 us, 16 x 6144 x 4096 50.7 -> 31.2, 16 x 5120 x 4096 54.5 -> 31.7, 16 x 8192 x 512 10.0 ->
// 7.7, 16 x 16384 x 4096 (two rounds either way) 58.6 -> 58.8; with exactly one round of
// 16-column blocks (N = 4096) they lost (K = 3072: 18.9 -> 23.7 us).
// A row-major FP32 B read in column pairs needs an even N and ldb and an 8-byte aligned B; a
// column-major B (any input type) takes two plain 16-column blocks per workgroup.
static bool pairs_ok(const Problem& p, int et) {
    if (p.oa != kRow || p.M < 1 || p.M > 16 || p.N < 2) return false;
    if (p.ob == kCol) return true;
    return et == kElemF32 && !(p.N & 1) && !(p.ldb & 1) && (reinterpret_cast<uintptr_t>(p.B) & 7) == 0;
}

bool skinny_pairs_applies(const Problem& p, int et, int cus) {
    const int64_t c = cus > 0 ? cus : 256;
    if (!pairs_ok(p, et) || p.K < kSkinnyPairsMinK || skinny_blocks(p, cus) != 1) return false;
    if (p.ob == kRow && (int64_t)(p.K + 4) * p.ldb * 4 + (int64_t)p.N * 4 >= ((int64_t)1 << 31)) return false;
    return (p.N + 15) / 16 > c;
}

hipError_t launch_skinny_pairs(const Problem& p, const Launch& l, int et) {
    if (!pairs_ok(p, et)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((p.N + 31) / 32), 1u), block(64 * kSkinnyWaves);
    const int va = l.vec_a, vb = l.vec_b, vc = l.vec_c;
    if (p.ob == kRow) {
        const int bb = (int64_t)(p.K + 4) * p.ldb * 4 + (int64_t)p.N * 4 < ((int64_t)1 << 31);
        hipLaunchKernelGGL((k_skinny<F32, 1, 2, kSkinnyWaves, false, false>), grid, block, 0, l.stream, p, va, vb, vc,
                           bb, p.K, nullptr, 0);
    } else if (et == kElemBf16) {
        hipLaunchKernelGGL((k_skinny<Bf16, 1, 2, kSkinnyWaves, true, false>), grid, block, 0, l.stream, p, va, vb, vc,
                           0, p.K, nullptr, 0);
    } else if (et == kElemF16) {
        hipLaunchKernelGGL((k_skinny<F16, 1, 2, kSkinnyWaves, true, false>), grid, block, 0, l.stream, p, va, vb, vc,
                           0, p.K, nullptr, 0);
    } else if (et == kElemF32) {
        hipLaunchKernelGGL((k_skinny<F32, 1, 2, kSkinnyWaves, true, false>), grid, block, 0, l.stream, p, va, vb, vc,
                           0, p.K, nullptr, 0);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_skinny_halves(const Problem& p, const Launch& l) {
    if (!skinny_halves_ok(p)) return hipErrorInvalidValue;
    const hipError_t e = launch_zero_c(p, l);
    if (e != hipSuccess) return e;
    // one 16-row strip: a workgroup per 32-column block and K half (grid y)
    const int bb = (int64_t)(p.K + 4) * p.ldb * 4 + (int64_t)p.N * 4 < ((int64_t)1 << 31);
    hipLaunchKernelGGL((k_skinny<F32, 1, 2, kSkinnyWaves, false, false>), dim3((unsigned)((p.N + 31) / 32), 2u),
                       dim3(64 * kSkinnyWaves), 0, l.stream, p, (int)l.vec_a, (int)l.vec_b, (int)l.vec_c, bb,
                       skinny_halves_kslice(p), nullptr, 1);
    return hipGetLastError();
}

hipError_t launch_skinny(const Problem& p, const Launch& l, int et, int fn, int fm, const SkinnySplit* sp,
                         float* part) {
    if (fm < 1 || fm > 4) return hipErrorInvalidValue;
    const bool split = sp != nullptr && sp->slices > 1 && part != nullptr;
    const int kslice = split ? sp->kslice : p.K, slices = split ? sp->slices : 1;
    float* out = split ? part : nullptr;
    if (et != kElemF32 && et != kElemBf16 && et != kElemF16) return hipErrorInvalidValue;
    if (split && l.batch > 1) return hipErrorInvalidValue;     // one workspace holds one entry's slices
    const hipError_t err = l.batch > 1
        ? launch_e<true>(batch_arg(p, l, et == kElemF32 ? 4 : 2), l, et, fn, fm, kslice, slices, out)
        : launch_e<false>(p, l, et, fn, fm, kslice, slices, out);
    if (err != hipSuccess || !split) return err;
    const int64_t threads = (int64_t)p.M * ((p.N + 3) / 4);
    const int vec = l.vec_c && (p.N & 3) == 0;
    hipLaunchKernelGGL(k_sum_slices, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, l.stream, part,
                       slices, p.M, p.N, p.C, p.ldc, vec);
    return hipGetLastError();
}

}  // namespace gemm
