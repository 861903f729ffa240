// FP32 GEMM on the matrix cores with direct global->LDS copies: v_mfma_f32_16x16x4_f32.
//
// Same operation as f32_mfma.hip (FP32 inputs, FP32 products and sums on the matrix cores,
// "A06 - Tiled Matrix Multiply (GEMM)", "Matrix cores: MFMA and Tensor Cores"), arranged
// so that the operands never pass through registers on their way to LDS and one 16-byte
// LDS read feeds four matrix instructions:
//
//  * Block tile BM x BN, k-tiles BK = 32 deep, 4 wavefronts in a 2 x 2 grid; a wavefront
//    owns (BM/2) x (BN/2) of C as 16 x 16 blocks (4 x 4 blocks = 64 accumulators per lane
//    at 128 x 128).
//  * Instruction: v_mfma_f32_16x16x4_f32.  Lane l supplies A[i = l % 16][slot l / 16] and
//    B[slot l / 16][j = l % 16]; the result of one block sits in lane l, register v at row
//    4 (l / 16) + v, column l % 16.  The four k-slots may be bound to any four k as long as
//    A and B agree: in k-group t (16 k) at step e (0..3), slot g stands for
//    k = 16 t + 4 g + e, so a lane's four consecutive k are one 16-byte run.
//  * LDS layout of an operand follows its layout in memory, so that the copy is a plain
//    copy ("GEMM Optimization", V3: stage tiles in shared memory, prefetch the next one):
//      - k-contiguous operand (row-major A, column-major B): one LDS row of BK floats
//        (128 bytes, 8 chunks of 16 bytes) per row of the tile, chunk c of row r stored at
//        c ^ s(r) (s(r) = (r mod 8) xor bit 3 of r): the 16 rows read at one logical chunk
//        land on 16 distinct 16-byte bank groups.  A lane's 16-byte read at chunk 4 t + g
//        holds its k-run for steps e = 0..3 of one block;
//      - row-contiguous operand (row-major B, column-major A): one LDS row of BN (BM)
//        floats per k, unpadded (16 lanes read 256 contiguous bytes).  A lane's 16-byte
//        read at k = 16 t + 4 g + e holds 4 consecutive columns n0 + 4 c .. +3 (c = l % 16);
//        element q of it goes to block q, so block q's column c is column n0 + 4 c + q of
//        C.  The epilogue undoes the interleave, and for a row-major B each lane stores 4
//        consecutive columns of C at once.
//  * Copies: global_load_lds_dwordx4, 1 KB per instruction (16 bytes per lane at LDS
//    position 16 l); a lane fetches the global chunk that belongs at its LDS position.
//    Two stages; the copies of k-tile kt + 2 are spread over the second k-group of tile kt
//    and the first of tile kt + 1, one barrier per k-tile (see the main loop).
//  * Tile order from the XCD-aware, group-M scheduler in common.hpp.
//  * Edges: k_f32_dma_edge, the same kernel except at three points, lets tiles overhang M
//    where A is row-major and N where B is column-major (the k-contiguous operands): a
//    copy row past the edge is fetched from the last row that exists (it only reaches rows
//    or columns of C that are not stored), the K tail zero-fills such rows, and stores past
//    M or N are skipped.  Problems of whole tiles run k_f32_dma, whose source is kept as it
//    was measured: the same changes made inside it (as a template flag, or unconditionally)
//    cost 4% at 4096^3 through the compiler's register assignment and scheduling of the
//    k-loop, with the loop's instructions unchanged.
//
// Requirements (checked by the host): K >= BK; M a multiple of the block tile unless A is
// row-major, N unless B is column-major (k_f32_dma: both multiples); a k-contiguous
// operand's copy block (32 rows) below 2^31 bytes.  Rows need element alignment only:
// gfx950's global->LDS copies accept unaligned sources.  A K tail takes one more k-tile
// loaded with bounds checks.  The host runs the rest of a ragged problem (strips along the
// other edges) as separate GEMMs.
#include <type_traits>

#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = 32;                      // k per k-tile (two k-groups of 16)
constexpr int KC_ROW = BK * 4;              // bytes per LDS row of a k-contiguous tile

__device__ __forceinline__ int swz8(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int BM_, int BN_, int WGM_, int WGN_, int S_, bool A_KC_, bool B_KC_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, S = S_, WGM = WGM_, WGN = WGN_;
    static constexpr bool A_KC = A_KC_, B_KC = B_KC_;
    static constexpr int NW = WGM * WGN, THREADS = 64 * NW;  // wavefronts, threads
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 16, FN = WN / 16;        // 16 x 16 blocks per wavefront
    static constexpr int A_BYTES = BM * BK * 4, B_BYTES = BN * BK * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_DMA = A_BYTES / 1024 / NW;       // copies per wavefront per k-tile
    static constexpr int B_DMA = B_BYTES / 1024 / NW;
    static constexpr int DMA = A_DMA + B_DMA;
    // 16-byte fragment reads per k-group: one per block for a k-contiguous operand, one per
    // step and 64 columns for a row-contiguous one
    static constexpr int A_RD = A_KC ? FM : 4 * (FM / 4);
    static constexpr int B_RD = B_KC ? FN : 4 * (FN / 4);
    static constexpr int MFMA_PER_GROUP = 4 * FM * FN;
    static_assert(FM % 4 == 0 && FN % 4 == 0, "wavefront tile must be a multiple of 64");
    static_assert(A_DMA >= 1 && B_DMA >= 1, "tile too small");
    // copy ranges per wavefront: k-contiguous, a multiple of 16 rows (the swizzle of copy j
    // then depends on the parity of j only); row-contiguous, whole copies of 256 / X k-rows
    static_assert(A_KC ? (BM / NW) % 16 == 0 : (BK / NW) % (BM >= 256 ? 1 : 256 / BM) == 0, "A copies");
    static_assert(B_KC ? (BN / NW) % 16 == 0 : (BK / NW) % (BN >= 256 ? 1 : 256 / BN) == 0, "B copies");
};

// One operand's copy plan for one wavefront: a wavefront-uniform base address plus a lane
// offset per copy parity.
//   k-contiguous (rows R = BM or BN, 8 rows per copy, NW wavefronts): wavefront w copies
//     rows w R/NW .. +R/NW-1; copy j covers rows +8 j .. +7, lane l row l / 8, LDS chunk
//     l % 8, logical chunk (l % 8) ^ s(row); s(row) depends on l and on the parity of j
//     only (R / NW is a multiple of 16).
//   row-contiguous (X = R floats per k, 1024 / (4 X) k-rows per copy): wavefront w copies
//     k-rows w BK/NW .. +BK/NW-1; lane l covers k-row l / (X / 4), floats 4 (l % (X / 4)).
template <bool KC, int R, int NW>
struct CopyPlan {
    const char* base;      // the wavefront's first row (k-contiguous) or k-row, at k = 0
    unsigned off[2];       // lane byte offset for even / odd copies
    int64_t step;          // bytes between consecutive copies in global memory
    int64_t kstep;         // bytes per k-tile in global memory

    __device__ void init(const float* p, int64_t ld, int x0, int wave, int lane) {
        if (KC) {
            base = reinterpret_cast<const char*>(p + (int64_t)(x0 + wave * (R / NW)) * ld);
            const int lr = lane / 8;
#pragma unroll
            for (int par = 0; par < 2; ++par) {
                const int c = (lane % 8) ^ swz8(lr + 8 * par);
                off[par] = (unsigned)((lr * ld + c * 4) * 4);
            }
            step = (int64_t)8 * ld * 4;
            kstep = BK * 4;
        } else {
            constexpr int LPR = R / 4;                  // lanes per k-row
            constexpr int RPC = 64 / LPR;               // k-rows per copy
            base = reinterpret_cast<const char*>(p + (int64_t)(wave * (BK / NW)) * ld + x0);
            off[0] = off[1] = (unsigned)(((lane / LPR) * ld + 4 * (lane % LPR)) * 4);
            step = (int64_t)RPC * ld * 4;
            kstep = (int64_t)BK * ld * 4;
        }
    }
};

// SPLIT: K slice blockIdx.y of one problem (slice 0 into C, the others into their slabs)
template <typename C, bool BATCH = false, bool SPLIT = false>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_f32_dma(std::conditional_t<SPLIT, SplitProblem, KArg<BATCH>> p, int tiles_m, int tiles_n, int group_m) {
    constexpr int BM = C::BM, BN = C::BN, S = C::S, FM = C::FM, FN = C::FN;
    constexpr bool A_KC = C::A_KC, B_KC = C::B_KC;
    static_assert(!(BATCH && SPLIT), "a batch is not split");
    __shared__ __align__(16) unsigned char smem[S * C::STAGE];
    if constexpr (SPLIT) p.select(blockIdx.y, 4);

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
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave / C::WGN) * C::WM, wn = (wave % C::WGN) * C::WN;
    const int nk = p.K / BK;
    const float* A = static_cast<const float*>(p.A);
    const float* B = static_cast<const float*>(p.B);

    // ---- copies (whole tiles only: the host keeps partial tiles away from this kernel)
    CopyPlan<A_KC, BM, C::NW> ca;
    CopyPlan<B_KC, BN, C::NW> cb;
    ca.init(A, p.lda, m0, wave, lane);
    cb.init(B, p.ldb, n0, wave, lane);
    // LDS: stage st = [A tile | B tile]; wavefront w's copies fill 1 KB blocks
    // w * X_DMA .. +X_DMA-1 of each tile
    auto issue_one = [&](int j, int kt, int st) {
        unsigned char* s = smem + st * C::STAGE;
        if (j < C::A_DMA) {
            const char* src = ca.base + kt * ca.kstep + j * ca.step + ca.off[j & 1];
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(s + (wave * C::A_DMA + j) * 1024), 16, 0, 0);
        } else {
            const int jb = j - C::A_DMA;
            const char* src = cb.base + kt * cb.kstep + jb * cb.step + cb.off[jb & 1];
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(s + C::A_BYTES + (wave * C::B_DMA + jb) * 1024),
                                             16, 0, 0);
        }
    };

    // ---- fragments of one k-group and the matrix instructions on them ----
    const int li = lane & 15, g = lane >> 4;
    // k-contiguous: block i's row wm + 16 i + li; swizzle depends on li only
    const int a_kc_off = (wm + li) * KC_ROW, b_kc_off = C::A_BYTES + (wn + li) * KC_ROW;
    const int sw = swz8(li);
    // row-contiguous: k-row 16 t + 4 g + e, columns x0 + 64 q + 4 li
    const int a_rc_off = (4 * g * BM + wm + 4 * li) * 4;
    const int b_rc_off = C::A_BYTES + (4 * g * BN + wn + 4 * li) * 4;

    struct Frags { f32x4 a[C::A_RD]; f32x4 b[C::B_RD]; };
    auto read_group = [&](const unsigned char* st, int t, Frags& f) {
        if (A_KC) {
            const int coff = ((4 * t + g) ^ sw) << 4;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                f.a[i] = *reinterpret_cast<const f32x4*>(st + a_kc_off + i * 16 * KC_ROW + coff);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int q = 0; q < FM / 4; ++q)
                    f.a[e * (FM / 4) + q] =
                        *reinterpret_cast<const f32x4*>(st + a_rc_off + ((16 * t + e) * BM + 64 * q) * 4);
        }
        if (B_KC) {
            const int coff = ((4 * t + g) ^ sw) << 4;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                f.b[j] = *reinterpret_cast<const f32x4*>(st + b_kc_off + j * 16 * KC_ROW + coff);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int q = 0; q < FN / 4; ++q)
                    f.b[e * (FN / 4) + q] =
                        *reinterpret_cast<const f32x4*>(st + b_rc_off + ((16 * t + e) * BN + 64 * q) * 4);
        }
    };
    // operand of block i (j) at step e
    auto a_val = [&](const Frags& f, int i, int e) -> float {
        return A_KC ? f.a[i][e] : f.a[e * (FM / 4) + i / 4][i % 4];
    };
    auto b_val = [&](const Frags& f, int j, int e) -> float {
        return B_KC ? f.b[j][e] : f.b[e * (FN / 4) + j / 4][j % 4];
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One k-group: 4 steps x FM x FN matrix instructions on the fragments in f; `slot(n)` is
    // called before the n-th instruction so that the caller can place copies and the reads
    // of the next fragments among them.  Source order is issue order (sched_barrier).
    auto group = [&](const Frags& f, auto slot) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    slot((e * FM + i) * FN + j);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_val(f, i, e), b_val(f, j, e), acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
    };

    // ---- software pipeline over k-tiles, two LDS stages.  Iteration kt multiplies tile kt
    // (stage kt % 2) as two k-groups; group 1's fragments are read under group 0's matrix
    // instructions.  The barrier before group 1 publishes tile kt+1 (every wavefront has
    // waited for its own copies of it) and frees stage kt % 2 (every wavefront's reads of
    // it have completed): during group 1 each wavefront reads group 0 of tile kt+1 and
    // starts the copies of tile kt+2 into the freed stage; they continue through group 0
    // of iteration kt+1 and have until its barrier to land.  So neither the barrier nor the
    // first LDS reads of a tile leave the matrix pipe without work.  Past the end of K the
    // copies repeat the last tile into a stage nobody reads and the fragments read for a
    // tile nk are never used: the loop body has no branch (a branch among the matrix
    // instructions costs more than the extra copies of one k-tile).
    static_assert(S == 2, "two-stage pipeline");
    constexpr int G = C::MFMA_PER_GROUP, W = 2 * G;    // copy window: two k-groups
    constexpr int SP = W / C::DMA;                      // one copy every SP instructions
    static_assert(W % C::DMA == 0, "copies evenly spread over the window");
    // the copy that falls on slot `n` of the window, if any
    auto copies_at = [&](int n, int kt, int st) {
        if (n % SP == 0) issue_one(n / SP, kt, st);
    };
    const int last = nk - 1;
    Frags f[2];
#pragma unroll
    for (int j = 0; j < C::DMA; ++j) issue_one(j, 0, 0);
#pragma unroll
    for (int n = 0; n < G; ++n) copies_at(n, min(1, last), 1);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_group(smem, 0, f[0]);
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        const int k1 = min(kt + 1, last), k2 = min(kt + 2, last);
        group(f[0], [&](int n) {
            copies_at(G + n, k1, st ^ 1);
            if (n == 0) read_group(smem + st * C::STAGE, 1, f[1]);
        });
        // own copies of tile kt+1 landed, own reads of stage st complete; a plain barrier
        // (__syncthreads() would also wait for the copies still in flight)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        group(f[1], [&](int n) {
            copies_at(n, k2, st);
            if (n == 0) read_group(smem + (st ^ 1) * C::STAGE, 0, f[0]);
        });
    }
    // the surplus copies must land before the workgroup's LDS is reused or released
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

    // ---- K tail (K not a multiple of BK): one more k-tile, staged through registers with
    // bounds checks and zero fill into the same LDS positions the copies would fill ----
    if (p.K % BK != 0) {                       // uniform
        __syncthreads();                       // every wavefront is done reading LDS
        const int k0 = nk * BK;
#pragma unroll
        for (int j = 0; j < C::DMA; ++j) {
            const bool is_a = j < C::A_DMA;
            const int jj = is_a ? j : j - C::A_DMA;
            const bool kc = is_a ? A_KC : B_KC;
            const float* src = is_a ? A : B;
            const int64_t ld = is_a ? p.lda : p.ldb;
            const int x0 = is_a ? m0 : n0, R = is_a ? BM : BN;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (kc) {
                // tile row r, logical chunk (lane % 8) ^ s(r): k = k0 + 4 c .. +3
                const int r = wave * (R / C::NW) + 8 * jj + lane / 8;
                const int k = k0 + 4 * ((lane % 8) ^ swz8(r));
                const float* q = src + (int64_t)(x0 + r) * ld + k;
                if (k + 3 < p.K) v = load16f(q);
                else {
                    if (k < p.K) v.x = q[0];
                    if (k + 1 < p.K) v.y = q[1];
                    if (k + 2 < p.K) v.z = q[2];
                }
            } else {
                // k-row k0 + w BK/NW + RPC jj + lane / LPR, columns x0 + 4 (lane % LPR) .. +3
                const int lpr = R / 4, rpc = 64 / lpr;
                const int kr = k0 + wave * (BK / C::NW) + rpc * jj + lane / lpr;
                if (kr < p.K) v = load16f(src + (int64_t)kr * ld + x0 + 4 * (lane % lpr));
            }
            unsigned char* dst = smem + (is_a ? (wave * C::A_DMA + jj) * 1024
                                              : C::A_BYTES + (wave * C::B_DMA + jj) * 1024) + 16 * lane;
            *reinterpret_cast<float4*>(dst) = v;
        }
        __syncthreads();
        read_group(smem, 0, f[0]);
        group(f[0], [&](int n) {
            if (n == 0) read_group(smem, 1, f[1]);
        });
        group(f[1], [](int) {});
    }

    // ---- epilogue: block (i, j), lane l, register v: block row 4 (l / 16) + v, block
    // column l % 16, mapped back through the operand layouts ----
    const bool vec_c = (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int br = 4 * g + v;
            const int row = m0 + wm + (A_KC ? 16 * i + br : 4 * br + i % 4 + 64 * (i / 4));
            float* crow = p.C + (int64_t)row * p.ldc;
            if (B_KC) {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int col = n0 + wn + 16 * j + li;
                    crow[col] = acc[i][j][v];
                }
            } else {
                // columns n0 + wn + 64 q + 4 li + (j % 4): 4 consecutive floats per lane
#pragma unroll
                for (int q = 0; q < FN / 4; ++q) {
                    const int col = n0 + wn + 64 * q + 4 * li;
                    const f32x4 val = {acc[i][4 * q][v], acc[i][4 * q + 1][v], acc[i][4 * q + 2][v],
                                       acc[i][4 * q + 3][v]};
                    if (vec_c) {
                        *reinterpret_cast<f32x4*>(crow + col) = val;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) crow[col + e] = val[e];
                    }
                }
            }
        }
}

// k_f32_dma_edge's plan for one operand: a k-contiguous operand gets one lane offset per
// copy, so that a row past `limit` (M or N) can be replaced by the last row that exists; a
// row-contiguous one is planned as in CopyPlan (its edge is never overhung).
template <bool KC, int R, int NW>
struct EdgeCopyPlan {
    static constexpr int NJ = KC ? R / NW / 8 : 1;
    CopyPlan<KC, R, NW> rc;     // row-contiguous operand
    const char* base;
    unsigned off[NJ];

    __device__ void init(const float* p, int64_t ld, int x0, int limit, int wave, int lane) {
        if (KC) {
            const int row0 = x0 + wave * (R / NW);
            const int first = min(row0, limit - 1);       // a row that exists
            base = reinterpret_cast<const char*>(p + (int64_t)first * ld);
            const int lr = lane / 8;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int c = (lane % 8) ^ swz8(lr + 8 * (j & 1));
                const int row = min(row0 + 8 * j + lr, limit - 1);
                off[j] = (unsigned)(((row - first) * ld + c * 4) * 4);
            }
        } else {
            rc.init(p, ld, x0, wave, lane);
        }
    }
    // source of copy j of k-tile kt
    __device__ const char* src(int j, int kt) const {
        if (KC) return base + kt * (BK * 4) + off[j];
        return rc.base + kt * rc.kstep + j * rc.step + rc.off[0];
    }
};

// EPI: the fused epilogue (both operands k-contiguous), C = act(alpha acc + beta C + bias) stored
// as FP32 or bf16 element by element from the accumulator layout.
template <typename C, bool BATCH = false, bool EPI = false>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_f32_dma_edge(std::conditional_t<EPI, EpiProblem, KArg<BATCH>> p, int tiles_m, int tiles_n, int group_m) {
    constexpr int BM = C::BM, BN = C::BN, S = C::S, FM = C::FM, FN = C::FN;
    constexpr bool A_KC = C::A_KC, B_KC = C::B_KC;
    static_assert(!EPI || (A_KC && B_KC && !BATCH), "the fused epilogue takes k-contiguous operands");
    __shared__ __align__(16) unsigned char smem[S * C::STAGE];

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
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave / C::WGN) * C::WM, wn = (wave % C::WGN) * C::WN;
    const int nk = p.K / BK;
    const float* A = static_cast<const float*>(p.A);
    const float* B = static_cast<const float*>(p.B);

    // ---- copies: rows of a k-contiguous operand past M (N) come from its last row
    EdgeCopyPlan<A_KC, BM, C::NW> ca;
    EdgeCopyPlan<B_KC, BN, C::NW> cb;
    ca.init(A, p.lda, m0, p.M, wave, lane);
    cb.init(B, p.ldb, n0, p.N, wave, lane);
    // LDS: stage st = [A tile | B tile]; wavefront w's copies fill 1 KB blocks
    // w * X_DMA .. +X_DMA-1 of each tile
    auto issue_one = [&](int j, int kt, int st) {
        unsigned char* s = smem + st * C::STAGE;
        if (j < C::A_DMA) {
            const char* src = ca.src(j, kt);
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(s + (wave * C::A_DMA + j) * 1024), 16, 0, 0);
        } else {
            const int jb = j - C::A_DMA;
            const char* src = cb.src(jb, kt);
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(s + C::A_BYTES + (wave * C::B_DMA + jb) * 1024),
                                             16, 0, 0);
        }
    };

    // ---- fragments of one k-group and the matrix instructions on them ----
    const int li = lane & 15, g = lane >> 4;
    // k-contiguous: block i's row wm + 16 i + li; swizzle depends on li only
    const int a_kc_off = (wm + li) * KC_ROW, b_kc_off = C::A_BYTES + (wn + li) * KC_ROW;
    const int sw = swz8(li);
    // row-contiguous: k-row 16 t + 4 g + e, columns x0 + 64 q + 4 li
    const int a_rc_off = (4 * g * BM + wm + 4 * li) * 4;
    const int b_rc_off = C::A_BYTES + (4 * g * BN + wn + 4 * li) * 4;

    struct Frags { f32x4 a[C::A_RD]; f32x4 b[C::B_RD]; };
    auto read_group = [&](const unsigned char* st, int t, Frags& f) {
        if (A_KC) {
            const int coff = ((4 * t + g) ^ sw) << 4;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                f.a[i] = *reinterpret_cast<const f32x4*>(st + a_kc_off + i * 16 * KC_ROW + coff);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int q = 0; q < FM / 4; ++q)
                    f.a[e * (FM / 4) + q] =
                        *reinterpret_cast<const f32x4*>(st + a_rc_off + ((16 * t + e) * BM + 64 * q) * 4);
        }
        if (B_KC) {
            const int coff = ((4 * t + g) ^ sw) << 4;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                f.b[j] = *reinterpret_cast<const f32x4*>(st + b_kc_off + j * 16 * KC_ROW + coff);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int q = 0; q < FN / 4; ++q)
                    f.b[e * (FN / 4) + q] =
                        *reinterpret_cast<const f32x4*>(st + b_rc_off + ((16 * t + e) * BN + 64 * q) * 4);
        }
    };
    // operand of block i (j) at step e
    auto a_val = [&](const Frags& f, int i, int e) -> float {
        return A_KC ? f.a[i][e] : f.a[e * (FM / 4) + i / 4][i % 4];
    };
    auto b_val = [&](const Frags& f, int j, int e) -> float {
        return B_KC ? f.b[j][e] : f.b[e * (FN / 4) + j / 4][j % 4];
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One k-group: 4 steps x FM x FN matrix instructions on the fragments in f; `slot(n)` is
    // called before the n-th instruction so that the caller can place copies and the reads
    // of the next fragments among them.  Source order is issue order (sched_barrier).
    auto group = [&](const Frags& f, auto slot) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    slot((e * FM + i) * FN + j);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_val(f, i, e), b_val(f, j, e), acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
    };

    // ---- software pipeline over k-tiles, two LDS stages.  Iteration kt multiplies tile kt
    // (stage kt % 2) as two k-groups; group 1's fragments are read under group 0's matrix
    // instructions.  The barrier before group 1 publishes tile kt+1 (every wavefront has
    // waited for its own copies of it) and frees stage kt % 2 (every wavefront's reads of
    // it have completed): during group 1 each wavefront reads group 0 of tile kt+1 and
    // starts the copies of tile kt+2 into the freed stage; they continue through group 0
    // of iteration kt+1 and have until its barrier to land.  So neither the barrier nor the
    // first LDS reads of a tile leave the matrix pipe without work.  Past the end of K the
    // copies repeat the last tile into a stage nobody reads and the fragments read for a
    // tile nk are never used: the loop body has no branch (a branch among the matrix
    // instructions costs more than the extra copies of one k-tile).
    static_assert(S == 2, "two-stage pipeline");
    constexpr int G = C::MFMA_PER_GROUP, W = 2 * G;    // copy window: two k-groups
    constexpr int SP = W / C::DMA;                      // one copy every SP instructions
    static_assert(W % C::DMA == 0, "copies evenly spread over the window");
    // the copy that falls on slot `n` of the window, if any
    auto copies_at = [&](int n, int kt, int st) {
        if (n % SP == 0) issue_one(n / SP, kt, st);
    };
    const int last = nk - 1;
    Frags f[2];
#pragma unroll
    for (int j = 0; j < C::DMA; ++j) issue_one(j, 0, 0);
#pragma unroll
    for (int n = 0; n < G; ++n) copies_at(n, min(1, last), 1);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_group(smem, 0, f[0]);
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        const int k1 = min(kt + 1, last), k2 = min(kt + 2, last);
        group(f[0], [&](int n) {
            copies_at(G + n, k1, st ^ 1);
            if (n == 0) read_group(smem + st * C::STAGE, 1, f[1]);
        });
        // own copies of tile kt+1 landed, own reads of stage st complete; a plain barrier
        // (__syncthreads() would also wait for the copies still in flight)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        group(f[1], [&](int n) {
            copies_at(n, k2, st);
            if (n == 0) read_group(smem + (st ^ 1) * C::STAGE, 0, f[0]);
        });
    }
    // the surplus copies must land before the workgroup's LDS is reused or released
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

    // ---- K tail (K not a multiple of BK): one more k-tile, staged through registers with
    // bounds checks and zero fill into the same LDS positions the copies would fill ----
    if (p.K % BK != 0) {                       // uniform
        __syncthreads();                       // every wavefront is done reading LDS
        const int k0 = nk * BK;
#pragma unroll
        for (int j = 0; j < C::DMA; ++j) {
            const bool is_a = j < C::A_DMA;
            const int jj = is_a ? j : j - C::A_DMA;
            const bool kc = is_a ? A_KC : B_KC;
            const float* src = is_a ? A : B;
            const int64_t ld = is_a ? p.lda : p.ldb;
            const int x0 = is_a ? m0 : n0, R = is_a ? BM : BN, limit = is_a ? p.M : p.N;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (kc) {
                // tile row r, logical chunk (lane % 8) ^ s(r): k = k0 + 4 c .. +3; rows past
                // the edge stay zero
                const int r = wave * (R / C::NW) + 8 * jj + lane / 8;
                const int k = k0 + 4 * ((lane % 8) ^ swz8(r));
                const float* q = src + (int64_t)min(x0 + r, limit - 1) * ld + k;
                if (x0 + r >= limit) {
                } else if (k + 3 < p.K) v = load16f(q);
                else {
                    if (k < p.K) v.x = q[0];
                    if (k + 1 < p.K) v.y = q[1];
                    if (k + 2 < p.K) v.z = q[2];
                }
            } else {
                // k-row k0 + w BK/NW + RPC jj + lane / LPR, columns x0 + 4 (lane % LPR) .. +3
                const int lpr = R / 4, rpc = 64 / lpr;
                const int kr = k0 + wave * (BK / C::NW) + rpc * jj + lane / lpr;
                if (kr < p.K) v = load16f(src + (int64_t)kr * ld + x0 + 4 * (lane % lpr));
            }
            unsigned char* dst = smem + (is_a ? (wave * C::A_DMA + jj) * 1024
                                              : C::A_BYTES + (wave * C::B_DMA + jj) * 1024) + 16 * lane;
            *reinterpret_cast<float4*>(dst) = v;
        }
        __syncthreads();
        read_group(smem, 0, f[0]);
        group(f[0], [&](int n) {
            if (n == 0) read_group(smem, 1, f[1]);
        });
        group(f[1], [](int) {});
    }

    // ---- epilogue: block (i, j), lane l, register v: block row 4 (l / 16) + v, block
    // column l % 16, mapped back through the operand layouts; on a tile that overhangs an
    // edge, rows and columns past it are not stored (interior tiles skip the checks) ----
    const bool vec_c = (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0;
    auto store = [&](auto guard) {
        constexpr bool G = decltype(guard)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int br = 4 * g + v;
                const int row = m0 + wm + (A_KC ? 16 * i + br : 4 * br + i % 4 + 64 * (i / 4));
                if (G && row >= p.M) continue;
                float* crow = p.C + (int64_t)row * p.ldc;
                if constexpr (EPI) {
                    // 16 consecutive columns per 16 lanes: one 64-byte run of C per row and j
                    const float brow = p.e.bias != nullptr && p.e.bias_rows ? p.e.bias[row] : 0.f;
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int col = n0 + wn + 16 * j + li;
                        if (G && col >= p.N) continue;
                        const int64_t off = (int64_t)row * p.ldc + col;
                        const float old = p.e.beta != 0.f ? epi_load(p.e, p.C, off) : 0.f;
                        const float b = p.e.bias == nullptr ? 0.f : p.e.bias_rows ? brow : p.e.bias[col];
                        epi_store(p.e, p.C, off, epi_apply(p.e, acc[i][j][v], old, b));
                    }
                } else if (B_KC) {
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int col = n0 + wn + 16 * j + li;
                        if (!G || col < p.N) crow[col] = acc[i][j][v];
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < FN / 4; ++q) {
                        const int col = n0 + wn + 64 * q + 4 * li;
                        const f32x4 val = {acc[i][4 * q][v], acc[i][4 * q + 1][v], acc[i][4 * q + 2][v],
                                           acc[i][4 * q + 3][v]};
                        if (vec_c && (!G || col + 3 < p.N)) {
                            *reinterpret_cast<f32x4*>(crow + col) = val;
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (!G || col + e < p.N) crow[col + e] = val[e];
                        }
                    }
                }
            }
    };
    if (m0 + BM <= p.M && n0 + BN <= p.N) store(std::false_type{});    // uniform
    else store(std::true_type{});
}

template <int BM, int BN, int WGM, int WGN, int S, bool BATCH>
hipError_t launch_cfg(const KArg<BATCH>& p, const Launch& l) {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const dim3 grid((unsigned)tiles_m * tiles_n, 1, BATCH ? l.batch : 1), block(64 * WGM * WGN);
    const bool akc = p.oa == kRow, bkc = p.ob == kCol;
    const int g = l.group_m;
    // tiles may overhang only the k-contiguous operands' edges
    const bool over_m = p.M % BM != 0, over_n = p.N % BN != 0;
    if ((over_m && !akc) || (over_n && !bkc)) return hipErrorInvalidValue;
    if (over_m || over_n) {
        if (akc && bkc)
            hipLaunchKernelGGL((k_f32_dma_edge<Cfg<BM, BN, WGM, WGN, S, true, true>, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g);
        else if (akc)
            hipLaunchKernelGGL((k_f32_dma_edge<Cfg<BM, BN, WGM, WGN, S, true, false>, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g);
        else
            hipLaunchKernelGGL((k_f32_dma_edge<Cfg<BM, BN, WGM, WGN, S, false, true>, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g);
        return hipGetLastError();
    }
    if (akc && bkc)
        hipLaunchKernelGGL((k_f32_dma<Cfg<BM, BN, WGM, WGN, S, true, true>, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g);
    else if (akc)
        hipLaunchKernelGGL((k_f32_dma<Cfg<BM, BN, WGM, WGN, S, true, false>, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g);
    else if (bkc)
        hipLaunchKernelGGL((k_f32_dma<Cfg<BM, BN, WGM, WGN, S, false, true>, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g);
    else
        hipLaunchKernelGGL((k_f32_dma<Cfg<BM, BN, WGM, WGN, S, false, false>, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g);
    return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int S>
hipError_t launch_any(const Problem& p, const Launch& l) {
    if (l.batch > 1) return launch_cfg<BM, BN, WGM, WGN, S, true>(batch_arg(p, l, 4), l);
    return launch_cfg<BM, BN, WGM, WGN, S, false>(p, l);
}

}  // namespace

bool f32_dma_applies(const Problem& p, const Launch& l, int bm, int bn) {
    // a k-contiguous operand's copy block (32 rows at both tile sizes) within 32-bit lane
    // offsets
    const int64_t rows = 32, lim = (int64_t)1 << 31;
    if ((p.oa == kRow && rows * p.lda * 4 >= lim) || (p.ob == kCol && rows * p.ldb * 4 >= lim)) return false;
    // at least one whole tile along each edge (the host plans overhangs and strips)
    return l.vec_a && l.vec_b && p.K >= BK && p.M >= bm && p.N >= bn;
}

// Fused epilogue on either tile, both operands k-contiguous, any M, N (tiles overhang both
// edges) and K >= BK.
hipError_t launch_f32_dma_epi(const EpiProblem& p, const Launch& l, int bm, int bn) {
    if (p.oa != kRow || p.ob != kCol || p.K < BK) return hipErrorInvalidValue;
    const int g = l.group_m;
    if (bm == 256 && bn == 256) {
        const int tm = (p.M + 255) / 256, tn = (p.N + 255) / 256;
        hipLaunchKernelGGL((k_f32_dma_edge<Cfg<256, 256, 4, 2, 2, true, true>, false, true>), dim3(tm * tn),
                           dim3(64 * 8), 0, l.stream, p, tm, tn, g);
    } else if (bm == 128 && bn == 128) {
        const int tm = (p.M + 127) / 128, tn = (p.N + 127) / 128;
        hipLaunchKernelGGL((k_f32_dma_edge<Cfg<128, 128, 2, 2, 2, true, true>, false, true>), dim3(tm * tn),
                           dim3(64 * 4), 0, l.stream, p, tm, tn, g);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Split-K on whole 256 x 256 tiles (M and N multiples of 256): `slices` K slices of s.kslice as
// the grid's second dimension, slices 1 .. S-1 into the slabs at s.part (16-byte aligned), then
// launch_add_slabs adds them to C in slice order.
hipError_t launch_f32_dma_split(const SplitProblem& s, int slices, const Launch& l) {
    if (s.M % 256 != 0 || s.N % 256 != 0) return hipErrorInvalidValue;
    const int tiles_m = s.M / 256, tiles_n = s.N / 256;
    const dim3 grid((unsigned)tiles_m * tiles_n, (unsigned)slices, 1), block(64 * 4 * 2);
    const bool akc = s.oa == kRow, bkc = s.ob == kCol;
    const int g = l.group_m;
    if (akc && bkc)
        hipLaunchKernelGGL((k_f32_dma<Cfg<256, 256, 4, 2, 2, true, true>, false, true>), grid, block, 0, l.stream, s, tiles_m, tiles_n, g);
    else if (akc)
        hipLaunchKernelGGL((k_f32_dma<Cfg<256, 256, 4, 2, 2, true, false>, false, true>), grid, block, 0, l.stream, s, tiles_m, tiles_n, g);
    else if (bkc)
        hipLaunchKernelGGL((k_f32_dma<Cfg<256, 256, 4, 2, 2, false, true>, false, true>), grid, block, 0, l.stream, s, tiles_m, tiles_n, g);
    else
        hipLaunchKernelGGL((k_f32_dma<Cfg<256, 256, 4, 2, 2, false, false>, false, true>), grid, block, 0, l.stream, s, tiles_m, tiles_n, g);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_add_slabs(s.C, s.ldc, s.M, s.N, s.part, slices - 1, l);
}

// Configurations: 256 x 256 with 8 wavefronts of 64 x 128 (2 per SIMD, 128 KB of LDS),
// 128 x 128 with 4 wavefronts of 64 x 64 (two workgroups per CU).
hipError_t launch_f32_dma(const Problem& p, const Launch& l, int bm, int bn) {
    if (bm == 256 && bn == 256) return launch_any<256, 256, 4, 2, 2>(p, l);
    if (bm == 128 && bn == 128) return launch_any<128, 128, 2, 2, 2>(p, l);
    return hipErrorInvalidValue;
}

}  // namespace gemm
