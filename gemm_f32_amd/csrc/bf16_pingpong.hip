// BF16-input, FP32-accumulate GEMM, 256 x 256 block tiles, eight wavefronts in ping-pong.
//
// Same operation and LDS layout as bf16_mfma.hip (k-contiguous LDS rows of 16-byte chunks,
// XOR-swizzled; direct global->LDS copies; v_mfma_f32_32x32x16_bf16), arranged for the way
// a CDNA4 CU issues work.  With one wavefront per SIMD, every stall of that wavefront on an
// LDS read, a copy or a barrier leaves the SIMD's matrix pipe idle (measured on gfx950: the
// same k-loop runs at about 60% of its matrix-only rate once the copies and LDS reads are
// added).  Here each SIMD holds two wavefronts, one from each of two groups, and the groups
// alternate between two kinds of phase, separated by workgroup barriers:
//
//   compute phase: 16 matrix instructions back to back on operands already in registers;
//   memory phase:  read the next k-tile's operands from LDS into registers and issue this
//                  wavefront's share of the global->LDS copies of a later k-tile.
//
// While one wavefront of a SIMD computes, the other one does memory work, so the matrix
// pipe is fed from registers and LDS or copy stalls only delay the wavefront that is not
// computing.  The pages' double buffering ("GEMM Optimization", V3; "A06 - Tiled Matrix
// Multiply (GEMM)", "The next two rungs") appears twice: S LDS stages of k-tiles, and the
// operands of the next compute phase loaded during the other group's compute phase.
//
// Wavefront w: group g = w / 4, index q = w % 4 (so each SIMD runs one wavefront of each
// group).  It owns rows 128 g .. +127 and columns 64 q .. +63 of the block tile: 4 x 2
// fragments of 32 x 32, 128 accumulators per lane; two wavefronts share a SIMD's
// registers.  k-tiles are BK = 32 deep (2 k-steps of 16): one compute phase multiplies one
// k-tile, with 12 fragment registers (48 VGPRs) of operands.
//
// Schedule.  k-tile t lives in LDS stage t % S (S = 4 stages of 32 KB).
//   phase 2t:     group 0 computes tile t   | group 1 reads tile t, copies its share of t+S-1
//   phase 2t + 1: group 1 computes tile t   | group 0 reads tile t+1, copies its share of t+S-1
// Stage (t-1) % S is last read in phase 2t-2, so tile t+S-1 may be copied into it from phase
// 2t on.  At the end of phase 2t every wavefront waits for its own copies of tile t+1 (the
// copies of later tiles may stay in flight) and the barrier publishes the tile; group 0
// reads it in phase 2t+1.  Copies have 2S-4 phases to land.  Wavefront w copies rows
// 64 w .. +63 of the stage's [A tile | B tile] (16 rows per 1 KB copy, lane l fetching the
// chunk that belongs at LDS position l).  Past the end of K the copies repeat the last
// k-tile into a stage nobody reads, so no phase has a branch.
//
// Requirements (checked by the host): row-major A and column-major B after the
// column-major-C swap (both k-contiguous), M and N multiples of 256, K a multiple of 32
// (the host runs the whole-tile part of a ragged problem here).
#include "common.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256, BK = 32, S = 4;
constexpr int ROW = BK * 2;                    // LDS row bytes: 4 chunks of 16 bytes
constexpr int A_BYTES = BM * ROW, STAGE = (BM + BN) * ROW;
constexpr int THREADS = 512;
constexpr int FM = 4, FN = 2, SUB = BK / 16;   // fragments per wavefront, k-steps per k-tile
constexpr int RPC = 1024 / ROW;                // rows per 1 KB copy
constexpr int CPT = 64 / RPC;                  // copies per wavefront per k-tile
static_assert((S - 2) * CPT < 64, "vmcnt range");

// chunk c of LDS row r sits at c ^ s(r): the 32 rows read at one logical chunk by a
// fragment read fall on distinct 16-byte bank groups
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_bf16_pingpong(Problem p, int tiles_m, int tiles_n, int group_m) {
    __shared__ __align__(16) unsigned char smem[S * STAGE];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2, q = wave & 3;
    const int nk = p.K / BK;

    // ---- copies: wavefront w fills rows 64 w .. +63 of [A tile | B tile]; copy j covers
    // RPC rows, lane l fetching row l / 4 of them at logical chunk (l % 4) ^ s(row), where
    // s(row) depends on l and the parity of j only
    const bool copies_a = wave < 4;
    const int64_t ld = copies_a ? p.lda : p.ldb;
    const char* gbase = reinterpret_cast<const char*>(
        copies_a ? static_cast<const u16*>(p.A) + (int64_t)(m0 + 64 * q) * p.lda
                 : static_cast<const u16*>(p.B) + (int64_t)(n0 + 64 * q) * p.ldb);
    const int lr = lane >> 2;
    unsigned goff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) goff[par] = (unsigned)((lr * ld + 8 * ((lane & 3) ^ swz(lr + RPC * par))) * 2);
    const int64_t gstep = (int64_t)RPC * ld * 2;
    unsigned char* lbase = smem + (copies_a ? 0 : A_BYTES) + q * 64 * ROW;
    auto copy_tile = [&](int t) {
        const int tc = min(t, nk - 1);
        unsigned char* dst = lbase + (t % S) * STAGE;
        const char* src = gbase + (int64_t)tc * ROW;
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            __builtin_amdgcn_global_load_lds(src + j * gstep + goff[j & 1], (lds_void*)(dst + j * 1024), 16, 0, 0);
    };

    // ---- fragments of one k-tile and the matrix instructions on them ----
    const int l32 = lane & 31, h = lane >> 5, sw = swz(l32);
    const int a_off = (128 * grp + l32) * ROW, b_off = A_BYTES + (64 * q + l32) * ROW;
    bf16x8 fa[SUB][FM], fb[SUB][FN];
    auto read_frags = [&](int t) {
        const unsigned char* st = smem + (t % S) * STAGE;
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            const int coff = ((2 * s + h) ^ sw) << 4;
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[s][i] = *reinterpret_cast<const bf16x8*>(st + a_off + i * 32 * ROW + coff);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[s][j] = *reinterpret_cast<const bf16x8*>(st + b_off + j * 32 * ROW + coff);
        }
    };
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    auto compute = [&]() {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < SUB; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
    };
    auto barrier = [] {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // ---- prologue: tiles 0 .. S-2 in flight; tile 0 published; group 0 holds its operands
#pragma unroll
    for (int t = 0; t + 1 < S; ++t) copy_tile(t);
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"((S - 2) * CPT) : "memory");
    barrier();
    if (grp == 0) {
        read_frags(0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    barrier();

    // ---- ping-pong ----
    for (int t = 0; t < nk; ++t) {
        // phase 2t; at its end tile t+1 must have landed (copies of later tiles may not)
        if (grp == 0) {
            compute();
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"((S - 3) * CPT) : "memory");
        } else {
            read_frags(t);
            copy_tile(t + S - 1);
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"((S - 2) * CPT) : "memory");
        }
        barrier();
        // phase 2t + 1
        if (grp == 1) {
            compute();
        } else {
            read_frags(t + 1);
            copy_tile(t + S - 1);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        barrier();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the surplus copies

    // ---- epilogue: lane l, register r of fragment (i, j) holds
    // C[m0 + 128 g + 32 i + 8 (r / 4) + 4 (l / 32) + r % 4][n0 + 64 q + 32 j + l % 32]
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + 64 * q + 32 * j + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 128 * grp + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                p.C[(int64_t)row * p.ldc + col] = acc[i][j][r];
            }
        }
}

}  // namespace

bool bf16_pingpong_applies(const Problem& p, const Launch&) {
    return p.oa == kRow && p.ob == kCol && p.M % BM == 0 && p.N % BN == 0 && p.K % BK == 0 && p.K >= BK;
}

hipError_t launch_bf16_pingpong(const Problem& p, const Launch& l) {
    const int tiles_m = p.M / BM, tiles_n = p.N / BN;
    hipLaunchKernelGGL(k_bf16_pingpong, dim3((unsigned)tiles_m * tiles_n), dim3(THREADS), 0,
                       l.stream, p, tiles_m, tiles_n, l.group_m);
    return hipGetLastError();
}

}  // namespace gemm
