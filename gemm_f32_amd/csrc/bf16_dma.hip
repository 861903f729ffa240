// BF16-input, FP32-accumulate GEMM with direct global->LDS copies: v_mfma_f32_32x32x16_bf16.
//
// Same operation as bf16_mfma.hip ("GEMM, step by step", Concept; "A06 - Tiled Matrix
// Multiply (GEMM)", "Matrix cores: MFMA and Tensor Cores"), for the layout a BF16 GEMM
// usually has (row-major A, column-major B: both operands contiguous along k), arranged so
// that the k-loop is one branch-free block:
//
//  * Block tile BM x BN, k-tiles BK = 64 (or 32) deep, WGM x WGN wavefronts; at 256 x 256
//    four wavefronts in a 2 x 2 grid own 128 x 128 of C each (4 x 4 fragments of 32 x 32 =
//    256 accumulators per lane), one wavefront per SIMD.
//  * LDS: one row of BK bf16 (128 bytes, 8 chunks of 16 bytes) per row of each tile, chunk
//    c of row r stored at c ^ s(r), s(r) = (r mod 8) xor bit 3 of r, so that the 32 rows
//    read at one logical chunk fall on distinct 16-byte bank groups.  A lane's 16-byte read
//    is one instruction's operand: at k-step s (16 k) lanes 0-31 read chunk 2 s, lanes
//    32-63 chunk 2 s + 1, for A and B alike (the pairing of k between the two operands is
//    what matters, not its order).
//  * Accumulator layout of a 32 x 32 fragment: lane l, register r holds row
//    8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
//  * Copies: global_load_lds_dwordx4, 1 KB per instruction, a lane fetching the chunk that
//    belongs at its LDS position; two stages ("GEMM Optimization", V3), software-pipelined
//    across k-tiles (see the main loop), one barrier per k-tile.  The loop body has no
//    branch: past the end of K the last k-tile is copied again into a stage nobody reads.
//  * Tile order from the XCD-aware, group-M scheduler in common.hpp.
//
// Requirements (checked by the host): row-major A and column-major B after the
// column-major-C swap (element alignment suffices: gfx950's global->LDS copies accept
// unaligned sources), K a multiple of BK, M and N multiples of the block tile (the host runs the whole-tile
// part of a ragged problem here and the edge strips with bf16_mfma.hip).
#include "common.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) void lds_void;

// chunk c of LDS row r is stored at c ^ swz<CH>(r), CH = 16-byte chunks per row: any 16
// consecutive rows read at one logical chunk hit 16 distinct 16-byte bank groups
template <int CH>
__device__ __forceinline__ int swz(int row) {
    if (CH == 8) return (row & 7) ^ ((row >> 3) & 1);
    return ((row >> 1) ^ (row >> 3)) & 3;
}

template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int S_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, S = S_;
    static constexpr int ROW = BK * 2, CH = BK / 8;          // LDS row bytes, chunks per row
    static constexpr int RPC = 1024 / ROW;                   // tile rows per 1 KB copy
    static constexpr int NW = WGM * WGN, THREADS = 64 * NW;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 32, FN = WN / 32;         // 32 x 32 fragments per wavefront
    static constexpr int A_BYTES = BM * ROW, B_BYTES = BN * ROW, STAGE = A_BYTES + B_BYTES;
    static_assert(BK == 32 || BK == 64, "k-tile depth");
    static constexpr int A_DMA = A_BYTES / 1024 / NW, B_DMA = B_BYTES / 1024 / NW;
    static constexpr int DMA = A_DMA + B_DMA;
    static constexpr int SUB = BK / 16;                      // k-steps per k-tile
    static constexpr int MF = FM * FN;                       // matrix instructions per k-step
    static_assert(FM >= 1 && FN >= 1 && A_DMA >= 1 && B_DMA >= 1, "tile too small");
    // a wavefront copies a multiple of 16 rows of each tile, so that the swizzle of copy j
    // depends on the parity of j at most
    static_assert((BM / NW) % 16 == 0 && (BN / NW) % 16 == 0, "copy ranges");
};

template <typename C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_bf16_dma(Problem p, int tiles_m, int tiles_n, int group_m) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, S = C::S, FM = C::FM, FN = C::FN, SUB = C::SUB;
    constexpr int ROW = C::ROW, CH = C::CH;
    __shared__ __align__(16) unsigned char smem[S * C::STAGE];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave / C::WGN) * C::WM, wn = (wave % C::WGN) * C::WN;
    const int nk = p.K / BK;

    // ---- copy plan: wavefront w fills rows w R/NW .. +R/NW-1 of each tile, RPC rows per
    // copy; lane l fetches row l / CH of the copy at logical chunk (l % CH) ^ s(row), which
    // depends on l and on the parity of the copy's first row / RPC only.
    const int lr = lane / CH;
    const char* abase = reinterpret_cast<const char*>(static_cast<const u16*>(p.A) +
                                                      (int64_t)(m0 + wave * (BM / C::NW)) * p.lda);
    const char* bbase = reinterpret_cast<const char*>(static_cast<const u16*>(p.B) +
                                                      (int64_t)(n0 + wave * (BN / C::NW)) * p.ldb);
    unsigned aoff[2], boff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int c = (lane % CH) ^ swz<CH>(lr + C::RPC * par);
        aoff[par] = (unsigned)((lr * p.lda + c * 8) * 2);
        boff[par] = (unsigned)((lr * p.ldb + c * 8) * 2);
    }
    // the swizzle of the wavefront's first copy: its first row is a multiple of 16, which
    // decides the copy parity when a copy spans 16 rows (4 chunks per row)
    if (((wave * (BM / C::NW)) / C::RPC) & 1) { const unsigned t = aoff[0]; aoff[0] = aoff[1]; aoff[1] = t; }
    if (((wave * (BN / C::NW)) / C::RPC) & 1) { const unsigned t = boff[0]; boff[0] = boff[1]; boff[1] = t; }
    const int64_t astep = (int64_t)C::RPC * p.lda * 2, bstep = (int64_t)C::RPC * p.ldb * 2;
    auto issue_one = [&](int j, int kt, int st) {
        unsigned char* s = smem + st * C::STAGE;
        if (j < C::A_DMA) {
            const char* src = abase + kt * (BK * 2) + j * astep + aoff[j & 1];
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(s + (wave * C::A_DMA + j) * 1024), 16, 0, 0);
        } else {
            const int jb = j - C::A_DMA;
            const char* src = bbase + kt * (BK * 2) + jb * bstep + boff[jb & 1];
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(s + C::A_BYTES + (wave * C::B_DMA + jb) * 1024),
                                             16, 0, 0);
        }
    };

    // ---- fragments and matrix instructions ----
    const int l32 = lane & 31, h = lane >> 5, sw = swz<CH>(l32);
    const int a_off = (wm + l32) * ROW, b_off = C::A_BYTES + (wn + l32) * ROW;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    struct Frags { bf16x8 a[FM]; bf16x8 b[FN]; };
    auto read_step = [&](const unsigned char* st, int s, Frags& f) {
        const int coff = ((2 * s + h) ^ sw) << 4;
#pragma unroll
        for (int i = 0; i < FM; ++i) f.a[i] = *reinterpret_cast<const bf16x8*>(st + a_off + i * 32 * ROW + coff);
#pragma unroll
        for (int j = 0; j < FN; ++j) f.b[j] = *reinterpret_cast<const bf16x8*>(st + b_off + j * 32 * ROW + coff);
    };
    // ---- software pipeline over k-tiles, two LDS stages.  Iteration kt multiplies tile kt
    // (stage kt % 2).  Its last k-step is preceded by the barrier that publishes tile kt+1
    // (every wavefront has waited for its own copies of it) and frees stage kt % 2 (every
    // wavefront's reads of it have completed).  During that last k-step each wavefront
    // reads the first fragments of tile kt+1 and issues the copies of tile kt+2 into the
    // freed stage, so neither the barrier nor the first LDS reads of a tile leave the matrix
    // pipe waiting.  Past the end of K the copies repeat the last tile into a stage nobody
    // reads and the reads of a tile nk are never used, which keeps the loop free of branches.
    static_assert(S == 2, "two-stage pipeline");
    // copies of the next tile spread over the last k-step: CPS per matrix instruction
    constexpr int CPS = (C::DMA + C::MF - 1) / C::MF;
#pragma unroll
    for (int j = 0; j < C::DMA; ++j) issue_one(j, 0, 0);
#pragma unroll
    for (int j = 0; j < C::DMA; ++j) issue_one(j, min(1, nk - 1), 1);
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(C::DMA) : "memory");   // own copies of tile 0
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    Frags f[2];
    read_step(smem, 0, f[0]);
    for (int kt = 0; kt < nk; ++kt) {
        const unsigned char* cur = smem + (kt & 1) * C::STAGE;
        const unsigned char* nxt = smem + ((kt + 1) & 1) * C::STAGE;
        const int kc = min(kt + 2, nk - 1);
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            if (s == SUB - 1) {
                // own copies of tile kt+1 landed and own reads of tile kt complete; a plain
                // barrier (the compiler's workgroup fence would also drain later copies)
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
#pragma unroll
            for (int m = 0; m < C::MF; ++m) {
                const int i = m / FN, j = m % FN;
                // after the first instruction of the step, so that the wait for this step's
                // fragments does not also cover the reads of the next one
                if (m == 1) read_step(s + 1 < SUB ? cur : nxt, (s + 1) % SUB, f[(s + 1) & 1]);
                if (s == SUB - 1)
#pragma unroll
                    for (int c = m * CPS; c < (m + 1) * CPS; ++c)
                        if (c < C::DMA) issue_one(c, kc, kt & 1);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[s & 1].a[i], f[s & 1].b[j], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // the surplus copies must land before the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue ----
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn + 32 * j + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                p.C[(int64_t)row * p.ldc + col] = acc[i][j][r];
            }
        }
}

template <int BM, int BN, int BK, int WGM, int WGN, int S>
hipError_t launch_cfg(const Problem& p, const Launch& l) {
    const int tiles_m = p.M / BM, tiles_n = p.N / BN;
    hipLaunchKernelGGL((k_bf16_dma<Cfg<BM, BN, BK, WGM, WGN, S>>), dim3((unsigned)tiles_m * tiles_n),
                       dim3(64 * WGM * WGN), 0, l.stream, p, tiles_m, tiles_n, l.group_m);
    return hipGetLastError();
}

}  // namespace

bool bf16_dma_applies(const Problem& p, const Launch& l, int bm, int bn) {
    return p.oa == kRow && p.ob == kCol && l.vec_a && l.vec_b && p.K >= 64 && p.K % 64 == 0 &&
           p.M >= bm && p.N >= bn;
}

// Configurations: 256 x 256 with four wavefronts of 128 x 128 (256 accumulators each, in
// the accumulation registers; 128 KB of LDS), 256 x 128 with four wavefronts of 128 x 64.
// (Eight wavefronts of 64 x 128 measured slower: more LDS reads per matrix instruction.)
hipError_t launch_bf16_dma(const Problem& p, const Launch& l, int bm, int bn) {
    if (bm == 256 && bn == 256) return launch_cfg<256, 256, 64, 2, 2, 2>(p, l);
    if (bm == 256 && bn == 128) return launch_cfg<256, 128, 64, 2, 2, 2>(p, l);
    return hipErrorInvalidValue;
}

}  // namespace gemm
