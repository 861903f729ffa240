// BF16-input, FP32-accumulate GEMM, 256 x 256 block tiles, eight wavefronts in ping-pong.
//
// Same operation and LDS layout as bf16_mfma.hip (k-contiguous 128-byte rows, 16-byte chunks
// XOR-swizzled, direct global->LDS copies, 32 x 32 x 16 BF16 matrix instructions), arranged
// for the way a CDNA4 CU actually issues: each SIMD holds two wavefronts, one from each of two
// groups.  The groups alternate between two kinds of phase, separated by workgroup barriers:
//
//   compute phase: 32 matrix instructions back to back, operands already in registers;
//   memory phase:  read the next k-tile's fragments from LDS into registers and, for group 0,
//                  issue the global->LDS copies of the k-tile after that.
//
// While one wavefront of a SIMD computes, the other one loads, so the matrix pipe is fed
// from registers and never waits for LDS or for the copies (measured on gfx950: LDS reads
// and LDS-DMA copies interfere, and a single wavefront that interleaves them with its own
// matrix instructions stalls).  The pages' double-buffering idea ("GEMM Optimization", V3;
// "A06 - Tiled Matrix Multiply (GEMM)", "The next two rungs") is kept at both levels: two LDS
// stages, and the register fragments of the next k-tile loaded while the previous one is
// multiplied.
//
// Wavefront w: group g = w / 4, index q = w % 4; it owns rows 128 g .. +127 and columns
// 64 q .. +63 of the block tile (4 x 2 fragments of 32 x 32, 128 accumulators per lane).
// Two wavefronts share a SIMD's 512 registers, so a wavefront has 256: 128 accumulators
// plus the fragments of one k-tile, which is why k-tiles are BK = 32 deep (48 registers of
// fragments; BK = 64 would need 96 and spill).
//
// Schedule (k-tile k lives in LDS stage k % S, S = 4 stages of 32 KB):
//   prologue: tiles 0 .. S-1 copied (half by each group); group 0 loads fragments of tile 0
//   phase 2k:   group 0 computes tile k           | group 1 loads fragments of tile k
//   phase 2k+1: group 1 computes tile k           | group 0 loads fragments of tile k+1 and
//                                                 | copies tile k+S into stage k % S
// Stage k % S is free in phase 2k+1: group 0 read tile k in phase 2k-1, group 1 in phase
// 2k.  Tile k+S is needed in phase 2(k+S)-1; group 0 waits for it at the end of its compute
// phase 2(k+S)-2, with the copies of the S-2 later tiles still allowed in flight.
//
// Requirements (checked by the host): row-major A and column-major B (both k-contiguous),
// M and N multiples of 256, K a multiple
// of 32.  Other problems use bf16_mfma.hip.
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
constexpr int FM = 4, FN = 2, SUB = BK / 16;   // fragments per wavefront, k sub-steps
constexpr int RPW = 64, RPI = 1024 / ROW;      // rows copied per wavefront / per 1 KB copy
constexpr int DMA = RPW / RPI;                 // copies per wavefront per operand per tile

// chunk c of LDS row r sits at c ^ s(r): any 16 consecutive rows read at one logical chunk
// hit 16 distinct 16-byte bank groups
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
    const int wm = grp * 128, wn = q * 64;
    const int nk = p.K / BK;

    const u16* A = static_cast<const u16*>(p.A);
    const u16* B = static_cast<const u16*>(p.B);

    // ---- copies: wavefront q of the copying group fills rows 64 q .. +63 of both tiles,
    // RPI = 16 rows (1 KB) per copy; lane l fetches row RPI j + l / 4, logical chunk
    // (l % 4) ^ s(row), so that its 16 bytes land swizzled at LDS position l of the block
    // (see bf16_mfma.hip).  s(row) depends on l and on the parity of j only.
    const char* abase = reinterpret_cast<const char*>(A + (int64_t)(m0 + q * RPW) * p.lda);
    const char* bbase = reinterpret_cast<const char*>(B + (int64_t)(n0 + q * RPW) * p.ldb);
    const int lrow = lane >> 2;
    unsigned aoff[2], boff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int c = (lane & 3) ^ swz(lrow + par * RPI);
        aoff[par] = (unsigned)((lrow * p.lda + c * 8) * 2);
        boff[par] = (unsigned)((lrow * p.ldb + c * 8) * 2);
    }
    auto copy_tile = [&](int k0, int stage) {
        unsigned char* sa = smem + stage * STAGE + q * RPW * ROW;
        unsigned char* sb = smem + stage * STAGE + A_BYTES + q * RPW * ROW;
#pragma unroll
        for (int j = 0; j < DMA; ++j) {
            __builtin_amdgcn_global_load_lds(abase + ((int64_t)j * RPI * p.lda + k0) * 2 + aoff[j & 1],
                                             (lds_void*)(sa + j * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(bbase + ((int64_t)j * RPI * p.ldb + k0) * 2 + boff[j & 1],
                                             (lds_void*)(sb + j * 1024), 16, 0, 0);
        }
    };

    // ---- fragments of one k-tile and the matrix instructions on them ----
    const int lr = lane & 31, h = lane >> 5, sw = swz(lr);
    const int a_off = (wm + lr) * ROW, b_off = A_BYTES + (wn + lr) * ROW;
    bf16x8 fa[SUB][FM], fb[SUB][FN];
    auto load_frags = [&](int stage) {
        const unsigned char* st = smem + stage * STAGE;
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            const int coff = ((2 * s + h) ^ sw) << 4;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[s][i] = *reinterpret_cast<const bf16x8*>(st + a_off + i * 32 * ROW + coff);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[s][j] = *reinterpret_cast<const bf16x8*>(st + b_off + j * 32 * ROW + coff);
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
#pragma unroll
        for (int s = 0; s < SUB; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
    };

    // ---- prologue: tiles 0 .. S-1 in flight, group 0 holds the fragments of tile 0 ----
#pragma unroll
    for (int t = 0; t < S; ++t)
        if ((t & 1) == grp && t < nk) copy_tile(t * BK, t);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (grp == 0) load_frags(0);
    __syncthreads();

    // ---- ping-pong ----
    for (int k = 0; k < nk; ++k) {
        if (grp == 0) {                           // phase 2k
            compute();
            // tile k+1 must have landed; copies of up to S-2 later tiles may stay in flight
            if (k + S - 1 < nk) asm volatile("s_waitcnt vmcnt(%0)" :: "n"((S - 2) * 2 * DMA) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else {
            load_frags(k % S);
        }
        __syncthreads();
        if (grp == 1) {                           // phase 2k+1
            compute();
        } else {
            if (k + 1 < nk) load_frags((k + 1) % S);
            if (k + S < nk) copy_tile((k + S) * BK, k % S);
        }
        __syncthreads();
    }

    // ---- epilogue: lane l, register r of fragment (i, j) holds
    // C[m0 + wm + 32 i + 8 (r / 4) + 4 (l / 32) + r % 4][n0 + wn + 32 j + l % 32]
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn + j * 32 + lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                p.C[(int64_t)row * p.ldc + col] = acc[i][j][r];
            }
        }
}

}  // namespace

bool bf16_pingpong_applies(const Problem& p, const Launch& l) {
    return p.oa == kRow && p.ob == kCol && l.vec_a && l.vec_b && p.M % BM == 0 &&
           p.N % BN == 0 && p.K % BK == 0 && p.K >= BK;
}

hipError_t launch_bf16_pingpong(const Problem& p, const Launch& l) {
    const int tiles_m = p.M / BM, tiles_n = p.N / BN;
    hipLaunchKernelGGL(k_bf16_pingpong, dim3((unsigned)tiles_m * tiles_n), dim3(THREADS), 0,
                       l.stream, p, tiles_m, tiles_n, l.group_m);
    return hipGetLastError();
}

}  // namespace gemm
