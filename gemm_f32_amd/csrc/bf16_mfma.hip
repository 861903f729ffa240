// BF16-input, FP32-accumulate GEMM on the CDNA4 matrix cores: v_mfma_f32_32x32x16_bf16.
//
// The pages' matrix-core rung: a wavefront hands whole fragments to one matrix
// instruction with BF16 inputs and FP32 sums ("GEMM, step by step", Concept; "How a
// Matrix Multiply Runs on a GPU", "Level 3: tensor cores"; "A06 - Tiled Matrix Multiply
// (GEMM)", "Matrix cores: MFMA and Tensor Cores").  Those kernels were written for other
// hardware; this one is laid out for gfx950:
//
//  * Block tile BM x BN (256 x 256, 256 x 128, 128 x 128 or 64 x 64) swept in BK = 64
//    slices, 4 wavefronts in a 2 x 2 grid.  A wavefront owns (BM/2) x (BN/2) of C as
//    32 x 32 fragments; at 256 x 256 that is 4 x 4 fragments = 256 FP32 accumulators
//    per lane, which the compiler keeps in the accumulation registers.  Large tiles are
//    what a matrix-core GEMM needs to stay fed ("A06", three consequences of matrix
//    cores: the ridge moves right).
//  * Both operands live in LDS k-contiguous: a row of 64 bf16 = 128 bytes = eight
//    16-byte chunks, tile rows are rows of A and columns of B.  One lane's operand for
//    one instruction is one 16-byte chunk (8 consecutive k), read with ds_read_b128.
//  * Chunk c of LDS row r is stored at position c ^ s(r), s(r) = (r mod 8) xor bit 3 of
//    r.  The 32 lanes that read one fragment read 32 consecutive rows at the same
//    logical chunk; the XOR spreads any 16 consecutive rows over 16 distinct 16-byte
//    bank groups, so the reads are free of bank conflicts whether the LDS serves 8 or 16
//    lanes of a 16-byte read per cycle.  (The pages pad rows by one word; the XOR does the
//    same job for 16-byte accesses without wasting LDS.)
//  * Fragment k-assignment: for sub-step s of a k-tile, lanes 0-31 supply chunk 2s and
//    lanes 32-63 chunk 2s+1, for A and B alike.  Any assignment that pairs the same k
//    on both operands gives the same sum of products, so the instruction's own k-lane
//    order never needs to match the memory order.
//  * Accumulator layout of the 32 x 32 result: lane l, register r holds C[i][j] with
//    j = l % 32 and i = 8 (r / 4) + 4 (l / 32) + r % 4.
//  * Double-buffered LDS (2 stages, 128 KB at 256 x 256 of the 160 KB per CU): the next
//    k-tile's global loads are issued into registers before the current tile's
//    fragments are read and multiplied, then stored to the other stage; one barrier per
//    k-tile ("GEMM Optimization", V3; "A06", "The next two rungs").
//  * Loads: a k-contiguous operand (row-major A, column-major B) is fetched in 16-byte
//    chunks along k; rows past the matrix edge are clamped to the last row (their
//    products only feed outputs that are never stored).  An operand contiguous along
//    M or N is fetched in 16-byte chunks along that dimension and scattered into the
//    k-contiguous LDS layout.  The K tail, misaligned pointers or leading dimensions,
//    and edge tiles of an M/N-contiguous operand take an element-wise path with bounds
//    checks and zero fill ("A06", "Pitfall 1 - The boundary guard that fails silently").
//  * Tile order from the XCD-aware, group-M scheduler in common.hpp.
#include "common.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;

template <int BM_, int BN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = 64;
    static constexpr int WM = BM / 2, WN = BN / 2;      // 2 x 2 wavefronts
    static constexpr int THREADS = 256;
    static constexpr int FM = WM / 32, FN = WN / 32;    // 32 x 32 fragments per wavefront
    static constexpr int A_CHUNKS = BM * 8 / THREADS;   // 16-byte chunks per thread per k-tile
    static constexpr int B_CHUNKS = BN * 8 / THREADS;
    static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
    static constexpr int STAGE = A_BYTES + B_BYTES;
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// One operand as the loader sees it: `rows` (M for A, N for B) by K, stored with k
// contiguous (KC) or with rows contiguous.
struct Operand {
    const u16* p;
    int64_t ld;
    int rows;
};

// Chunk q of a KC operand tile: tile row q / 8, chunk q % 8 (k = 8 * (q % 8) .. +7).
template <int TR>
__device__ __forceinline__ uint4 load_kc(const Operand& x, int row0, int k0, int K, int q,
                                         bool fast) {
    const int r = q >> 3, c = q & 7;
    if (fast) {
        const int row = min(row0 + r, x.rows - 1);
        return *reinterpret_cast<const uint4*>(x.p + (int64_t)row * x.ld + k0 + c * 8);
    }
    u16 v[8];
    const int row = row0 + r;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int k = k0 + c * 8 + e;
        v[e] = (row < x.rows && k < K) ? x.p[(int64_t)row * x.ld + k] : (u16)0;
    }
    return make_uint4(v[0] | (unsigned)v[1] << 16, v[2] | (unsigned)v[3] << 16,
                      v[4] | (unsigned)v[5] << 16, v[6] | (unsigned)v[7] << 16);
}

template <int TR>
__device__ __forceinline__ void store_kc(unsigned char* s, int q, uint4 v) {
    const int r = q >> 3, c = q & 7;
    *reinterpret_cast<uint4*>(s + r * 128 + ((c ^ swz(r)) << 4)) = v;
}

// Chunk q of a row-contiguous operand tile: k = q / (TR / 8), rows 8 * (q % (TR / 8)) .. +7.
template <int TR>
__device__ __forceinline__ uint4 load_rc(const Operand& x, int row0, int k0, int K, int q,
                                         bool fast) {
    constexpr int CPK = TR / 8;   // chunks per k
    const int k = q / CPK, r = (q % CPK) * 8;
    if (fast) return *reinterpret_cast<const uint4*>(x.p + (int64_t)(k0 + k) * x.ld + row0 + r);
    u16 v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int row = row0 + r + e;
        v[e] = (row < x.rows && k0 + k < K) ? x.p[(int64_t)(k0 + k) * x.ld + row] : (u16)0;
    }
    return make_uint4(v[0] | (unsigned)v[1] << 16, v[2] | (unsigned)v[3] << 16,
                      v[4] | (unsigned)v[5] << 16, v[6] | (unsigned)v[7] << 16);
}

template <int TR>
__device__ __forceinline__ void store_rc(unsigned char* s, int q, uint4 v) {
    constexpr int CPK = TR / 8;
    const int k = q / CPK, r = (q % CPK) * 8;
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int row = r + e;
        *reinterpret_cast<u16*>(s + row * 128 + (((k >> 3) ^ swz(row)) << 4) + (k & 7) * 2) =
            (u16)(w[e >> 1] >> (16 * (e & 1)));
    }
}

template <int BM, int BN, bool A_KC, bool B_KC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_bf16_mfma(Problem p, int tiles_m, int tiles_n, int group_m, int vec_a, int vec_b) {
    using T = Tile<BM, BN>;
    __shared__ __align__(16) unsigned char smem[2 * T::STAGE];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 1) * T::WM, wn = (wave & 1) * T::WN;
    const int K = p.K;
    const int nk = (K + T::BK - 1) / T::BK;
    const bool interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);

    const Operand a{static_cast<const u16*>(p.A), p.lda, p.M};
    const Operand b{static_cast<const u16*>(p.B), p.ldb, p.N};
    // 16-byte loads need aligned pointers/leading dimensions; a row-contiguous operand also
    // needs its whole tile inside the matrix (no clamping across a chunk).
    const bool fast_a = vec_a && (A_KC || m0 + BM <= p.M);
    const bool fast_b = vec_b && (B_KC || n0 + BN <= p.N);

    uint4 ra[T::A_CHUNKS], rb[T::B_CHUNKS];
    auto gload = [&](int k0) {
        const bool full = k0 + T::BK <= K;
#pragma unroll
        for (int s = 0; s < T::A_CHUNKS; ++s) {
            const int q = t + s * T::THREADS;
            ra[s] = A_KC ? load_kc<BM>(a, m0, k0, K, q, fast_a && full)
                         : load_rc<BM>(a, m0, k0, K, q, fast_a && full);
        }
#pragma unroll
        for (int s = 0; s < T::B_CHUNKS; ++s) {
            const int q = t + s * T::THREADS;
            rb[s] = B_KC ? load_kc<BN>(b, n0, k0, K, q, fast_b && full)
                         : load_rc<BN>(b, n0, k0, K, q, fast_b && full);
        }
    };
    auto lstore = [&](int stage) {
        unsigned char* sa = smem + stage * T::STAGE;
        unsigned char* sb = sa + T::A_BYTES;
#pragma unroll
        for (int s = 0; s < T::A_CHUNKS; ++s) {
            const int q = t + s * T::THREADS;
            if (A_KC) store_kc<BM>(sa, q, ra[s]); else store_rc<BM>(sa, q, ra[s]);
        }
#pragma unroll
        for (int s = 0; s < T::B_CHUNKS; ++s) {
            const int q = t + s * T::THREADS;
            if (B_KC) store_kc<BN>(sb, q, rb[s]); else store_rc<BN>(sb, q, rb[s]);
        }
    };

    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    gload(0);
    lstore(0);
    __syncthreads();

    const int lr = lane & 31, h = lane >> 5;
    const int sw = swz(lr);                    // == swz(wm + 32 i + lr): wm, 32 i are multiples of 32
    const int a_off = (wm + lr) * 128;
    const int b_off = T::A_BYTES + (wn + lr) * 128;

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) gload((kt + 1) * T::BK);
        const unsigned char* st = smem + cur * T::STAGE;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int coff = ((2 * s + h) ^ sw) << 4;
            bf16x8 fa[T::FM], fb[T::FN];
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                fa[i] = *reinterpret_cast<const bf16x8*>(st + a_off + i * 32 * 128 + coff);
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                fb[j] = *reinterpret_cast<const bf16x8*>(st + b_off + j * 32 * 128 + coff);
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (more) lstore(cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const int col = n0 + wn + j * 32 + lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (interior || (row < p.M && col < p.N))
                    p.C[(int64_t)row * p.ldc + col] = acc[i][j][r];
            }
        }
}

template <int BM, int BN>
hipError_t launch_tile(const Problem& p, const Launch& l) {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const dim3 grid((unsigned)tiles_m * tiles_n), block(256);
    const bool akc = p.oa == kRow, bkc = p.ob == kCol;
    const int va = l.vec_a, vb = l.vec_b, g = l.group_m;
    if (akc && bkc)
        hipLaunchKernelGGL((k_bf16_mfma<BM, BN, true, true>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb);
    else if (akc)
        hipLaunchKernelGGL((k_bf16_mfma<BM, BN, true, false>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb);
    else if (bkc)
        hipLaunchKernelGGL((k_bf16_mfma<BM, BN, false, true>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb);
    else
        hipLaunchKernelGGL((k_bf16_mfma<BM, BN, false, false>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_mfma(const Problem& p, const Launch& l, int bm, int bn) {
    if (bm == 256 && bn == 256) return launch_tile<256, 256>(p, l);
    if (bm == 256 && bn == 128) return launch_tile<256, 128>(p, l);
    if (bm == 128 && bn == 128) return launch_tile<128, 128>(p, l);
    if (bm == 64 && bn == 64) return launch_tile<64, 64>(p, l);
    return hipErrorInvalidValue;
}

}  // namespace gemm
