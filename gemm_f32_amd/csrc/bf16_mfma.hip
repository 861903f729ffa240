// BF16-input, FP32-accumulate GEMM on the CDNA4 matrix cores: v_mfma_f32_32x32x16_bf16.
//
// The pages' matrix-core rung: a wavefront hands whole fragments to one matrix
// instruction with BF16 inputs and FP32 sums ("GEMM, step by step", Concept; "How a
// Matrix Multiply Runs on a GPU", "Level 3: tensor cores"; "A06 - Tiled Matrix Multiply
// (GEMM)", "Matrix cores: MFMA and Tensor Cores").  Those kernels were written for other
// hardware; this one is laid out for gfx950:
//
//  * Block tile BM x BN (256 x 128, 128 x 128 or 64 x 64) swept in BK = 32 or
//    64 slices, 4 wavefronts in a 2 x 2 grid.  A wavefront owns (BM/2) x (BN/2) of C as
//    32 x 32 fragments; at 256 x 256 that is 4 x 4 fragments = 256 FP32 accumulators
//    per lane, which the compiler keeps in the accumulation registers.  Large tiles are
//    what a matrix-core GEMM needs to stay fed ("A06", three consequences of matrix
//    cores: the ridge moves right).
//  * Both operands live in LDS k-contiguous: a row of BK bf16 = BK/8 16-byte chunks,
//    tile rows are rows of A and columns of B.  One lane's operand for one instruction is
//    one 16-byte chunk (8 consecutive k), read with ds_read_b128.
//  * Chunk c of LDS row r is stored at position c ^ s(r).  The 32 lanes that read one
//    fragment read 32 consecutive rows at the same logical chunk; s spreads any 16
//    consecutive rows over 16 distinct 16-byte bank groups (8 chunks per row: s(r) =
//    (r mod 8) xor bit 3 of r; 4 chunks: s(r) = (r/2 xor r/8) mod 4), so the reads are
//    free of bank conflicts whether the LDS serves 8 or 16 lanes of a 16-byte read per
//    cycle.  (The pages pad rows by one word; the XOR does the same job for 16-byte
//    accesses without wasting LDS.)
//  * Fragment k-assignment: for sub-step s of a k-tile, lanes 0-31 supply chunk 2s and
//    lanes 32-63 chunk 2s+1, for A and B alike.  Any assignment that pairs the same k
//    on both operands gives the same sum of products, so the instruction's own k-lane
//    order never needs to match the memory order.
//  * Accumulator layout of the 32 x 32 result: lane l, register r holds C[i][j] with
//    j = l % 32 and i = 8 (r / 4) + 4 (l / 32) + r % 4.
//  * Multi-stage LDS pipeline ("GEMM Optimization", V3; "A06", "The next two rungs"):
//    with S stages the copies of k-tile kt + S - 1 are in flight while tile kt is
//    multiplied (256 x 256 uses BK = 32 and 4 stages = 128 KB of the 160 KB per CU), one
//    barrier per k-tile.  Aligned, interior tiles with both operands k-contiguous copy
//    global -> LDS directly (global_load_lds_dwordx4, no registers); other tiles stage
//    through registers with 2 stages.
//  * Loads: a k-contiguous operand (row-major A, column-major B) is fetched in 16-byte
//    chunks along k; rows past the matrix edge are clamped to the last row (their
//    products only feed outputs that are never stored).  An operand contiguous along
//    M or N is fetched in 16-byte chunks along that dimension and scattered into the
//    k-contiguous LDS layout.  16-byte loads need element alignment only (gfx950 serves
//    unaligned vector loads and global->LDS copies).  The K tail and
//    edge tiles of an M/N-contiguous operand take an element-wise path with bounds checks
//    and zero fill ("A06", "Pitfall 1 - The boundary guard that fails silently").
//  * Tile order from the XCD-aware, group-M scheduler in common.hpp.
#include "common.hpp"
#include "launch.hpp"
#include "mma16.hpp"

namespace gemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) void lds_void;

template <int BM_, int BN_, int BK_, int S_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_;
    static constexpr int CH = BK / 8;                   // 16-byte chunks per LDS row
    static constexpr int ROW = BK * 2;                  // LDS row bytes
    static constexpr int SUB = BK / 16;                 // matrix-instruction k-steps per tile
    static constexpr int WM = BM / 2, WN = BN / 2;      // 2 x 2 wavefronts
    static constexpr int THREADS = 256;
    static constexpr int FM = WM / 32, FN = WN / 32;    // 32 x 32 fragments per wavefront
    static constexpr int A_CHUNKS = BM * CH / THREADS;  // 16-byte chunks per thread per k-tile
    static constexpr int B_CHUNKS = BN * CH / THREADS;
    static constexpr int A_BYTES = BM * ROW, B_BYTES = BN * ROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = (S > 2 ? S : 2) * STAGE;
    // direct global->LDS copies: each wavefront fills BM/4 rows of A and BN/4 rows of B,
    // RPI rows (1 KB, one 16-byte chunk per lane) per instruction
    static constexpr int RPI = 1024 / ROW;
    static constexpr int A_RPW = BM / 4, B_RPW = BN / 4;
    static constexpr int A_DMA = A_RPW / RPI, B_DMA = B_RPW / RPI;
    static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1 && A_DMA >= 1 && B_DMA >= 1, "tile too small");
    static_assert(A_RPW % 16 == 0 && B_RPW % 16 == 0, "wavefront row blocks must be 16-aligned");
};

template <int CH>
__device__ __forceinline__ int swz(int row) {
    if (CH == 8) return (row & 7) ^ ((row >> 3) & 1);
    return ((row >> 1) ^ (row >> 3)) & 3;
}

// One operand as the loader sees it: `rows` (M for A, N for B) by K, stored with k
// contiguous (KC) or with rows contiguous (RC).
struct Operand {
    const u16* p;
    int64_t ld;
    int rows;
};

__device__ __forceinline__ uint4 pack8(const u16 (&v)[8]) {
    return make_uint4(v[0] | (unsigned)v[1] << 16, v[2] | (unsigned)v[3] << 16,
                      v[4] | (unsigned)v[5] << 16, v[6] | (unsigned)v[7] << 16);
}

// Chunk q of a KC tile: tile row q / CH, k = 8 * (q % CH) .. +7.  The fast form needs a
// full k-tile; rows past the edge are clamped to the last row.
template <int CH>
__device__ __forceinline__ uint4 load_kc_fast(const Operand& x, int row0, int k0, int q) {
    const int row = min(row0 + q / CH, x.rows - 1);
    return load16(x.p + (int64_t)row * x.ld + k0 + (q % CH) * 8);
}
template <int CH>
__device__ __forceinline__ uint4 load_kc_checked(const Operand& x, int row0, int k0, int K, int q) {
    const int row = row0 + q / CH, kb = k0 + (q % CH) * 8;
    u16 v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = (row < x.rows && kb + e < K) ? x.p[(int64_t)row * x.ld + kb + e] : (u16)0;
    return pack8(v);
}
template <int CH>
__device__ __forceinline__ void store_kc(unsigned char* s, int q, uint4 v) {
    const int r = q / CH, c = q % CH;
    *reinterpret_cast<uint4*>(s + r * CH * 16 + ((c ^ swz<CH>(r)) << 4)) = v;
}

// Chunk q of an RC tile: k = q / (TR / 8), tile rows 8 * (q % (TR / 8)) .. +7.  The fast
// form needs the whole tile inside the matrix and a full k-tile.
template <int TR>
__device__ __forceinline__ uint4 load_rc_fast(const Operand& x, int row0, int k0, int q) {
    constexpr int CPK = TR / 8;
    return load16(x.p + (int64_t)(k0 + q / CPK) * x.ld + row0 + (q % CPK) * 8);
}
template <int TR>
__device__ __forceinline__ uint4 load_rc_checked(const Operand& x, int row0, int k0, int K, int q) {
    constexpr int CPK = TR / 8;
    const int k = k0 + q / CPK, r = row0 + (q % CPK) * 8;
    u16 v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = (r + e < x.rows && k < K) ? x.p[(int64_t)k * x.ld + r + e] : (u16)0;
    return pack8(v);
}
// Scatter the 8 values of an RC chunk into the k-contiguous LDS layout.
template <int TR, int CH>
__device__ __forceinline__ void store_rc(unsigned char* s, int q, uint4 v) {
    constexpr int CPK = TR / 8;
    const int k = q / CPK, r = (q % CPK) * 8;
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int row = r + e;
        *reinterpret_cast<u16*>(s + row * CH * 16 + (((k >> 3) ^ swz<CH>(row)) << 4) + (k & 7) * 2) =
            (u16)(w[e >> 1] >> (16 * (e & 1)));
    }
}

template <int BM, int BN, int BK, int S, bool A_KC, bool B_KC, bool F16 = false, bool BATCH = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_bf16_mfma(KArg<BATCH> p, int tiles_m, int tiles_n, int group_m, int vec_a, int vec_b, int direct) {
    using T = Tile<BM, BN, BK, S>;
    constexpr int CH = T::CH;
    // the direct path issues one tile's copies in the first SUB * FM * FN instruction slots
    static_assert(T::SUB * T::FM * T::FN >= T::A_DMA + T::B_DMA, "too few slots for the copies");
    __shared__ __align__(16) unsigned char smem[T::LDS];

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
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = (wave >> 1) * T::WM, wn = (wave & 1) * T::WN;
    const int K = p.K;
    const int nk = (K + BK - 1) / BK;
    const int nfull = K / BK;
    const bool interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);

    const Operand a{static_cast<const u16*>(p.A), p.lda, p.M};
    const Operand b{static_cast<const u16*>(p.B), p.ldb, p.N};
    // 16-byte loads of a whole k-tile: aligned operands, and a row-contiguous operand only
    // when its tile lies inside the matrix (a k-contiguous one clamps edge rows instead)
    const bool vec_tiles = vec_a && vec_b && (A_KC || m0 + BM <= p.M) && (B_KC || n0 + BN <= p.N);

    // ---- register-staged 16-byte loads (full k-tiles when the direct copy does not apply)
    uint4 ra[T::A_CHUNKS], rb[T::B_CHUNKS];
    auto gload_fast = [&](int k0) {
#pragma unroll
        for (int s = 0; s < T::A_CHUNKS; ++s)
            ra[s] = A_KC ? load_kc_fast<CH>(a, m0, k0, t + s * T::THREADS)
                         : load_rc_fast<BM>(a, m0, k0, t + s * T::THREADS);
#pragma unroll
        for (int s = 0; s < T::B_CHUNKS; ++s)
            rb[s] = B_KC ? load_kc_fast<CH>(b, n0, k0, t + s * T::THREADS)
                         : load_rc_fast<BN>(b, n0, k0, t + s * T::THREADS);
    };
    auto lstore = [&](int stage) {
        unsigned char* sa = smem + stage * T::STAGE;
        unsigned char* sb = sa + T::A_BYTES;
#pragma unroll
        for (int s = 0; s < T::A_CHUNKS; ++s) {
            if (A_KC) store_kc<CH>(sa, t + s * T::THREADS, ra[s]);
            else store_rc<BM, CH>(sa, t + s * T::THREADS, ra[s]);
        }
#pragma unroll
        for (int s = 0; s < T::B_CHUNKS; ++s) {
            if (B_KC) store_kc<CH>(sb, t + s * T::THREADS, rb[s]);
            else store_rc<BN, CH>(sb, t + s * T::THREADS, rb[s]);
        }
    };
    // ---- element-wise loads with bounds checks and zero fill into the same staging
    // registers (K tail, edge tiles of a row-contiguous operand): issued before
    // a k-tile's matrix instructions and stored after them, like the 16-byte loads
    auto gload_checked = [&](int k0) {
#pragma unroll
        for (int s = 0; s < T::A_CHUNKS; ++s)
            ra[s] = A_KC ? load_kc_checked<CH>(a, m0, k0, K, t + s * T::THREADS)
                         : load_rc_checked<BM>(a, m0, k0, K, t + s * T::THREADS);
#pragma unroll
        for (int s = 0; s < T::B_CHUNKS; ++s)
            rb[s] = B_KC ? load_kc_checked<CH>(b, n0, k0, K, t + s * T::THREADS)
                         : load_rc_checked<BN>(b, n0, k0, K, t + s * T::THREADS);
    };
    // ---- the same, one chunk at a time (the K tail after the direct path, where the
    // registers are taken by the direct path's addressing)
    auto load_store_checked = [&](int k0, int stage) {
        unsigned char* sa = smem + stage * T::STAGE;
        unsigned char* sb = sa + T::A_BYTES;
#pragma unroll 1
        for (int s = 0; s < T::A_CHUNKS; ++s) {
            const int q = t + s * T::THREADS;
            if (A_KC) store_kc<CH>(sa, q, load_kc_checked<CH>(a, m0, k0, K, q));
            else store_rc<BM, CH>(sa, q, load_rc_checked<BM>(a, m0, k0, K, q));
        }
#pragma unroll 1
        for (int s = 0; s < T::B_CHUNKS; ++s) {
            const int q = t + s * T::THREADS;
            if (B_KC) store_kc<CH>(sb, q, load_kc_checked<CH>(b, n0, k0, K, q));
            else store_rc<BN, CH>(sb, q, load_rc_checked<BN>(b, n0, k0, K, q));
        }
    };

    // ---- fragments and matrix instructions on one LDS stage ----
    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int lr = lane & 31, h = lane >> 5;
    const int sw = swz<CH>(lr);     // == swz(wm + 32 i + lr): s depends on row bits 0-4 only
    const int a_off = (wm + lr) * T::ROW;
    const int b_off = T::A_BYTES + (wn + lr) * T::ROW;
    auto read_frags = [&](const unsigned char* st, int s, bf16x8 (&fa)[T::FM], bf16x8 (&fb)[T::FN]) {
        const int coff = ((2 * s + h) ^ sw) << 4;
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
            fa[i] = *reinterpret_cast<const bf16x8*>(st + a_off + i * 32 * T::ROW + coff);
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
            fb[j] = *reinterpret_cast<const bf16x8*>(st + b_off + j * 32 * T::ROW + coff);
    };
    // One k-tile: SUB sub-steps of 16 k.  Fragments are double-buffered in registers so
    // that the LDS reads of sub-step s + 1 are in flight while the matrix instructions of
    // sub-step s run.  `copy(n)` is called before the n-th matrix instruction to fold
    // another tile's global->LDS copies into the same instruction stream.  Source order is
    // issue order (sched_barrier fences).
    auto compute = [&](int stage, auto copy) {
        const unsigned char* st = smem + stage * T::STAGE;
        bf16x8 fa[2][T::FM], fb[2][T::FN];
        read_frags(st, 0, fa[0], fb[0]);
#pragma unroll
        for (int s = 0; s < T::SUB; ++s) {
            const int coff = ((2 * (s + 1) + h) ^ sw) << 4;
            // MF matrix instructions and RD fragment reads per sub-step; small tiles have
            // fewer instructions than reads, so the loop runs over the larger count
            constexpr int MF = T::FM * T::FN, RD = T::FM + T::FN;
            const bool next = s + 1 < T::SUB;
#pragma unroll
            for (int m = 0; m < (MF > RD ? MF : RD); ++m) {
                if (m < MF) copy(s * MF + m);
                if (next && m < T::FM)
                    fa[(s + 1) & 1][m] = *reinterpret_cast<const bf16x8*>(st + a_off + m * 32 * T::ROW + coff);
                else if (next && m < RD)
                    fb[(s + 1) & 1][m - T::FM] =
                        *reinterpret_cast<const bf16x8*>(st + b_off + (m - T::FM) * 32 * T::ROW + coff);
                if (m < MF) {
                    const int i = m / T::FN, j = m % T::FN;
                    acc[i][j] = mma_32x32x16<F16>(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    auto no_copy = [](int) {};

    int kt = 0;
    if (A_KC && B_KC && direct && interior && nfull > 0) {
        // ---- direct path: full k-tiles copied global -> LDS without registers, S stages ----
        // Copy j of a wavefront fills tile rows r0 + RPI j .. +RPI-1 (r0 = the wavefront's
        // first row, a multiple of 16); lane l fetches the chunk that belongs at LDS
        // position l of that 1 KB block: row r0 + RPI j + l / CH, logical chunk
        // (l % CH) ^ s(row).  s(row) depends on l and on the parity of r0 / RPI + j only,
        // so a lane needs two byte offsets on top of a wavefront-uniform row address.
        const int arow0 = m0 + wave * T::A_RPW, brow0 = n0 + wave * T::B_RPW;
        const char* abase = reinterpret_cast<const char*>(a.p + (int64_t)arow0 * a.ld);
        const char* bbase = reinterpret_cast<const char*>(b.p + (int64_t)brow0 * b.ld);
        const int lrow = lane / CH, lc = lane % CH;
        unsigned aoff[2], boff[2];
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int c = lc ^ swz<CH>(lrow + par * T::RPI);
            aoff[par] = (unsigned)((lrow * a.ld + c * 8) * 2);
            boff[par] = (unsigned)((lrow * b.ld + c * 8) * 2);
        }
        const int apar = (arow0 / T::RPI) & 1, bpar = (brow0 / T::RPI) & 1;
        auto issue_one = [&](int j, int k0, int stage) {   // copy j of this wavefront
            unsigned char* sa = smem + stage * T::STAGE + wave * T::A_RPW * T::ROW;
            unsigned char* sb = smem + stage * T::STAGE + T::A_BYTES + wave * T::B_RPW * T::ROW;
            if (j < T::A_DMA) {
                const char* g = abase + ((int64_t)j * T::RPI * a.ld + k0) * 2;
                __builtin_amdgcn_global_load_lds(g + aoff[(apar + j) & 1], (lds_void*)(sa + j * 1024), 16, 0, 0);
            } else {
                const int jb = j - T::A_DMA;
                const char* g = bbase + ((int64_t)jb * T::RPI * b.ld + k0) * 2;
                __builtin_amdgcn_global_load_lds(g + boff[(bpar + jb) & 1], (lds_void*)(sb + jb * 1024), 16, 0, 0);
            }
        };
        constexpr int DMA = T::A_DMA + T::B_DMA;
        constexpr int SPREAD = T::SUB * T::FM * T::FN >= 2 * DMA ? 2 : 1;
        // prologue: tiles 0 .. S-2 in flight
#pragma unroll
        for (int st = 0; st + 1 < S; ++st)
            if (st < nfull)
                for (int j = 0; j < DMA; ++j) issue_one(j, st * BK, st);
        for (; kt < nfull; ++kt) {
            // Tile kt has landed once at most the copies of tiles kt+1 .. kt+S-2 are pending,
            // and stage (kt-1) % S is free once this wavefront's reads of it have returned.
            // Then a plain barrier: __syncthreads() would also wait for the later tiles'
            // copies (the compiler's workgroup fence covers the global->LDS copies), which
            // would cut the pipeline back to two stages.
            static_assert((S - 2) * DMA < 64, "vmcnt range");
            if (kt + S - 2 < nfull) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"((S - 2) * DMA) : "memory");
            else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();   // tile kt visible to all; stage (kt-1) % S free
            asm volatile("" ::: "memory");
            const int kn = kt + S - 1;
            const bool copies = kn < nfull;          // wavefront-uniform
            const int k0n = kn * BK, stn = kn % S;
            // one copy every SPREAD instruction slots: the copies share the CU's 64-byte/clk
            // vector-memory path, and bursts of them stall the in-order wavefront
            compute(kt % S, [&](int n) {
                if (n % SPREAD == 0 && n / SPREAD < DMA && copies) issue_one(n / SPREAD, k0n, stn);
            });
        }
        if (nk > nfull) {      // the K tail: bounds-checked loads into the next free stage
            __syncthreads();
            load_store_checked(nfull * BK, nfull % S);
            __syncthreads();
            compute(nfull % S, no_copy);
        }
    } else {
        // ---- register-staged path, 2 stages.  Checked loads are staged in registers too
        // where the registers allow it (all but the mixed-layout 256 x 256 tiles, which load
        // and store them a chunk at a time) ----
        constexpr bool STAGE_CHECKED = A_KC == B_KC || T::A_CHUNKS + T::B_CHUNKS <= 12;
        if (vec_tiles && nfull > 0) { gload_fast(0); lstore(0); }
        else if (STAGE_CHECKED) { gload_checked(0); lstore(0); }
        else load_store_checked(0, 0);
        __syncthreads();
        for (; kt < nk; ++kt) {
            const int k0n = (kt + 1) * BK, stn = (kt + 1) & 1;
            const bool more = kt + 1 < nk;
            const bool next_fast = more && vec_tiles && k0n + BK <= K;
            if (next_fast) gload_fast(k0n);
            else if (more && STAGE_CHECKED) gload_checked(k0n);
            compute(kt & 1, no_copy);
            if (next_fast || (more && STAGE_CHECKED)) lstore(stn);
            else if (more) load_store_checked(k0n, stn);
            __syncthreads();
        }
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

template <int BM, int BN, int BK, int S, bool F16, bool BATCH>
hipError_t launch_tile_t(const KArg<BATCH>& p, const Launch& l) {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const dim3 grid((unsigned)tiles_m * tiles_n, 1, BATCH ? l.batch : 1), block(256);
    const bool akc = p.oa == kRow, bkc = p.ob == kCol;
    const int va = l.vec_a, vb = l.vec_b, g = l.group_m, al = l.vec_a && l.vec_b;   // direct copies allowed
    if (akc && bkc)
        hipLaunchKernelGGL((k_bf16_mfma<BM, BN, BK, S, true, true, F16, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb, al);
    else if (akc)
        hipLaunchKernelGGL((k_bf16_mfma<BM, BN, BK, S, true, false, F16, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb, al);
    else if (bkc)
        hipLaunchKernelGGL((k_bf16_mfma<BM, BN, BK, S, false, true, F16, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb, al);
    else
        hipLaunchKernelGGL((k_bf16_mfma<BM, BN, BK, S, false, false, F16, BATCH>), grid, block, 0, l.stream, p, tiles_m, tiles_n, g, va, vb, al);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int S>
hipError_t launch_tile(const Problem& p, const Launch& l, bool f16) {
    if (l.batch > 1) {
        const BatchProblem b = batch_arg(p, l, 2);
        return f16 ? launch_tile_t<BM, BN, BK, S, true, true>(b, l) : launch_tile_t<BM, BN, BK, S, false, true>(b, l);
    }
    return f16 ? launch_tile_t<BM, BN, BK, S, true, false>(p, l) : launch_tile_t<BM, BN, BK, S, false, false>(p, l);
}

}  // namespace

// Tile configurations: block tile, k-tile depth and LDS stages.
hipError_t launch_bf16_mfma(const Problem& p, const Launch& l, int bm, int bn, bool f16) {
    if (bm == 256 && bn == 128) return launch_tile<256, 128, 64, 3>(p, l, f16);   // 144 KB
    if (bm == 128 && bn == 128) return launch_tile<128, 128, 64, 2>(p, l, f16);   //  64 KB
    if (bm == 64 && bn == 64) return launch_tile<64, 64, 64, 2>(p, l, f16);       //  32 KB
    return hipErrorInvalidValue;
}

}  // namespace gemm
