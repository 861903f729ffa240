// 16-bit- and 8-bit-input, FP32-accumulate GEMM with direct global->LDS copies:
// v_mfma_f32_32x32x16_bf16 / _f16, and for the OCP 8-bit formats (E4M3, E5M2)
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales.
//
// Same operation as bf16_mfma.hip ("GEMM, step by step", Concept; "A06 - Tiled Matrix
// Multiply (GEMM)", "Matrix cores: MFMA and Tensor Cores"), for the layout a BF16 GEMM
// usually has (row-major A, column-major B: both operands contiguous along k), arranged so
// that the k-loop is one branch-free block:
//
//  * Block tile BM x BN, k-tiles of 128 bytes per row (BK = 64 16-bit or 128 8-bit
//    elements), WGM x WGN wavefronts.  At 256 x 256 four
//    wavefronts in a 2 x 2 grid own 128 x 128 of C each (4 x 4 fragments of 32 x 32 = 256
//    accumulators per lane), one per SIMD.  At 256 x 128, eight wavefronts of 64 x 64, two
//    per SIMD.
//  * LDS: one row of BK elements (128 bytes, 8 chunks of 16 bytes) per row of each tile, chunk
//    c of row r stored at c ^ s(r), s(r) = (r mod 8) xor bit 3 of r, so that the 32 rows
//    read at one logical chunk fall on distinct 16-byte bank groups.  A lane's 16-byte read
//    is one instruction's operand: at k-step s (16 k) lanes 0-31 read chunk 2 s, lanes
//    32-63 chunk 2 s + 1, for A and B alike (the pairing of k between the two operands is
//    what matters, not its order).  With 8-bit inputs an operand is 32 bytes: at k-step s
//    (64 k) lanes 0-31 read chunks 4 s and 4 s + 1, lanes 32-63 chunks 4 s + 2 and 4 s + 3.
//  * Accumulator layout of a 32 x 32 fragment: lane l, register r holds row
//    8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
//  * Copies: buffer loads of 1 KB per instruction straight into LDS, a lane fetching the
//    chunk that belongs at its LDS position; the per-lane offset is fixed, the k-tile and
//    the copy's row block are a scalar offset.  Each wavefront's buffer covers exactly the
//    rows of its copy block that exist, so rows past M (N) read as zero: edge tiles need no
//    separate code in the k-loop.  (Buffer loads, like global ones, accept the 2-byte
//    aligned rows of odd leading dimensions on gfx950, and the byte-aligned rows of 8-bit
//    operands.)
//  * Staging ahead ("GEMM Optimization", V3: stage the next tile while the current one is
//    multiplied), software-pipelined across k-tiles, one barrier per k-tile: at 256 x 256 a
//    ring of five half-stage buffers (an A or a B tile each, 160 KB) that lets each copy
//    start one to two k-tiles before its tile is multiplied; at 256 x 128 three whole
//    stages.
//  * K tail: a last k-tile staged through registers with bounds checks and zero fill into
//    the same LDS positions ("A06 - Tiled Matrix Multiply (GEMM)", "Pitfall 1 - The
//    boundary guard that fails silently": a ragged K needs the zero fill).
//  * Epilogue: each wavefront passes its accumulators through LDS one 32-row band at a time
//    and stores whole rows with 16-byte stores (straight from the accumulators, C rows are
//    written 4 bytes per lane, 128 bytes per 32 lanes, which takes four times as many
//    store instructions for the same 64 MB at 4096^2); stores past M or N are skipped.
//  * Tile order from the XCD-aware, group-M scheduler in common.hpp.
//
// Requirements (checked by the host): row-major A and column-major B after the
// column-major-C swap (both k-contiguous), K >= 64 for 16-bit inputs (any K >= 1 for 8-bit
// ones), and byte offsets of a wavefront's row block below 2^31.  Any M, N.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"
#include "mma16.hpp"

namespace gemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// input element types of the kernel: 16-bit, or 8-bit as kInFp8 + 2 fmt_a + fmt_b
enum InType { kInBf16 = 0, kInF16 = 1, kInFp8 = 2 };

// gfx950 buffer resource, word 3: 32-bit unformatted data, no swizzle
constexpr int kBufWord3 = 0x00020000;

// gfx950's transposing LDS read of four 16-bit values per lane.  (Through a restrict-qualified
// parameter: the inlined read then carries alias information, without which the compiler makes
// it wait for every copy into LDS in flight, as it does not for the plain vector reads.)
__device__ __forceinline__ s16x4 lds_read_tr16(lds_s16x4* __restrict__ p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}

// the lane's index within its wavefront
__device__ __forceinline__ int lane_id() {
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & 63;     // (the mask: a known range)
}

// chunk c of LDS row r is stored at c ^ swz(r): any 16 consecutive rows read at one
// logical chunk hit 16 distinct 16-byte bank groups
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// RING: the five-buffer half-stage pipeline of the main loop below (BM == BN) instead of S
// whole stages.  ES: bytes per input element, 2 (bf16, fp16) or 1 (the 8-bit formats); a
// k-tile is one 128-byte row either way, 64 or 128 k deep.
template <int BM_, int BN_, int WGM_, int WGN_, int CSPAN_, int S_, bool RING_ = false, int ES_ = 2>
struct Cfg {
    static constexpr int ES = ES_;
    static constexpr int BM = BM_, BN = BN_, BK = 128 / ES, WGM = WGM_, WGN = WGN_, S = S_;
    static constexpr bool RING = RING_;
    static constexpr int ROW = BK * ES;                      // LDS row bytes (8 chunks)
    // k of one matrix instruction (32x32x16 on 16-bit inputs, 32x32x64 on 8-bit ones) and the
    // 16-byte chunks of a row each lane supplies to it
    static constexpr int KSTEP = ES == 2 ? 16 : 64, FC = KSTEP * ES / 32;
    static constexpr int RPC = 1024 / ROW;                   // tile rows per 1 KB copy
    static constexpr int NW = WGM * WGN, THREADS = 64 * NW;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 32, FN = WN / 32;         // 32 x 32 fragments per wavefront
    static constexpr int A_BYTES = BM * ROW, B_BYTES = BN * ROW, STAGE = A_BYTES + B_BYTES;
    static constexpr int A_RPW = BM / NW, B_RPW = BN / NW;   // tile rows copied per wavefront
    static constexpr int A_DMA = A_RPW / RPC, B_DMA = B_RPW / RPC;
    static constexpr int DMA = A_DMA + B_DMA;                // copies per wavefront per k-tile
    static constexpr int SUB = BK / KSTEP;                   // k-steps per k-tile
    static constexpr int MF = FM * FN;                       // matrix instructions per k-step
    static constexpr int RD = FM + FN;                       // fragment reads per k-step
    // the copies of k-tile t are spread over CSPAN k-steps (the last one of k-tile t - S
    // and the first CSPAN - 1 of k-tile t - S + 1), one every W / DMA instruction slots;
    // HEAD of them fall on the first of those k-steps
    static constexpr int CSPAN = CSPAN_, W = CSPAN * MF;
    static constexpr int HEAD = (MF * DMA + W - 1) / W;
    static_assert(ES == 1 || ES == 2, "element size");
    static_assert(FM >= 1 && FN >= 1 && A_DMA >= 1 && B_DMA >= 1, "tile too small");
    static_assert(A_RPW % 16 == 0 && B_RPW % 16 == 0, "copy blocks start at even swizzle parity");
    static_assert(RD <= MF, "one fragment read per instruction slot");
    static_assert(S == 2 || S == 3, "LDS stages");
    // with two stages the copies of tile kt+1 are issued and land within iteration kt; with
    // three they have until the barrier of iteration kt+1
    static_assert(CSPAN >= 1 && (S == 2 ? CSPAN < SUB : CSPAN <= SUB), "copies land before their barrier");
    static_assert(W >= DMA, "at most one copy per instruction slot");
    static_assert(!RING || (BM == BN && B_DMA <= MF && A_DMA <= (SUB - 1) * MF), "ring layout");
    static constexpr int LDS = RING ? 5 * A_BYTES : S * STAGE;
    // epilogue: a 32 x WN band per wavefront, rows padded by 8 floats (the two half-waves
    // of one accumulator register, 4 rows apart, land on different banks)
    static constexpr int EP = WN + 8;
    static_assert(NW * 32 * EP * 4 <= LDS, "epilogue staging fits in the stages");
    static_assert(NW % 4 == 0, "whole wavefronts per SIMD");
};

using Cfg256 = Cfg<256, 256, 2, 2, 2, 2, true>;

// 8-bit configurations: 256 x 256 on the ring, 256 x 128 with three stages (copies spread over
// both k-steps of a 128-deep k-tile)
using Cfg256F8 = Cfg<256, 256, 2, 2, 1, 2, true, 1>;
using Cfg256x128F8 = Cfg<256, 128, 4, 2, 2, 3, false, 1>;

// IT: input type, kInBf16, kInF16 or, for 8-bit inputs, kInFp8 + 2 fmt_a + fmt_b (format 0 E4M3,
// 1 E5M2, the operand-format codes of the gfx950 8-bit matrix instruction).
// MODE: kPlain, kBatched (entry blockIdx.z of a strided batch), kEpilogue (the fused epilogue,
// one problem) or kSplitK (K slice blockIdx.y of one problem).
// TK: K below one 16-byte chunk of 8-bit elements (K < 16): no k-loop, the K tail read byte by
// byte.  (A separate kernel: with byte loads anywhere in the function, the compiler adds waits
// for all copies in flight before every LDS read of the k-loop.)
// BRM: row-major B (n contiguous; 16-bit inputs).  The B tile is then held in LDS as it lies in
// memory, BK k-rows of BN columns, and read with gfx950's transposing LDS read, which hands each
// lane four consecutive k of one column (the layout of the B tile and its reads are described at
// the copy plan below).
template <typename C, bool VEC_C, int IT, int MODE, bool TK = false, bool BRM = false>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::NW / 4, C::NW / 4)))
void k_bf16_dma(typename ModeArgT<MODE>::type p, int tiles_m, int tiles_n, int group_m) {
    constexpr bool BATCH = MODE == kBatched, EPI = MODE == kEpilogue;
    static_assert((IT >= kInFp8) == (C::ES == 1), "8-bit inputs take the 8-bit configurations");
    static_assert(!TK || C::ES == 1, "byte-wise K tail for 8-bit inputs only");
    static_assert(!BRM || C::ES == 2, "row-major B for 16-bit inputs only");
    constexpr int ES = C::ES;
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, FM = C::FM, FN = C::FN, SUB = C::SUB;
    constexpr int ROW = C::ROW, MF = C::MF;
    __shared__ __align__(16) unsigned char smem[C::LDS];
    if constexpr (MODE == kSplitK) p.select(blockIdx.y, ES);

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
    const bool interior = m0 + BM <= p.M && n0 + BN <= p.N;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave / C::WGN) * C::WM, wn = (wave % C::WGN) * C::WN;
    const int nk = p.K / BK;                  // whole k-tiles; a K tail follows the loop
    const unsigned char* A = static_cast<const unsigned char*>(p.A);
    const unsigned char* B = static_cast<const unsigned char*>(p.B);

    // ---- copy plan: wavefront w fills rows w A_RPW .. +A_RPW-1 of the A tile (and the same
    // for B), RPC rows per copy; lane l fetches row l / 8 of the copy at logical chunk
    // (l % 8) ^ s(row), where s(row) depends on l and on the parity of the copy only
    // (copy blocks start at multiples of 16 rows).  Offsets are in bytes.
    const int lr = lane / 8;
    unsigned aoff[2], boff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int c = (lane % 8) ^ swz(lr + C::RPC * par);
        aoff[par] = (unsigned)(lr * p.lda * ES + c * 16);
        boff[par] = (unsigned)(lr * p.ldb * ES + c * 16);
    }
    // buffer resources over the rows of this wavefront's copy blocks that exist: the
    // hardware returns zero for the rest (the host checks that offsets fit in 31 bits)
    const int arow0 = m0 + wave * C::A_RPW, brow0 = n0 + wave * C::B_RPW;
    // (wavefront-uniform values; readfirstlane tells the compiler so, which keeps the buffer
    // resources in scalar registers)
    const int avalid = __builtin_amdgcn_readfirstlane(max(0, min(C::A_RPW, p.M - arow0)));
    const int bvalid = __builtin_amdgcn_readfirstlane(max(0, min(C::B_RPW, p.N - brow0)));
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(avalid > 0 ? A + (int64_t)arow0 * p.lda * ES : A), (short)0, (int)(avalid * p.lda * ES), kBufWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(bvalid > 0 ? B + (int64_t)brow0 * p.ldb * ES : B), (short)0, (int)(bvalid * p.ldb * ES), kBufWord3);
    // byte distance between consecutive copies of a wavefront
    const int astep = C::RPC * (int)p.lda * ES, bstep = C::RPC * (int)p.ldb * ES;

    // ---- row-major B (BRM).  The B tile of a k-tile is BK = 64 k-rows of BN columns, RP = 2 BN
    // bytes each, in RP / 64 groups of 64 bytes (32 columns).  Group q of k-row kr is stored at
    // q ^ bsw(kr), bsw taking bits 0, 1 and 3 of kr (as many as there are groups), so that the
    // k-rows one transposing read takes together (four consecutive ones, and the four 8 rows on
    // that the other half-wavefront takes) fall on distinct banks.  A copy fills 1024 / RP whole
    // k-rows; the lane that stores position l of it fetches k-row l / (RP / 16), physical chunk
    // c = l % (RP / 16), which holds logical chunk c ^ 4 bsw(kr) (8 columns).  Chunks past N (the
    // last column tile) fetch the row's last 8 columns instead: they feed only columns of C that
    // are never stored, and every fetch stays inside the operand (the host requires N % 8 == 0).
    // bsw of a copy's k-row is the xor of bsw of its parts (the wavefront's first k-row, the
    // copy's first row, the lane's row in the copy: disjoint bits), so a copy's lane offset
    // depends on the copy only through one of at most RP / 64 group patterns.
    constexpr int RP = BN * 2, RPC2 = 1024 / RP, KRW = BK / C::NW, GM = RP / 64 - 1;
    auto bsw = [](int kr) { return ((kr & 3) | ((kr >> 1) & 4)) & GM; };
    const int lr2 = lane / (RP / 16), cc2 = lane % (RP / 16);
    const int bsw_w = __builtin_amdgcn_readfirstlane(bsw(wave * KRW));
    // offset of this lane's 16 bytes from the wavefront's first k-row of the k-tile, for a copy
    // whose k-rows have pattern f
    auto brm_lane = [&](int f) -> unsigned {
        const int col = min(n0 + 8 * (cc2 ^ (4 * (bsw(lr2) ^ f))), p.N - 8);
        return (unsigned)(lr2 * (int)p.ldb * 2 + 2 * (col - n0));
    };
    // the resource starts at the wavefront's first k-row, column n0, and ends after element
    // (K-1, N-1), which no fetch passes (the host requires K ldb 2 < 2^31)
    const int brm_row0 = wave * KRW;
    const __amdgpu_buffer_rsrc_t rbr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(B + ((int64_t)brm_row0 * p.ldb + n0) * 2), (short)0,
        (int)(((int64_t)(p.K - 1 - brm_row0) * p.ldb + p.N - n0) * 2), kBufWord3);
    const int brm_kt = BK * (int)p.ldb * 2, brm_step = RPC2 * (int)p.ldb * 2;   // per k-tile, per copy
    // B copy jb of k-tile kt into the LDS block at dst
    // (offsets as named values: with the lambda call inside the builtin's argument list the host
    // pass of this compiler silently drops the kernel's launch stub)
    auto copy_b = [&](int jb, int kt, lds_void* dst) {
        if constexpr (BRM) {
            const unsigned vo = brm_lane(bsw_w ^ bsw(jb * RPC2));
            const int so = kt * brm_kt + jb * brm_step;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rbr, dst, 16, vo, so, 0, 0);
        } else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, boff[jb & 1] + jb * bstep, kt * ROW, 0, 0);
    };
    // copy j (of DMA) of k-tile kt (source) into stage st.  (The LDS pointer is a named
    // variable: cast inline in the builtin's argument list, the host pass of this compiler
    // silently drops the kernel's launch stub.)
    // The copy's row block is part of the lane offset, the k-tile the scalar offset: rows past
    // the buffer's range then read as zero whether or not the range check counts the scalar
    // offset (a k offset stays inside its row).
    auto issue_one = [&](int j, int kt, int st) {
        unsigned char* s = smem + st * C::STAGE;
        if (j < C::A_DMA) {
            lds_void* dst = (lds_void*)(s + (wave * C::A_DMA + j) * 1024);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, aoff[j & 1] + j * astep, kt * ROW, 0, 0);
        } else {
            const int jb = j - C::A_DMA;
            lds_void* dst = (lds_void*)(s + C::A_BYTES + (wave * C::B_DMA + jb) * 1024);
            copy_b(jb, kt, dst);
        }
    };
    // the copies that fall on slot `slot` of the window (copy q sits at slot q W / DMA)
    auto copies_at = [&](int slot, int kt, int st) {
#pragma unroll
        for (int q = 0; q < C::DMA; ++q)
            if ((q * C::W) / C::DMA == slot) issue_one(q, kt, st);
    };

    // ---- fragments and matrix instructions ----
    const int l32 = lane & 31, h = lane >> 5, sw = swz(l32);
    const int a_off = (wm + l32) * ROW;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // a lane's operand of one matrix instruction: 8 bf16 / fp16 values, or 32 8-bit values (two
    // chunks).  At k-step s lanes 0-31 take the FC chunks FC (2 s) .. and lanes 32-63 the FC
    // chunks after them, for A and B alike (which k goes to which lane only has to agree
    // between the two operands).
    using Frag = std::conditional_t<ES == 2, bf16x8, i32x8>;
    Frag fa[2][FM], fb[2][FN];
    auto frag_at = [&](const unsigned char* row, int s) -> Frag {
        if constexpr (C::FC == 1) {
            return *reinterpret_cast<const bf16x8*>(row + (((2 * s + h) ^ sw) << 4));
        } else {
            // (read as 16-bit vectors: with that access type the compiler adds no wait for the
            // copies in flight before these reads; the waits in the loop below order them)
            const i32x4 lo = __builtin_bit_cast(i32x4, *reinterpret_cast<const bf16x8*>(row + (((4 * s + 2 * h) ^ sw) << 4)));
            const i32x4 hi = __builtin_bit_cast(i32x4, *reinterpret_cast<const bf16x8*>(row + (((4 * s + 2 * h + 1) ^ sw) << 4)));
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    // BRM: lane L of 16-lane group g = L / 16 (l = L % 16) takes, for B fragment j at k-step s,
    // column wn + 32 j + L % 32 at k = 16 s + 8 h + 0..7 (the k of A's lane L) from two
    // transposing reads of four k-rows each.  In such a read the lanes of a group address k-rows
    // kb + l / 4, the four columns from 4 (l % 4) of the group's 16, and lane l receives element
    // l % 4 of the 8-byte chunks of lanes 4 e + l / 4, e = 0..3: column l of the 16 at k-rows
    // kb .. kb + 3.  The lane's k-row 8 h + l / 4 (plus 16 s + 4 t) fixes its group pattern, and
    // fragment j's group index (wn / 32 + j, wn / 32 a multiple of the fragment count) differs
    // from fragment 0's in the low bits only: fragment j's offset is fragment 0's xor 64 j.
    const int l16 = lane & 15;
    const int brm_kr = 8 * h + (l16 >> 2);
    const unsigned brm_rd = (unsigned)(brm_kr * RP + (((wn >> 5) ^ bsw(brm_kr)) << 6) + 32 * ((lane >> 4) & 1) +
                                       8 * (l16 & 3));
    // (The tile's LDS offset, a multiple of the row block, is added before the xor, so that the
    // fragments' offsets are formed per k-tile rather than held in registers across the loop.)
    auto frag_rm = [&](int tile, int s, int j) -> bf16x8 {
        const unsigned char* q = smem + ((unsigned)(tile + brm_rd) ^ (unsigned)(j << 6)) + 16 * s * RP;
        const s16x4 lo = lds_read_tr16((lds_s16x4*)q);
        const s16x4 hi = lds_read_tr16((lds_s16x4*)(q + 4 * RP));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // B fragment j at k-step s of the B tile at LDS offset `tile`
    auto frag_b = [&](int tile, int s, int j) -> Frag {
        if constexpr (BRM) return frag_rm(tile, s, j);
        else return frag_at(smem + tile + (wn + l32) * ROW + j * 32 * ROW, s);
    };
    // fragment read `m` (A fragments first, then B) of k-step s of stage st into buffer b
    auto read_slot = [&](int st, int s, int m, int b) {
        const unsigned char* base = smem + st * C::STAGE;
        if (m < FM) fa[b][m] = frag_at(base + a_off + m * 32 * ROW, s);
        else if (m < C::RD) fb[b][m - FM] = frag_b(st * C::STAGE + C::A_BYTES, s, m - FM);
    };
    auto mfma = [&](int m, int b) {
        const int i = m / FN, j = m % FN;
        if constexpr (IT >= kInFp8)     // unit scales (E8M0 127 = 2^0): a plain 8-bit product
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[b][i], fb[b][j], acc[i][j],
                                                                         (IT - kInFp8) >> 1, (IT - kInFp8) & 1,
                                                                         0, 127, 0, 127);
        else
            acc[i][j] = mma_32x32x16<IT == kInF16>(fa[b][i], fb[b][j], acc[i][j]);
    };

    // ---- software pipeline over k-tiles, S LDS stages (tile t in stage t % S).  Iteration
    // kt multiplies tile kt k-step by k-step, with the fragments of the next k-step read
    // under the current one's matrix instructions.  Its last k-step is preceded by the
    // barrier that publishes tile kt+1 (every wavefront has waited for its own copies of
    // it) and frees stage kt % S (every wavefront's reads of it have completed): during that
    // k-step each wavefront reads the first fragments of tile kt+1 and starts the copies of
    // tile kt+S into the freed stage, which continue through the first CSPAN - 1 k-steps of
    // iteration kt+1 and have until the barrier of iteration kt+S-1 to land.  The copies
    // are spread out because the CU moves about one 1 KB copy per 16 cycles: bunched
    // together they stall the wavefront that issues them, and with it its matrix
    // instructions.  Past the end of K the copies repeat the last tile into a stage nobody
    // reads, and the fragments read for a tile nk are never used, so the loop body has no
    // branch.
    if constexpr (TK) {
        // K < 16: no whole k-tile
    } else if constexpr (C::RING) {
        // ---- ring of five half-stages (160 KB at 256 x 256): the A tile of k-tile t lives in
        // buffer 2t mod 5, its B tile in buffer 2t+1 mod 5.  The barrier of iteration kt (before
        // its last k-step) frees both buffers of tile kt.  The B tile of kt+2 is copied into the
        // first during that last k-step and has until the next barrier to land; the A tile of
        // kt+3 is copied into the second during the first SUB-1 k-steps of iteration kt+1 and
        // has until the barrier after next.  Against two whole stages, every copy has one to two
        // k-tiles to arrive instead of one to three k-steps, and a k-tile's copies are spread
        // over all of its k-steps (measured at 4096^3: 2300 instead of 2750 cycles per k-tile,
        // against 2048 of matrix work).
        if (nk > 0) {                         // uniform
            const int last = nk - 1;
            auto read_ring = [&](int abuf, int bbuf, int s, int m, int b) {
                if (m < FM) fa[b][m] = frag_at(smem + abuf * C::A_BYTES + a_off + m * 32 * ROW, s);
                else if (m < C::RD) fb[b][m - FM] = frag_b(bbuf * C::A_BYTES, s, m - FM);
            };
            auto issue_a = [&](int j, int kt, int buf) {
                lds_void* dst = (lds_void*)(smem + buf * C::A_BYTES + (wave * C::A_DMA + j) * 1024);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, aoff[j & 1] + j * astep, kt * ROW, 0, 0);
            };
            auto issue_b = [&](int j, int kt, int buf) {
                lds_void* dst = (lds_void*)(smem + buf * C::A_BYTES + (wave * C::B_DMA + j) * 1024);
                copy_b(j, kt, dst);
            };
            // instruction slots between two copies: B over the last k-step, A over the others
            constexpr int BSL = MF / C::B_DMA, ASL = (SUB - 1) * MF / C::A_DMA;
#pragma unroll
            for (int j = 0; j < C::A_DMA; ++j) issue_a(j, 0, 0);
#pragma unroll
            for (int j = 0; j < C::B_DMA; ++j) issue_b(j, 0, 1);
#pragma unroll
            for (int j = 0; j < C::A_DMA; ++j) issue_a(j, min(1, last), 2);
#pragma unroll
            for (int j = 0; j < C::B_DMA; ++j) issue_b(j, min(1, last), 3);
            // tile 0 landed; tile 1 may be in flight
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(C::A_DMA + C::B_DMA) : "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
#pragma unroll
            for (int m = 0; m < C::RD; ++m) read_ring(0, 1, 0, m, 0);
            int ab = 0;                        // 2 kt mod 5: the A buffer of tile kt
            for (int kt = 0; kt < nk; ++kt) {
                const int bb = ab == 4 ? 0 : ab + 1;                  // B buffer of tile kt
                const int a2 = ab >= 1 ? ab - 1 : 4;                  // 2 kt + 4 mod 5: A of tile kt+2
                const int a1 = ab >= 3 ? ab - 3 : ab + 2;             // 2 kt + 2 mod 5: A of tile kt+1
                const int b1 = a1 == 4 ? 0 : a1 + 1;                  // B of tile kt+1
                const int k2 = min(kt + 2, last);
#pragma unroll
                for (int s = 0; s < SUB - 1; ++s) {
#pragma unroll
                    for (int m = 0; m < MF; ++m) {
#pragma unroll
                        for (int q = 0; q < C::A_DMA; ++q)
                            if (q * ASL == s * MF + m) issue_a(q, k2, a2);
                        read_ring(ab, bb, s + 1, m, (s + 1) & 1);
                        mfma(m, s & 1);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                // tile kt+1 landed (the A copies of tile kt+2 issued above may be in flight);
                // own reads of tile kt complete
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(C::A_DMA) : "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
#pragma unroll
                for (int m = 0; m < MF; ++m) {
#pragma unroll
                    for (int q = 0; q < C::B_DMA; ++q)
                        if (q * BSL == m) issue_b(q, k2, ab);         // B of tile kt+2: 2 kt + 5 mod 5
                    read_ring(a1, b1, 0, m, 0);
                    mfma(m, (SUB - 1) & 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
                ab = a1;
            }
            // the surplus copies land before LDS is reused or released
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        }
    } else if (nk > 0) {                      // uniform
        constexpr int S = C::S;
        const int last = nk - 1;
#pragma unroll
        for (int t = 0; t + 1 < S; ++t)
#pragma unroll
            for (int j = 0; j < C::DMA; ++j) issue_one(j, min(t, last), t);
#pragma unroll
        for (int slot = 0; slot < MF; ++slot) copies_at(slot, min(S - 1, last), S - 1);
        // tile 0 landed: at most tiles 1 .. S-2 and the first copies of tile S-1 pending
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"((S - 2) * C::DMA + C::HEAD) : "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int m = 0; m < C::RD; ++m) read_slot(0, 0, m, 0);
        for (int kt = 0; kt < nk; ++kt) {
            const int st = kt % S, st1 = (kt + 1) % S, stt = (kt + S - 1) % S;
            const int kh = min(kt + S, last), kq = min(kt + S - 1, last);   // head / tail tiles
#pragma unroll
            for (int s = 0; s < SUB - 1; ++s) {
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    if (s < C::CSPAN - 1) copies_at(MF + s * MF + m, kq, stt);
                    read_slot(st, s + 1, m, (s + 1) & 1);
                    mfma(m, s & 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // own copies of tile kt+1 landed (those of tiles kt+2 .. kt+S-1 may not have),
            // own reads of stage st complete; a plain barrier (the compiler's workgroup fence
            // would also wait for the copies still in flight)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"((S - 2) * C::DMA) : "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
#pragma unroll
            for (int m = 0; m < MF; ++m) {
                copies_at(m, kh, st);
                read_slot(st1, 0, m, 0);
                mfma(m, (SUB - 1) & 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the surplus copies land before LDS is reused or released
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }

    // ---- K tail: one more k-tile staged through registers with bounds checks and zero fill
    // into the LDS positions the copies would have filled (stage 0).  Branch-free, so that
    // all loads are in flight together: every lane loads 16 in-bounds bytes -- its chunk
    // when the chunk lies inside K, else the last CE elements of the row -- and keeps what
    // belongs to its chunk (shifted into place for the chunk that straddles K), zero for the
    // rest and for rows past M or N.  Rows shorter than one chunk (8-bit inputs with K < 16,
    // the TK kernel; 16-bit inputs have K >= 64 by the host check) are read byte by byte. ----
    if (p.K % BK != 0) {                      // uniform
        constexpr int CE = 16 / ES;           // elements per 16-byte chunk
        const int k0 = nk * BK;
        uint4 v[C::DMA];
        // the chunk of copy j that this lane stages: its row, first k, row in range
        auto chunk = [&](int j, const unsigned char*& src, int& k, bool& keep) {
            const bool is_a = j < C::A_DMA;
            const int jj = is_a ? j : j - C::A_DMA;
            const int tr = wave * (is_a ? C::A_RPW : C::B_RPW) + jj * C::RPC + lr;
            const int grow = (is_a ? m0 : n0) + tr, rows = is_a ? p.M : p.N;
            src = (is_a ? A : B) + (int64_t)min(grow, rows - 1) * (is_a ? p.lda : p.ldb) * ES;
            k = k0 + CE * ((lane % 8) ^ swz(lr + C::RPC * (jj & 1)));
            keep = grow < rows && k < p.K;
        };
        // BRM: B chunk j of the copy plan, k-row kr of the tile: its source (clamped to an element
        // of B) and whether it lies inside K and N
        auto chunk_rm = [&](int jb, const unsigned char*& src, bool& keep) {
            const int lt = lane_id();         // (formed anew, as in the epilogue)
            const int kr = brm_row0 + jb * RPC2 + lt / (RP / 16);
            const int n = n0 + 8 * ((lt % (RP / 16)) ^ (4 * bsw(kr)));
            src = B + ((int64_t)min(k0 + kr, p.K - 1) * p.ldb + min(n, p.N - 8)) * 2;
            keep = k0 + kr < p.K && n < p.N;
        };
        if constexpr (!TK) {                  // K >= CE (16-bit inputs: K >= 64)
#pragma unroll
            for (int j = 0; j < C::DMA; ++j) {    // all loads first
                const unsigned char* src; int k; bool keep;
                if (BRM && j >= C::A_DMA) {
                    chunk_rm(j - C::A_DMA, src, keep);
                    v[j] = load16(src);
                    continue;
                }
                chunk(j, src, k, keep);
                v[j] = load16(src + (int64_t)(k + CE <= p.K ? k : p.K - CE) * ES);
            }
#pragma unroll
            for (int j = 0; j < C::DMA; ++j) {    // then keep, shift or clear, as arithmetic
                const unsigned char* src; int k; bool keep;
                if (BRM && j >= C::A_DMA) {       // whole k-rows: keep or clear
                    chunk_rm(j - C::A_DMA, src, keep);
                    if (!keep) v[j] = make_uint4(0u, 0u, 0u, 0u);
                    continue;
                }
                chunk(j, src, k, keep);
                // straddling chunk: its r valid elements are the top r of the last CE of the row
                const int r = min(max(p.K - k, 1), CE - 1);
                const unsigned sh = 8 * ES * (CE - r);            // bits to drop, 8 ES .. 128 - 8 ES
                const uint64_t lo = v[j].x | (uint64_t)v[j].y << 32, hi = v[j].z | (uint64_t)v[j].w << 32;
                const uint64_t slo = sh < 64 ? (lo >> sh) | (hi << (64 - sh)) : hi >> (sh - 64);
                const uint64_t shi = sh < 64 ? hi >> sh : 0;
                const uint64_t full = k + CE <= p.K ? ~0ull : 0ull, kept = keep ? ~0ull : 0ull;
                const uint64_t olo = ((lo & full) | (slo & ~full)) & kept, ohi = ((hi & full) | (shi & ~full)) & kept;
                v[j] = make_uint4((unsigned)olo, (unsigned)(olo >> 32), (unsigned)ohi, (unsigned)(ohi >> 32));
            }
        } else {
#pragma unroll
            for (int j = 0; j < C::DMA; ++j) {
                const unsigned char* src; int k; bool keep;
                chunk(j, src, k, keep);
                unsigned w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int b = 0; b < 16; ++b)
                    if (keep && k + b < p.K) w[b / 4] |= (unsigned)src[k + b] << (8 * (b % 4));
                v[j] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        __syncthreads();                      // every wavefront is done with the stages
#pragma unroll
        for (int j = 0; j < C::DMA; ++j) {
            const bool is_a = j < C::A_DMA;
            const int jj = is_a ? j : j - C::A_DMA;
            unsigned char* dst = smem + (is_a ? (wave * C::A_DMA + jj) * 1024
                                              : C::A_BYTES + (wave * C::B_DMA + jj) * 1024) + 16 * lane;
            *reinterpret_cast<uint4*>(dst) = v[j];
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < C::RD; ++m) read_slot(0, 0, m, 0);
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
#pragma unroll
            for (int m = 0; m < MF; ++m) {
                if (s + 1 < SUB) read_slot(0, s + 1, m, (s + 1) & 1);
                mfma(m, s & 1);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    // ---- epilogue: stores past M or N are skipped ----
    // every path stages a 32-row band through LDS and stores whole rows, 16 bytes per lane
    // where C allows (VEC_C) and the four columns lie inside, else element by element
    __builtin_amdgcn_s_barrier();          // every wavefront is done with the stages
    asm volatile("" ::: "memory");
    // the lane's index formed anew rather than kept live across the k-loop
    const int lane_e = lane_id(), l32e = lane_e & 31, he = lane_e >> 5;
    constexpr int LPR = C::WN / 4, RPI = 64 / LPR;   // lanes per C row, rows per store
    constexpr int Q = 32 / RPI;                       // stores per 32-row band
    float* band = reinterpret_cast<float*>(smem) + wave * 32 * C::EP;
    const int cc = 4 * (lane_e % LPR), col = n0 + wn + cc;    // this lane's four columns, every store
    // fused epilogue: a column bias is the same for every store of the lane, loaded once
    float bcol[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (EPI) {
        if (p.e.bias != nullptr && !p.e.bias_rows) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (col + e < p.N) bcol[e] = p.e.bias[col + e];
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                band[(8 * (r >> 2) + 4 * he + (r & 3)) * C::EP + 32 * j + l32e] = acc[i][j][r];
        const int row0 = m0 + wm + 32 * i + lane_e / LPR;     // row of store q: row0 + q RPI
        if constexpr (EPI) {
            // The fused epilogue on the staged values, four columns of a row per store.  C's previous
            // values (beta != 0) and a row bias are loaded one store ahead, so that their latency
            // overlaps the previous store's arithmetic.  The loop stays rolled: unrolled, its code
            // grows enough that the loop over i is left rolled too and the accumulators go to
            // scratch memory.
            auto load_ahead = [&](int q, float (&old)[4], float& brow) {
                const int row = row0 + q * RPI;
                const int64_t off = (int64_t)row * p.ldc + col;
                brow = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) old[e] = 0.f;
                if (row < p.M) {
                    if (p.e.bias != nullptr && p.e.bias_rows) brow = p.e.bias[row];
                    if (p.e.beta != 0.f) {
                        if (VEC_C && (interior || col + 3 < p.N)) {
                            epi_load4(p.e, p.C, off, old);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (col + e < p.N) old[e] = epi_load(p.e, p.C, off + e);
                        }
                    }
                }
            };
            float old_n[4], brow_n;
            if (VEC_C && interior) {      // uniform: every store whole, no bounds to check
                auto load_whole = [&](int q, float (&old)[4], float& brow) {
                    const int row = row0 + q * RPI;
                    brow = p.e.bias != nullptr && p.e.bias_rows ? p.e.bias[row] : 0.f;
                    if (p.e.beta != 0.f) epi_load4(p.e, p.C, (int64_t)row * p.ldc + col, old);
                    else old[0] = old[1] = old[2] = old[3] = 0.f;
                };
                load_whole(0, old_n, brow_n);
#pragma unroll 1
                for (int q = 0; q < Q; ++q) {
                    const float old[4] = {old_n[0], old_n[1], old_n[2], old_n[3]};
                    const float brow = brow_n;
                    if (q + 1 < Q) load_whole(q + 1, old_n, brow_n);
                    const int rr = q * RPI + lane_e / LPR, row = row0 + q * RPI;
                    const f32x4 v = *reinterpret_cast<const f32x4*>(band + rr * C::EP + cc);
                    float y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        y[e] = fmaf(p.e.alpha, v[e], fmaf(p.e.beta, old[e], p.e.bias_rows ? brow : bcol[e]));
                    if (p.e.act == kActRelu) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = fmaxf(y[e], 0.f);
                    } else if (p.e.act == kActGelu) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = gelu(y[e]);
                    }
                    epi_store4(p.e, p.C, (int64_t)row * p.ldc + col, y);
                }
                continue;
            }
            load_ahead(0, old_n, brow_n);
#pragma unroll 1
            for (int q = 0; q < Q; ++q) {
                const float old[4] = {old_n[0], old_n[1], old_n[2], old_n[3]};
                const float brow = brow_n;
                if (q + 1 < Q) load_ahead(q + 1, old_n, brow_n);
                const int rr = q * RPI + lane_e / LPR, row = row0 + q * RPI;
                const f32x4 v = *reinterpret_cast<const f32x4*>(band + rr * C::EP + cc);
                const int64_t off = (int64_t)row * p.ldc + col;
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = epi_apply(p.e, v[e], old[e], p.e.bias_rows ? brow : bcol[e]);
                if (VEC_C && (interior || (row < p.M && col + 3 < p.N))) {
                    epi_store4(p.e, p.C, off, y);
                } else if (row < p.M) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < p.N) epi_store(p.e, p.C, off + e, y[e]);
                }
            }
        } else if constexpr (!VEC_C) {
            // C rows not 16-byte aligned: 4-byte stores with lane l on column 64 c + l of a band
            // row, so that each store instruction writes 256 contiguous bytes (four stores per lane
            // on its own four columns wrote 16-byte-strided pieces: at 4095 x 4097 x 1023 the
            // kernel took 64 us against about 38 for 16-byte rows)
            static_assert(C::WN % 64 == 0, "whole 64-column chunks per band row");
            const int rb = m0 + wm + 32 * i;
#pragma unroll
            for (int r = 0; r < 32; ++r) {
#pragma unroll
                for (int c = 0; c < C::WN / 64; ++c) {
                    const int row = rb + r, cx = n0 + wn + 64 * c + lane_e;
                    const float v = band[r * C::EP + 64 * c + lane_e];
                    if (row < p.M && cx < p.N) {
                        float* dst = p.C + (int64_t)row * p.ldc + cx;
                        if constexpr (BATCH) __builtin_nontemporal_store(v, dst);
                        else *dst = v;
                    }
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int rr = q * RPI + lane_e / LPR, row = row0 + q * RPI;
                const f32x4 v = *reinterpret_cast<const f32x4*>(band + rr * C::EP + cc);
                const int64_t off = (int64_t)row * p.ldc + col;
                if (interior || (row < p.M && col + 3 < p.N)) {
                    // a batch streams C once (attention's scores): non-temporal stores keep it from
                    // displacing the operands in the caches
                    if constexpr (BATCH) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p.C + off));
                    else *reinterpret_cast<f32x4*>(p.C + off) = v;
                } else if (row < p.M) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < p.N) p.C[off + e] = v[e];
                }
            }
        }
    }
}

// One launch of configuration C in mode MODE for input type `it`: tiles along x, grid_y K
// slices, grid_z batch entries.  16-bit inputs with row-major B take the BRM build.
template <typename C, int MODE, int IT, bool TK = false>
hipError_t launch_it(const typename ModeArgT<MODE>::type& p, const Launch& l, int grid_y) {
    const int tiles_m = (p.M + C::BM - 1) / C::BM, tiles_n = (p.N + C::BN - 1) / C::BN;
    const dim3 grid((unsigned)tiles_m * tiles_n, (unsigned)grid_y, MODE == kBatched ? l.batch : 1), block(C::THREADS);
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, block, 0, l.stream, p, tiles_m, tiles_n, l.group_m);
        return hipGetLastError();
    };
    if constexpr (C::ES == 2) {
        if (p.ob == kRow)
            return l.vec_c ? go(k_bf16_dma<C, true, IT, MODE, TK, true>) : go(k_bf16_dma<C, false, IT, MODE, TK, true>);
    }
    return l.vec_c ? go(k_bf16_dma<C, true, IT, MODE, TK>) : go(k_bf16_dma<C, false, IT, MODE, TK>);
}

template <typename C, int MODE, bool TK = false>
hipError_t launch_cfg(const typename ModeArgT<MODE>::type& p, const Launch& l, int it, int grid_y = 1) {
    if constexpr (C::ES == 2) {
        if (it == kInBf16) return launch_it<C, MODE, kInBf16>(p, l, grid_y);
        if (it == kInF16) return launch_it<C, MODE, kInF16>(p, l, grid_y);
    } else {
        switch (it) {
            case kInFp8 + 0: return launch_it<C, MODE, kInFp8 + 0, TK>(p, l, grid_y);
            case kInFp8 + 1: return launch_it<C, MODE, kInFp8 + 1, TK>(p, l, grid_y);
            case kInFp8 + 2: return launch_it<C, MODE, kInFp8 + 2, TK>(p, l, grid_y);
            case kInFp8 + 3: return launch_it<C, MODE, kInFp8 + 3, TK>(p, l, grid_y);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

template <typename C>
hipError_t launch_any(const Problem& p, const Launch& l, int it) {
    if (l.batch > 1) return launch_cfg<C, kBatched>(batch_arg(p, l, C::ES), l, it);
    return launch_cfg<C, kPlain>(p, l, it);
}

int in16(bool f16) { return f16 ? kInF16 : kInBf16; }

}  // namespace

bool bf16_dma_applies(const Problem& p, const Launch&, int, int) {
    // one bound for both configurations: 64 rows per wavefront copy block at most.  Row-major B
    // (the BRM build): whole 8-column chunks (N % 8 == 0), and byte offsets into B up to element
    // (K-1, N-1) below 2^31
    const int64_t lim = (int64_t)1 << 31;
    if (p.oa != kRow || p.K < 64 || (int64_t)64 * p.lda * 2 >= lim) return false;
    if (p.ob == kRow) return p.N % 8 == 0 && ((int64_t)(p.K - 1) * p.ldb + p.N) * 2 < lim;
    return p.ob == kCol && (int64_t)64 * p.ldb * 2 < lim;
}

bool fp8_dma_applies(const Problem& p) {
    const int64_t lim = (int64_t)1 << 31;
    return p.oa == kRow && p.ob == kCol && p.K >= 1 && (int64_t)64 * p.lda < lim && (int64_t)64 * p.ldb < lim;
}

// Configurations.  256 x 256: four wavefronts of 128 x 128 (one per SIMD, 256 accumulators
// each in accumulation registers) on the five-buffer ring (160 KB of LDS).  Against eight
// wavefronts of 128 x 64 on two whole stages (the previous layout) it reads a third less from LDS
// per product, and the ring gives every copy one to two k-tiles to land: at 4096^3,
// interleaved with the FP32 GEMM as the benchmark step runs them, 116 -> 108 us (2750 -> 2300
// cycles per k-tile against 2048 of matrix work; the shader clock, set by the power limit, went
// 1.79 -> 1.68 GHz).  256 x 128: eight wavefronts of 64 x 64 and three whole stages (144 KB),
// the copies spread over four k-steps (1350 cycles per k-tile against 1024; four wavefronts of
// 128 x 64: 1425 with three stages, 1540-1630 with two).
hipError_t launch_bf16_dma(const Problem& p, const Launch& l, int bm, int bn, bool f16) {
    if (bm == 256 && bn == 256) return launch_any<Cfg256>(p, l, in16(f16));
    if (bm == 256 && bn == 128) return launch_any<Cfg<256, 128, 4, 2, 4, 3>>(p, l, in16(f16));
    return hipErrorInvalidValue;
}

hipError_t launch_bf16_dma_epi(const EpiProblem& p, const Launch& l, int bm, int bn, bool f16) {
    if (bm == 256 && bn == 256) return launch_cfg<Cfg256, kEpilogue>(p, l, in16(f16));
    if (bm == 256 && bn == 128) return launch_cfg<Cfg<256, 128, 4, 2, 4, 3>, kEpilogue>(p, l, in16(f16));
    return hipErrorInvalidValue;
}

// Split-K: s.part holds the slabs of slices 1 .. S-1 (16-byte aligned; l.vec_c also covers their
// rows, N % 4 == 0), then the slabs are added to C in slice order.
hipError_t launch_bf16_dma_split(const SplitProblem& s, int slices, const Launch& l, int bm, int bn, bool f16) {
    hipError_t err = hipErrorInvalidValue;
    if (bm == 256 && bn == 256) err = launch_cfg<Cfg256, kSplitK>(s, l, in16(f16), slices);
    else if (bm == 256 && bn == 128) err = launch_cfg<Cfg<256, 128, 4, 2, 4, 3>, kSplitK>(s, l, in16(f16), slices);
    if (err != hipSuccess) return err;
    return launch_add_slabs(s.C, s.ldc, s.M, s.N, s.part, slices - 1, l);
}

// 8-bit inputs (format codes 0 E4M3, 1 E5M2) on the same skeleton: a k-tile is 128 deep, one
// 32 x 32 x 64 matrix instruction per fragment pair and k-step, with unit block scales.
hipError_t launch_fp8_dma(const Problem& p, const Launch& l, int bm, int bn, int fmt_a, int fmt_b) {
    if ((fmt_a != 0 && fmt_a != 1) || (fmt_b != 0 && fmt_b != 1)) return hipErrorInvalidValue;
    const int it = kInFp8 + 2 * fmt_a + fmt_b;
    if (p.K < 16) return launch_cfg<Cfg256x128F8, kPlain, true>(p, l, it);     // either tile: no k-loop
    if (bm == 256 && bn == 256) return launch_cfg<Cfg256F8, kPlain>(p, l, it);
    if (bm == 256 && bn == 128) return launch_cfg<Cfg256x128F8, kPlain>(p, l, it);
    return hipErrorInvalidValue;
}

}  // namespace gemm
