// Shared definitions of libgemm's kernels: the normalised problem descriptor and the
// tile scheduler.  Everything here is device/host plumbing; no arithmetic of C = A.B.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gemm {

enum Order : int { kRow = 0, kCol = 1 };

// A problem after the host has normalised it: C is row-major M x N with leading
// dimension ldc (a column-major C is handled by computing C^T = B^T A^T instead).
// A (M x K) and B (K x N) keep their own order and leading dimension.  Sizes fit in
// int32 (checked on the host); offsets are formed in int64.
struct Problem {
    int M, N, K;
    const void* A;
    int64_t lda;
    int oa;
    const void* B;
    int64_t ldb;
    int ob;
    float* C;
    int64_t ldc;
};

// A strided batch of problems of one shape: entry z reads A + z*sa and B + z*sb (bytes) and
// writes C + z*sc (floats).  The batched instantiation of a kernel takes its entry from
// blockIdx.z and moves the three pointers before anything else; the plain instantiation takes
// a Problem and has no such step.
struct BatchProblem : Problem {
    int64_t sa, sb, sc;
    __device__ __forceinline__ void select(int64_t z) {
        A = static_cast<const char*>(A) + z * sa;
        B = static_cast<const char*>(B) + z * sb;
        C += z * sc;
    }
};
template <bool BATCH> using KArg = std::conditional_t<BATCH, BatchProblem, Problem>;

// One problem with K split across workgroups ("A06 - Tiled Matrix Multiply (GEMM)", "The next
// two rungs": split-K, each worker sums part of K and a second step adds the partial sums).
// Slice z (blockIdx.y) takes k in [z kslice, min(K, (z+1) kslice)); slice 0 writes C, slice
// z >= 1 the dense M x N slab part + (z-1) M N (leading dimension N), which a second kernel adds
// to C in slice order.
struct SplitProblem : Problem {
    int kslice;
    float* part;
    __device__ __forceinline__ void select(int z, int elem_bytes) {
        const int64_t k0 = (int64_t)z * kslice;
        A = static_cast<const char*>(A) + (oa == kRow ? k0 : k0 * lda) * elem_bytes;
        B = static_cast<const char*>(B) + (ob == kCol ? k0 : k0 * ldb) * elem_bytes;
        K = (int)(K - k0 < kslice ? K - k0 : kslice);
        if (z > 0) {
            C = part + (int64_t)(z - 1) * M * N;
            ldc = N;
        }
    }
};

// Instantiation kinds of a tile kernel and the argument each takes.
enum KernelMode : int { kPlain = 0, kBatched = 1, kEpilogue = 2, kSplitK = 3 };
template <int MODE> struct ModeArgT { using type = Problem; };
template <> struct ModeArgT<kBatched> { using type = BatchProblem; };
template <> struct ModeArgT<kSplitK> { using type = SplitProblem; };

// Offset of logical element (r, c) in an operand with leading dimension ld and order o.
__device__ __forceinline__ int64_t elem_offset(int64_t r, int64_t c, int64_t ld, int o) {
    return o == kRow ? r * ld + c : r + c * ld;
}

// ---------------------------------------------------------------------------------------
// Tile scheduler: linear workgroup id -> (tile row, tile column) of C.
//
// Two remaps, both bijections on [0, tiles):
//  1. XCD grouping.  MI355X has 8 XCDs, each with its own L2, and the dispatcher hands
//     consecutive workgroup ids to the XCDs in turn (id w runs on XCD w % 8).  The remap
//     renumbers ids so that the workgroups resident on one XCD receive consecutive
//     logical tile numbers, i.e. neighbouring tiles of C that share A row-panels and B
//     column-panels sit behind the same L2.
//  2. Group-M ordering.  Logical tile numbers run down a band of `group_m` tile rows
//     before moving one tile column right, so a run of consecutive numbers covers a
//     near-square patch of C instead of one long row.
// The pages describe the second idea for one shared L2 ("GEMM Optimization", section "L2
// Cache and Wave Analysis"; "GEMM, step by step", Concept: neighbouring blocks working on
// the same rows and columns); the first is what it takes on a chip with eight L2s.
// ---------------------------------------------------------------------------------------
constexpr int kNumXcds = 8;

// Group-M order: logical tile id -> (tile row, tile column).
__host__ __device__ __forceinline__ void band_coords(int id, int tiles_m, int tiles_n, int group_m, int& tile_m,
                                                     int& tile_n) {
    const int band = group_m * tiles_n;
    const int first_m = (id / band) * group_m;
    const int rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int in_band = id % band;
    tile_m = first_m + in_band % rows;
    tile_n = in_band / rows;
}

// group_m <= 0 turns both remaps off (tiles in plain row-major order of workgroup ids), for
// measuring what they are worth.
__host__ __device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n,
                                                     int group_m, int& tile_m, int& tile_n) {
    if (group_m <= 0) {
        tile_m = wg / tiles_n;
        tile_n = wg % tiles_n;
        return;
    }
    const int total = tiles_m * tiles_n;
    const int per_xcd = total / kNumXcds;
    int id = wg;
    if (wg < per_xcd * kNumXcds) id = (wg % kNumXcds) * per_xcd + wg / kNumXcds;
    band_coords(id, tiles_m, tiles_n, group_m, tile_m, tile_n);
}

// A strided-batch launch has the tiles of one entry along x and the entries along z; the
// dispatcher numbers workgroups x first (id x + tiles z).  An entry of at least 16 tiles is
// grouped on its own, as one problem (each XCD takes a patch of every entry).  Fewer tiles would
// leave at most one of an entry's tiles per XCD: then the XCD grouping runs over the tiles of all
// entries in dispatch order, so that the workgroups on one XCD take whole entries, whose tiles
// share the entry's operand panels; group-M order within the entry.  (Measured on attention,
// 32 entries: P.V, 8 tiles of 256 x 128 per entry, 83.4 -> 78.9 us, its B fetched once instead
// of by every L2; the scores Q.K^T, 64 tiles of 256^2, 130 us grouped per entry against 134 us
// by whole entries.)  (bx, bz): the workgroup's x and z, nz entries.  group_m <= 0: entry bz,
// tiles in row-major order.
__host__ __device__ __forceinline__ void batch_tile_coords(int bx, int bz, int nz, int tiles_m, int tiles_n,
                                                           int group_m, int& entry, int& tile_m, int& tile_n) {
    if (group_m <= 0 || tiles_m * tiles_n >= 2 * kNumXcds) {
        entry = bz;
        tile_coords(bx, tiles_m, tiles_n, group_m, tile_m, tile_n);
        return;
    }
    const int64_t per = (int64_t)tiles_m * tiles_n, total = per * nz;
    const int64_t wg = bx + per * bz;
    const int64_t per_xcd = total / kNumXcds;
    int64_t id = wg;
    if (wg < per_xcd * kNumXcds) id = (wg % kNumXcds) * per_xcd + wg / kNumXcds;
    entry = (int)(id / per);
    band_coords((int)(id - entry * per), tiles_m, tiles_n, group_m, tile_m, tile_n);
}

// Launch options the host chooses per call.
struct Launch {
    hipStream_t stream;
    int group_m;        // tile-scheduler band height (>= 1)
    bool vec_a, vec_b;  // 16-byte loads of the operand are allowed (load16 / load16f)
    bool vec_c;         // C pointer and ldc allow 16-byte stores
    int batch = 1;      // entries of a strided batch (gridDim.z); 1: one problem
    int64_t sa = 0, sb = 0, sc = 0;   // element strides between entries (A, B; C in floats)
};

// The kernel argument of a batched launch: strides of A and B turned into bytes.
inline BatchProblem batch_arg(const Problem& p, const Launch& l, int elem_bytes) {
    BatchProblem b{};
    static_cast<Problem&>(b) = p;
    b.sa = l.sa * elem_bytes;
    b.sb = l.sb * elem_bytes;
    b.sc = l.sc;
    return b;
}

// 16-byte global loads from addresses aligned to the element only.  gfx950 serves unaligned
// vector loads from global memory, and its 16-byte global->LDS copies too (the parity tests
// with padded and odd leading dimensions cover both), so operands whose rows are not
// 16-byte aligned still move 16 bytes per lane.
typedef unsigned int u32x4_ua __attribute__((ext_vector_type(4), aligned(2)));
typedef float f32x4_ua __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ uint4 load16(const void* p) {
    const u32x4_ua v = *reinterpret_cast<const u32x4_ua*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load16f(const float* p) {
    const f32x4_ua v = *reinterpret_cast<const f32x4_ua*>(p);
    return make_float4(v.x, v.y, v.z, v.w);
}

}  // namespace gemm
