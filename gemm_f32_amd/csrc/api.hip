// libgemm's C ABI: argument validation, normalisation of a column-major C, kernel choice
// and launch.  The operation and its contract are documented in include/gemm.h.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gemm.h"
#include "common.hpp"
#include "launch.hpp"

// Scratch memory of gemm_bf16_f32acc_noalloc: the split-K partial sums that the _ws calls keep
// in a caller's workspace, here in a fixed array of device memory.  Every GPU the library runs
// on holds its own copy until the process ends.  In host code this name only stands for the
// array; the device address of the current device's copy comes from hipGetSymbolAddress
// (scratch_address below), and only that address is passed to kernels.
constexpr size_t kScratchBytes = GEMM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace gemm {
namespace {

thread_local int t_last_hip_error = 0;
thread_local const char* t_last_kernel = "none";

enum class In { F32, BF16, F16, FP8 };

int elem_of(In in) {
    return in == In::F32 ? kElemF32 : in == In::BF16 ? kElemBf16 : in == In::F16 ? kElemF16 : kElemFp8;
}

struct DeviceInfo {
    bool supported = false;
    int cus = 0;
};

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];

// Per-device properties, queried once.  Returns false if the device cannot be queried.
bool device_info(DeviceInfo& out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
    std::call_once(g_dev_once[dev], [dev] {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
            g_dev[dev].supported = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            g_dev[dev].cus = prop.multiProcessorCount;
        }
    });
    out = g_dev[dev];
    return true;
}

// The device address of the current device's copy of `scratch`, looked up once per device
// with that device current (the lookup's error is kept and returned on every later call).
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

hipError_t scratch_address(void*& ptr) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    ptr = g_scratch_ptr[dev];
    return g_scratch_err[dev];
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

gemm_status_t validate(In in, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                       int oa, const void* B, int64_t ldb, int ob, const void* C, int64_t ldc,
                       int oc, uintptr_t c_align = 4) {
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_VALUE;
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return GEMM_ERR_INVALID_VALUE;
    for (int o : {oa, ob, oc})
        if (o != GEMM_ROW_MAJOR && o != GEMM_COL_MAJOR) return GEMM_ERR_INVALID_VALUE;
    auto at_least = [](int64_t v) { return v > 1 ? v : 1; };
    if (lda < at_least(oa == GEMM_ROW_MAJOR ? K : M)) return GEMM_ERR_INVALID_VALUE;
    if (ldb < at_least(ob == GEMM_ROW_MAJOR ? N : K)) return GEMM_ERR_INVALID_VALUE;
    if (ldc < at_least(oc == GEMM_ROW_MAJOR ? N : M)) return GEMM_ERR_INVALID_VALUE;
    if (M > 0 && N > 0 && C == nullptr) return GEMM_ERR_INVALID_VALUE;
    if (M > 0 && N > 0 && K > 0 && (A == nullptr || B == nullptr)) return GEMM_ERR_INVALID_VALUE;
    const uintptr_t e = in == In::F32 ? 4 : in == In::FP8 ? 1 : 2;
    if (!aligned(A, e) || !aligned(B, e) || !aligned(C, c_align)) return GEMM_ERR_INVALID_VALUE;
    return GEMM_OK;
}

// GEMM_TILE_ORDER=rowmajor in the environment (read once) turns the tile scheduler's remaps
// off, so that what they buy can be measured.
bool plain_tile_order() {
    static const bool plain = [] {
        const char* v = std::getenv("GEMM_TILE_ORDER");
        return v != nullptr && std::strcmp(v, "rowmajor") == 0;
    }();
    return plain;
}

int pick_group_m(int tiles_m, int tiles_n) {
    if (plain_tile_order()) return 0;
    // Make the run of tiles that one XCD receives (total / 8 consecutive ids) cover a
    // near-square patch of C: group_m x (per_xcd / group_m) tiles.
    const int per_xcd = (tiles_m * tiles_n) / kNumXcds;
    int g = 1;
    while (2 * g <= tiles_m && (2 * g) * (2 * g) <= per_xcd) g *= 2;
    return g;
}

int64_t tiles(int64_t M, int64_t N, int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); }

// AUTO takes the small-problem kernel for few rows, when even 64 x 64 tiles would leave more
// than half of the CUs idle (each such tile walks all of K alone), or when 128 x 128 tiles
// cannot give every CU one while the small-problem kernel's 64 x 64 blocks still fit in one
// round: its K split over eight wavefronts then beats the tile kernels, whose few tiles each
// wait on memory latency (rocprofv3: 1000^3 FP32 58 -> 40 us, BF16 16.2 -> 13.9 us;
// 1024 x 1024 x 4096 BF16 46.6 -> 36.6 us).  With more blocks than CUs it loses
// (1500 x 1500 x 512: FP32 58 against 49 us, BF16 29 against 13 us).
bool prefer_small(const Problem& p, int cus) {
    const int64_t c = cus > 0 ? cus : 256;
    const int64_t t64 = tiles(p.M, p.N, 64, 64);
    return p.M <= kSkinnyMaxM || t64 * 2 < c || (tiles(p.M, p.N, 128, 128) < c && t64 <= c);
}

// 16-bit inputs: where the small-problem kernel would run for lack of tiles but its 64-column
// blocks would not give every CU one (it then falls back to 16-column blocks, several rounds of
// them), the register-staged kernel's 64 x 64 tiles run faster as long as they still occupy at
// least half of the CUs in one round and K is at most 2048.  rocprofv3 kernel times, BF16, operands
// rotating over more than 512 MB as in the benchmark (small-problem -> 64 x 64 tiles): 768^3 20.5 ->
// 11.5 us, 800 x 1200 x 1000 28.9 -> 16.1.  Where the 64-column blocks fill the CUs the small-problem
// kernel stays (1000^3 14.1 against 16.4 us, 1024 x 1024 x 2048 23.3 against 25.6).
constexpr int64_t kSmallTileMaxK = 2048;
bool small_tiles16(const Problem& p, int cus) {
    const int64_t c = cus > 0 ? cus : 256, t64 = tiles(p.M, p.N, 64, 64);
    return p.M > kSkinnyMaxM && 2 * t64 >= c && t64 < c && p.K <= kSmallTileMaxK;
}

// Kernel names as gemm_last_kernel() reports them: the input type, then the kernel.
const char* skinny_name(int et, int fn) {
    static const char* names[3][2] = {{"f32_skinny16", "f32_skinny64"}, {"bf16_skinny16", "bf16_skinny64"},
                                      {"f16_skinny16", "f16_skinny64"}};
    return names[et][fn == 4 ? 1 : 0];
}

// FP32, few rows, row-major B: two K halves of 32-column blocks added into a zeroed C
constexpr const char* kSkinnyHalvesName = "f32_skinny32_halves";
// 32-column blocks over the whole of K where 16-column blocks would take more than one round
constexpr const char* kSkinnyPairsNames[3] = {"f32_skinny32", "bf16_skinny32", "f16_skinny32"};

// A strided batch on the normalised problem (element strides; C's in floats); n == 1: one problem.
struct Batch {
    int64_t n = 1, sa = 0, sb = 0, sc = 0;
};

// A caller's workspace (gemm_*_ws); empty for the plain entry points.
struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};

// The split the small-problem kernel takes with this workspace (slices == 1: none).
SkinnySplit split_with(const Problem& p, int et, int cus, const Workspace& ws) {
    if (ws.ptr == nullptr || !aligned(ws.ptr, 16)) return SkinnySplit{};
    const SkinnySplit sp = skinny_split(p, et != kElemF32, cus);
    return sp.slices > 1 && sp.bytes <= ws.bytes ? sp : SkinnySplit{};
}

// The small-problem kernel, with 1 or 4 column blocks of 16 per workgroup; `choose`: the default
// choice, which also takes the two-halves mode where it applies (a forced GEMM_ALGO_SKINNY keeps
// the plain blocks).
hipError_t run_skinny(const Problem& p, const Launch& l, int et, int cus, const char*& name,
                      const Workspace& ws = Workspace{}, bool choose = false) {
    const SkinnySplit sp = split_with(p, et, cus, ws);
    if (sp.slices > 1) {       // K split across workgroups too: partial products in the workspace
        static const char* names[3] = {"f32_skinny64_splitk", "bf16_skinny64_splitk", "f16_skinny64_splitk"};
        name = names[et];
        return launch_skinny(p, l, et, sp.fn, sp.fm, &sp, static_cast<float*>(ws.ptr));
    }
    if (choose && et == kElemF32 && l.batch == 1 && l.vec_a && skinny_halves_applies(p, cus)) {
        name = kSkinnyHalvesName;
        return launch_skinny_halves(p, l);
    }
    if (choose && l.batch == 1 && l.vec_a && skinny_pairs_applies(p, et, cus)) {
        name = kSkinnyPairsNames[et];
        return launch_skinny_pairs(p, l, et);
    }
    const int fn = skinny_blocks(p, cus);
    name = skinny_name(et, fn);
    return launch_skinny(p, l, et, fn, skinny_strips(p, fn, cus));
}

// Block-tile choice.  The grid runs in rounds of cus x per_cu resident blocks (per_cu: how
// many blocks of that kernel share a CU); a CU's round costs (blocks it holds) x (work per
// tile / relative throughput of the kernel and tile), so estimate time as the sum over rounds
// and take the cheapest.  Relative throughputs are the kernels' measured rates at 4096^3 with
// full rounds, against the fastest kernel of the dtype.
struct TileOpt {
    int bm, bn;
    double eff;
    int per_cu;
    bool dma;       // the direct-copy kernel (else the register-staged one)
};
// FP32: direct-copy 256^2 and 128^2, register-staged 128^2 and 64^2 (f32_mfma.hip)
constexpr TileOpt kF32DmaOpts[] = {{256, 256, 1.0, 1, true}, {128, 128, 0.85, 2, true}};
constexpr TileOpt kF32MfmaOpts[] = {{128, 128, 0.85, 4, false}, {64, 64, 0.75, 4, false}};
// BF16: direct-copy 256^2 and 256x128, register-staged tiles of bf16_mfma.hip
constexpr TileOpt kBf16DmaOpts[] = {{256, 256, 1.0, 1, true}, {256, 128, 0.71, 1, true}};
constexpr TileOpt kBf16MfmaOpts[] = {{256, 128, 0.72, 1, false}, {128, 128, 0.69, 2, false},
                                     {64, 64, 0.33, 4, false}};

double round_cost(int64_t n, int bm, int bn, double eff, int per_cu, int cus) {
    const double c = cus > 0 ? cus : 256;
    const double full = std::floor((double)n / (c * per_cu)), rest = (double)n - full * c * per_cu;
    return (full * per_cu + std::ceil(rest / c)) * bm * bn / eff;
}

// A kernel's launch over a core of C (rows 0 .. mc-1, columns 0 .. nc-1) plus the strips
// that complete it, each a separate GEMM through the same choice on the same stream, run after
// the core.  Per edge the core either ends with tiles that overhang it (where the kernel allows:
// part_m / part_n), or stops at the last whole tile, or stops after the tiles that fill exactly
// one round of the CUs (the rest of the edge becomes a strip for smaller tiles).  4095 x 4097 on
// 256^2 tiles: 16 x 16 tiles (one round) and a one-column strip, against 16 x 17 tiles (two
// rounds); 2048 x 11008 BF16: 8 x 32 tiles of 256^2 (one round) and a 2048 x 2816 strip on
// 256 x 128 tiles (one round), against 688 tiles of 256 x 128 (2.7 rounds).
struct Plan {
    TileOpt opt{};
    int mc = 0, nc = 0;
    double cost = 1e300;
};

// A strip's price: its cheapest option among the given tile kernels, in rounds.
struct StripPricer {
    const TileOpt* a;
    int na;
    const TileOpt* b;
    int nb;
    int cus;
    double operator()(int64_t m, int64_t n) const {
        double best = 1e300;
        for (int i = 0; i < na + nb; ++i) {
            const TileOpt& o = i < na ? a[i] : b[i - na];
            best = std::min(best, round_cost(tiles(m, n, o.bm, o.bn), o.bm, o.bn, o.eff, o.per_cu, cus));
        }
        return best;
    }
};

Plan plan_core(const Problem& p, const TileOpt& o, bool part_m, bool part_n, int cus, const StripPricer& strip) {
    Plan best;
    best.opt = o;
    const int64_t slots = (int64_t)(cus > 0 ? cus : 256) * o.per_cu;    // blocks in one round
    auto consider = [&](int mc, int nc) {
        if (mc <= 0 || nc <= 0 || mc > p.M || nc > p.N) return;
        // a core ends on a tile boundary, except where its last tiles may overhang C's edge
        if ((mc % o.bm && (mc < p.M || !part_m)) || (nc % o.bn && (nc < p.N || !part_n))) return;
        double c = round_cost(tiles(mc, nc, o.bm, o.bn), o.bm, o.bn, o.eff, o.per_cu, cus);
        if (mc < p.M) c += strip(p.M - mc, p.N);
        if (nc < p.N) c += strip(mc, p.N - nc);
        if (c < best.cost) { best.cost = c; best.mc = mc; best.nc = nc; }
    };
    int ms[2], ns[2], nm = 0, nn = 0;
    if (part_m) ms[nm++] = p.M;
    ms[nm++] = p.M / o.bm * o.bm;
    if (part_n) ns[nn++] = p.N;
    ns[nn++] = p.N / o.bn * o.bn;
    for (int i = 0; i < nm; ++i)
        for (int j = 0; j < nn; ++j) consider(ms[i], ns[j]);
    // one round exactly: as many tiles along one edge as fill the CUs with the other edge's
    for (int i = 0; i < nm; ++i) {
        const int64_t tm = (ms[i] + o.bm - 1) / o.bm;
        if (tm > 0) consider(ms[i], (int)std::min<int64_t>(p.N, slots / tm * o.bn));
    }
    for (int j = 0; j < nn; ++j) {
        const int64_t tn = (ns[j] + o.bn - 1) / o.bn;
        if (tn > 0) consider((int)std::min<int64_t>(p.M, slots / tn * o.bm), ns[j]);
    }
    return best;
}

// A kernel that takes any shape: the whole of C is its core.
Plan plan_whole(const Problem& p, const TileOpt& o, int cus) {
    Plan pl;
    pl.opt = o;
    pl.mc = p.M;
    pl.nc = p.N;
    pl.cost = round_cost(tiles(p.M, p.N, o.bm, o.bn), o.bm, o.bn, o.eff, o.per_cu, cus);
    return pl;
}

// Options for a (sub-)problem whose C starts at p.C: 16-byte stores need an aligned C and
// ldc; 16-byte loads and global->LDS copies need only element alignment on gfx950.
Launch launch_for(const Problem& p, hipStream_t stream, const Batch& b = Batch{}) {
    Launch o{};
    o.stream = stream;
    o.vec_a = o.vec_b = true;
    o.vec_c = (p.ldc % 4 == 0) && aligned(p.C, 16) && (b.n == 1 || b.sc % 4 == 0);
    o.batch = (int)b.n;
    o.sa = b.sa;
    o.sb = b.sb;
    o.sc = b.sc;
    return o;
}

// Sub-problem: rows r0 .. r0+m-1 and columns c0 .. c0+n-1 of C (row-major C).
Problem sub_problem(const Problem& p, int r0, int m, int c0, int n, int elem) {
    Problem s = p;
    s.M = m;
    s.N = n;
    const char* A = static_cast<const char*>(p.A);
    const char* B = static_cast<const char*>(p.B);
    s.A = A + (p.oa == kRow ? (int64_t)r0 * p.lda : (int64_t)r0) * elem;
    s.B = B + (p.ob == kCol ? (int64_t)c0 * p.ldb : (int64_t)c0) * elem;
    s.C = p.C + (int64_t)r0 * p.ldc + c0;
    return s;
}

hipError_t dispatch(const Problem& p, hipStream_t stream, gemm_algo_t algo, int et, const DeviceInfo& dev,
                    const char*& name, gemm_status_t& st, const Workspace& ws = Workspace{},
                    const Batch& b = Batch{});

// Run a plan's core with `core` and its strips through the default choice, on one stream.
template <typename CoreFn>
hipError_t run_plan(const Problem& p, hipStream_t stream, const Plan& pl, int et, const DeviceInfo& dev,
                    const Batch& b, CoreFn core) {
    const int e = et == kElemF32 ? 4 : 2;
    const Problem c = sub_problem(p, 0, pl.mc, 0, pl.nc, e);
    Launch lc = launch_for(c, stream, b);
    lc.group_m = pick_group_m((c.M + pl.opt.bm - 1) / pl.opt.bm, (c.N + pl.opt.bn - 1) / pl.opt.bn);
    hipError_t err = core(c, lc);
    const char* ignored = nullptr;
    gemm_status_t st = GEMM_OK;
    if (err == hipSuccess && pl.mc < p.M)        // rows mc .. M-1, all columns
        err = dispatch(sub_problem(p, pl.mc, p.M - pl.mc, 0, p.N, e), stream, GEMM_ALGO_AUTO, et, dev, ignored, st,
                       Workspace{}, b);
    if (err == hipSuccess && pl.nc < p.N)        // rows 0 .. mc-1, columns nc .. N-1
        err = dispatch(sub_problem(p, 0, pl.mc, pl.nc, p.N - pl.nc, e), stream, GEMM_ALGO_AUTO, et, dev, ignored, st,
                       Workspace{}, b);
    return err;
}

const char* f32_name(const TileOpt& o) {
    if (o.dma) return o.bm == 256 ? "f32_dma256x256" : "f32_dma128x128";
    return o.bm == 64 ? "f32_mfma64x64" : "f32_mfma128x128";
}
const char* b16_name(const TileOpt& o, int et) {
    static const char* names[2][5] = {
        {"bf16_dma256x256", "bf16_dma256x128", "bf16_mfma256x128", "bf16_mfma128x128", "bf16_mfma64x64"},
        {"f16_dma256x256", "f16_dma256x128", "f16_mfma256x128", "f16_mfma128x128", "f16_mfma64x64"}};
    const int i = o.dma ? (o.bn == 256 ? 0 : 1) : (o.bm == 256 ? 2 : (o.bm == 128 ? 3 : 4));
    return names[et == kElemF16 ? 1 : 0][i];
}

// The FP32 matrix-core kernels: the cheapest plan over the allowed options.
Plan choose_f32_tiles(const Problem& p, gemm_algo_t algo, int cus) {
    const Launch l = launch_for(p, nullptr);
    const bool part_m = p.oa == kRow, part_n = p.ob == kCol;   // k-contiguous operands
    const StripPricer f32_strips{kF32DmaOpts, 2, kF32MfmaOpts, 2, cus};
    Plan best;
    auto consider = [&](const Plan& pl) { if (pl.cost < best.cost) best = pl; };
    const bool any = algo == GEMM_ALGO_AUTO || algo == GEMM_ALGO_MFMA;
    for (const TileOpt& o : kF32DmaOpts) {
        const bool want = any || algo == GEMM_ALGO_MFMA_DMA || (algo == GEMM_ALGO_MFMA_256x256 && o.bm == 256);
        if (want && f32_dma_applies(p, l, o.bm, o.bn))
            consider(plan_core(p, o, part_m, part_n, cus, f32_strips));
    }
    for (const TileOpt& o : kF32MfmaOpts) {
        const bool want = any || (algo == GEMM_ALGO_MFMA_128x128 && o.bm == 128) ||
                          (algo == GEMM_ALGO_MFMA_64x64 && o.bm == 64);
        if (want) consider(plan_whole(p, o, cus));
    }
    return best;
}

// A split of K over the tiles of the direct-copy kernels (slices == 1: none), the workspace it
// needs and its slice depth; chosen by tile_split (16-bit) and f32_tile_split below.
struct TileSplit {
    int slices = 1, kslice = 0;
    size_t bytes = 0;
};
TileSplit tile_split_with(const Problem& p, int cus, const Workspace& ws, bool f32);

hipError_t run_f32_tiles(const Problem& p, hipStream_t stream, gemm_algo_t algo, const DeviceInfo& dev,
                         const char*& name, gemm_status_t& st, const Batch& b, const Workspace& ws = Workspace{}) {
    const Plan best = choose_f32_tiles(p, algo, dev.cus);
    if (best.cost >= 1e300) { st = GEMM_ERR_INVALID_VALUE; return hipSuccess; }
    if (algo == GEMM_ALGO_AUTO && b.n == 1) {
        const TileSplit t = tile_split_with(p, dev.cus, ws, true);
        if (t.slices > 1) {
            SplitProblem sp{};
            static_cast<Problem&>(sp) = p;
            sp.kslice = t.kslice;
            sp.part = static_cast<float*>(ws.ptr);
            Launch l = launch_for(p, stream);
            l.vec_c = l.vec_c && p.N % 4 == 0;
            l.group_m = pick_group_m(p.M / 256, p.N / 256);
            name = "f32_dma256x256_splitk";
            return launch_f32_dma_split(sp, t.slices, l);
        }
    }
    name = f32_name(best.opt);
    const TileOpt o = best.opt;
    return run_plan(p, stream, best, kElemF32, dev, b, [&](const Problem& c, const Launch& lc) {
        return o.dma ? launch_f32_dma(c, lc, o.bm, o.bn) : launch_f32_mfma(c, lc, o.bm);
    });
}

// The BF16 tile kernels: the direct-copy kernel where it applies (any M, N: its tiles may
// overhang both edges), else, or for an explicitly chosen tile, the register-staged kernels.
Plan choose_bf16_tiles(const Problem& p, gemm_algo_t algo, int cus) {
    const Launch l = launch_for(p, nullptr);
    const bool dma = bf16_dma_applies(p, l, 256, 256);
    const StripPricer bf16_strips{kBf16DmaOpts, 2, kBf16MfmaOpts, 3, cus};
    Plan best;
    auto consider = [&](const Plan& pl) { if (pl.cost < best.cost) best = pl; };
    const bool any = algo == GEMM_ALGO_AUTO || algo == GEMM_ALGO_MFMA;
    if (dma)
        for (const TileOpt& o : kBf16DmaOpts) {
            const bool want = any || algo == GEMM_ALGO_MFMA_DMA || (algo == GEMM_ALGO_MFMA_256x256 && o.bn == 256) ||
                              (algo == GEMM_ALGO_MFMA_256x128 && o.bn == 128);
            if (want) consider(plan_core(p, o, true, true, cus, bf16_strips));
        }
    for (const TileOpt& o : kBf16MfmaOpts) {
        // with the direct-copy kernel available, the default choice leaves the 256-row tiles to it
        const bool want = (any && !(dma && o.bm == 256)) || (algo == GEMM_ALGO_MFMA_256x128 && o.bm == 256 && !dma) ||
                          (algo == GEMM_ALGO_MFMA_128x128 && o.bm == 128) || (algo == GEMM_ALGO_MFMA_64x64 && o.bm == 64);
        if (want) consider(plan_whole(p, o, cus));
    }
    return best;
}

// Split-K on the 16-bit direct-copy kernel's 256 x 256 tiles, for problems whose tiles leave
// CUs idle: S slices of K per tile as a second grid dimension (one round: tiles x S <= CUs),
// each slice at least kMinSliceK deep; the slabs of slices 1 .. S-1 need (S-1) M N floats of
// workspace and a second pass adds them to C.  S and the choice against the unsplit kernels come
// from a time model fitted to measurements (rocprofv3 and HIP events, interleaved with the FP32
// 4096^3 GEMM as the benchmark runs): per 64-deep k-tile and round, 1.5 us at 256 x 256 and
// 1.0 us at 256 x 128 (0.65 of the 256 x 256 figure, as measured standalone: FFN-down 2048 x 4096
// x 11008 against 4096^3) with every CU busy, times 0.75 + 0.25 u when only a fraction u of the
// CUs holds a tile (the clock the power limit allows rises); 2 us per launch; C (or the slabs)
// written at 5 TB/s; the slab pass 3 us plus (S+1) M N floats at 6 TB/s.  Measured against that:
// 4096 x 512 x 4096, 4 slices 40.1 us (8: 45.7, unsplit 55.3); 2048 x 2048 x 8192, 4 slices
// 78.4 us (unsplit 105.6); 1024 x 1024 x 8192, 8 slices 40.6 us (unsplit 88.8); no split where the
// tiles fill the chip or K is short (2048 x 4096 x 4096: 2 slices 79.8 us, unsplit 67.0); FFN-down
// 2048 x 4096 x 11008, 2 slices 176-180 us (unsplit 256 x 128: 185-190).
constexpr int kMinSliceK = 512;
constexpr double kTau256 = 1.5e-6, kTau128 = 1.0e-6, kLaunchSec = 2e-6, kWriteBps = 5e12, kSumSec = 3e-6,
                 kSumBps = 6e12;

double occupancy_factor(int64_t units, int cus) {
    const double u = std::min(1.0, (double)units / (cus > 0 ? cus : 256));
    return 0.75 + 0.25 * u;
}

// Seconds of the unsplit direct-copy kernel on tiles bm x bn.
double dma_plain_seconds(const Problem& p, int bn, int cus) {
    const int64_t c = cus > 0 ? cus : 256, n = tiles(p.M, p.N, 256, bn);
    const int64_t rounds = (n + c - 1) / c, last = n - (rounds - 1) * c;
    const double step = (p.K / 64.0) * (bn == 256 ? kTau256 : kTau128);
    return (rounds - 1) * (kLaunchSec + step) + kLaunchSec + step * occupancy_factor(last, cus) +
           4.0 * p.M * p.N / kWriteBps;
}

double split_seconds(const Problem& p, const TileSplit& t, int cus) {
    const int64_t units = tiles(p.M, p.N, 256, 256) * t.slices;
    return kLaunchSec + (t.kslice / 64.0) * kTau256 * occupancy_factor(units, cus) + units * 65536.0 * 4 / kWriteBps +
           kSumSec + (t.slices + 1) * 4.0 * p.M * p.N / kSumBps;
}

// The best split by the model (slices == 1: none better than the unsplit direct-copy kernel by 5%).
TileSplit tile_split(const Problem& p, int cus) {
    TileSplit best;
    if (!bf16_dma_applies(p, Launch{}, 256, 256)) return best;
    const int64_t c = cus > 0 ? cus : 256, n = tiles(p.M, p.N, 256, 256);
    const int64_t most = std::min<int64_t>(c / std::max<int64_t>(n, 1), p.K / kMinSliceK);
    double best_t = 0.95 * std::min(dma_plain_seconds(p, 256, cus), dma_plain_seconds(p, 128, cus));
    for (int s = 2; s <= most; ++s) {
        TileSplit t;
        t.kslice = (int)(((p.K + s - 1) / s + 63) / 64 * 64);
        t.slices = (p.K + t.kslice - 1) / t.kslice;
        if (t.slices != s || p.K - (int64_t)(s - 1) * t.kslice < 64) continue;
        t.bytes = (size_t)(s - 1) * p.M * p.N * sizeof(float);
        const double sec = split_seconds(p, t, cus);
        if (sec < best_t) {
            best_t = sec;
            best = t;
        }
    }
    return best;
}

// FP32: whole 256 x 256 tiles of the direct-copy kernel split into at most one round's worth of
// slices, each at least kMinSliceK deep, when the same time model with the FP32 kernel's own
// figure (7.7 us per 32-deep k-tile and round with every CU busy, from 4096^3) prices the split
// below the default plan.  The default plan's kernels (register-staged 64^2 and 128^2 tiles,
// the 128^2 direct-copy tile) are priced by their round cost: a 256^2 tile's round of
// 65536 units costs K / 32 k-tiles of that figure (no margin: this pricing is optimistic for the
// register-staged tiles, 164 against 194-209 us measured on the shard).  Measured (events,
// interleaved runs):
// 4096 x 512 x 4096 209 / 194 -> 160 / 150 us, 4096 x 512 x 8192 362 -> 264 us, 2048^2 x 4096
// 280 -> 264 us; 4096 x 768 x 2048 is left unsplit (126 against 137 us split).
constexpr double kTauF32 = 7.7e-6;

double f32_split_seconds(const Problem& p, const TileSplit& t, int cus) {
    const int64_t units = tiles(p.M, p.N, 256, 256) * t.slices;
    return kLaunchSec + (t.kslice / 32.0) * kTauF32 * occupancy_factor(units, cus) +
           (t.slices - 1) * 4.0 * p.M * p.N / kWriteBps + kSumSec + (t.slices + 1) * 4.0 * p.M * p.N / kSumBps;
}

TileSplit f32_tile_split(const Problem& p, int cus) {
    TileSplit best;
    const int64_t c = cus > 0 ? cus : 256;
    if (p.M % 256 != 0 || p.N % 256 != 0 || !f32_dma_applies(p, launch_for(p, nullptr), 256, 256)) return best;
    const int64_t n = tiles(p.M, p.N, 256, 256);
    const int64_t most = std::min<int64_t>(c / std::max<int64_t>(n, 1), p.K / kMinSliceK);
    const Plan plain = choose_f32_tiles(p, GEMM_ALGO_AUTO, cus);
    double best_t = plain.cost / 65536.0 * (p.K / 32.0) * kTauF32;
    for (int s = 2; s <= most; ++s) {
        TileSplit t;
        t.kslice = (int)(((p.K + s - 1) / s + 63) / 64 * 64);
        t.slices = (p.K + t.kslice - 1) / t.kslice;
        if (t.slices != s) continue;
        t.bytes = (size_t)(s - 1) * p.M * p.N * sizeof(float);
        const double sec = f32_split_seconds(p, t, cus);
        if (sec < best_t) {
            best_t = sec;
            best = t;
        }
    }
    return best;
}

// The split the default choice takes with this workspace (slices == 1: none).
TileSplit tile_split_with(const Problem& p, int cus, const Workspace& ws, bool f32) {
    if (ws.ptr == nullptr || !aligned(ws.ptr, 16)) return TileSplit{};
    const TileSplit t = f32 ? f32_tile_split(p, cus) : tile_split(p, cus);
    return t.slices > 1 && t.bytes <= ws.bytes ? t : TileSplit{};
}

hipError_t run_b16_tiles(const Problem& p, hipStream_t stream, gemm_algo_t algo, int et, const DeviceInfo& dev,
                         const char*& name, gemm_status_t& st, const Batch& b, const Workspace& ws = Workspace{}) {
    const Plan best = choose_bf16_tiles(p, algo, dev.cus);
    if (best.cost >= 1e300) { st = GEMM_ERR_INVALID_VALUE; return hipSuccess; }
    if (algo == GEMM_ALGO_AUTO && b.n == 1) {
        const TileSplit t = tile_split_with(p, dev.cus, ws, false);
        if (t.slices > 1) {
            SplitProblem sp{};
            static_cast<Problem&>(sp) = p;
            sp.kslice = t.kslice;
            sp.part = static_cast<float*>(ws.ptr);
            Launch l = launch_for(p, stream);
            l.vec_c = l.vec_c && p.N % 4 == 0;
            l.group_m = pick_group_m((p.M + 255) / 256, (p.N + 255) / 256);
            name = et == kElemF16 ? "f16_dma256x256_splitk" : "bf16_dma256x256_splitk";
            return launch_bf16_dma_split(sp, t.slices, l, 256, 256, et == kElemF16);
        }
    }
    name = b16_name(best.opt, et);
    const TileOpt o = best.opt;
    const bool f16 = et == kElemF16;
    return run_plan(p, stream, best, et, dev, b, [&](const Problem& c, const Launch& lc) {
        return o.dma ? launch_bf16_dma(c, lc, o.bm, o.bn, f16) : launch_bf16_mfma(c, lc, o.bm, o.bn, f16);
    });
}

// Kernel choice and launch for a normalised problem (row-major C, K > 0).  A status other
// than GEMM_OK in `st` means the request is invalid (nothing launched).
hipError_t dispatch(const Problem& p, hipStream_t stream, gemm_algo_t algo, int et, const DeviceInfo& dev,
                    const char*& name, gemm_status_t& st, const Workspace& ws, const Batch& b) {
    Launch l = launch_for(p, stream, b);
    if (et == kElemF32) {
        switch (algo) {
            case GEMM_ALGO_NAIVE_UNCOALESCED: name = "f32_naive_uncoalesced"; return launch_naive(p, l, false);
            case GEMM_ALGO_NAIVE: name = "f32_naive"; return launch_naive(p, l, true);
            case GEMM_ALGO_TILED: name = "f32_tiled32"; return launch_tiled(p, l);
            case GEMM_ALGO_REGBLOCK:
                l.group_m = pick_group_m((p.M + kRegblockBM - 1) / kRegblockBM, (p.N + kRegblockBN - 1) / kRegblockBN);
                name = "f32_regblock128x128";
                return launch_regblock(p, l);
            case GEMM_ALGO_SKINNY:
                if (!skinny_applies(p, false)) { st = GEMM_ERR_INVALID_VALUE; return hipSuccess; }
                return run_skinny(p, l, kElemF32, dev.cus, name);
            default:
                if (algo == GEMM_ALGO_AUTO && prefer_small(p, dev.cus) && skinny_applies(p, false))
                    return run_skinny(p, l, kElemF32, dev.cus, name, ws, true);
                return run_f32_tiles(p, stream, algo, dev, name, st, b, ws);
        }
    }
    const bool small = algo == GEMM_ALGO_AUTO && prefer_small(p, dev.cus) && skinny_applies(p, true);
    if (small && b.n == 1 && small_tiles16(p, dev.cus))
        return run_b16_tiles(p, stream, GEMM_ALGO_MFMA_64x64, et, dev, name, st, b);
    if (algo == GEMM_ALGO_SKINNY || small) {
        if (!skinny_applies(p, true)) { st = GEMM_ERR_INVALID_VALUE; return hipSuccess; }
        return run_skinny(p, l, et, dev.cus, name, algo == GEMM_ALGO_AUTO ? ws : Workspace{}, algo == GEMM_ALGO_AUTO);
    }
    return run_b16_tiles(p, stream, algo, et, dev, name, st, b, ws);
}

// The problem the library computes for extents and orders with tight leading dimensions and
// no memory (a column-major C becomes C^T = B^T A^T), for queries that launch nothing.
Problem query_problem(int64_t M, int64_t N, int64_t K, int oa, int ob, int oc) {
    const int64_t lda = oa == GEMM_ROW_MAJOR ? std::max<int64_t>(K, 1) : M;
    const int64_t ldb = ob == GEMM_ROW_MAJOR ? N : std::max<int64_t>(K, 1);
    if (oc == GEMM_ROW_MAJOR) return Problem{(int)M, (int)N, (int)K, nullptr, lda, oa, nullptr, ldb, ob, nullptr, N};
    return Problem{(int)N, (int)M, (int)K, nullptr, ldb, 1 - ob, nullptr, lda, 1 - oa, nullptr, M};
}

// Workspace bytes with which the _ws entry points split K (0: they never do for this problem).
size_t split_bytes(const Problem& p, int et, int cus) {
    if (p.M == 0 || p.N == 0 || p.K == 0 || et == kElemFp8) return 0;
    if (prefer_small(p, cus) && skinny_applies(p, et != kElemF32)) {
        if (et != kElemF32 && small_tiles16(p, cus)) return 0;
        const SkinnySplit sp = skinny_split(p, et != kElemF32, cus);
        return sp.slices > 1 ? sp.bytes : 0;
    }
    const TileSplit t = et == kElemF32 ? f32_tile_split(p, cus) : tile_split(p, cus);
    return t.slices > 1 ? t.bytes : 0;
}

// What the default choice runs for a normalised problem with K > 0, without launching: the
// kernel's name and the rows and columns of C its own launch covers (the rest are strips).
// The tile of the 8-bit kernel: the cheaper of its two configurations over the whole of C
// (256 x 128, whose build has a byte-wise K tail, for K < 16).
Plan plan_fp8(const Problem& p, int cus) {
    if (p.K < 16) return plan_whole(p, kBf16DmaOpts[1], cus);
    Plan best;
    for (const TileOpt& o : kBf16DmaOpts) {
        const Plan pl = plan_whole(p, o, cus);
        if (pl.cost < best.cost) best = pl;
    }
    return best;
}

const char* fp8_name(const TileOpt& o) { return o.bn == 256 ? "fp8_dma256x256" : "fp8_dma256x128"; }

const char* plan_auto(const Problem& p, int et, int cus, int& mc, int& nc) {
    const bool f32 = et == kElemF32;
    mc = p.M;
    nc = p.N;
    if (et == kElemFp8) return fp8_name(plan_fp8(p, cus).opt);
    const bool small = prefer_small(p, cus) && skinny_applies(p, !f32);
    if (small && f32 && skinny_halves_applies(p, cus)) return kSkinnyHalvesName;
    if (small && skinny_pairs_applies(p, et, cus) && (f32 || !small_tiles16(p, cus))) return kSkinnyPairsNames[et];
    if (small && (f32 || !small_tiles16(p, cus))) return skinny_name(et, skinny_blocks(p, cus));
    const Plan pl = f32 ? choose_f32_tiles(p, GEMM_ALGO_AUTO, cus)
                        : choose_bf16_tiles(p, small ? GEMM_ALGO_MFMA_64x64 : GEMM_ALGO_AUTO, cus);
    mc = pl.mc;
    nc = pl.nc;
    return f32 ? f32_name(pl.opt) : b16_name(pl.opt, et);
}

template <typename Elem>
gemm_status_t run(In in, gemm_algo_t algo, int64_t M, int64_t N, int64_t K, const Elem* A,
                  int64_t lda, gemm_order_t oa, const Elem* B, int64_t ldb, gemm_order_t ob,
                  float* C, int64_t ldc, gemm_order_t oc, hipStream_t stream,
                  const Workspace& ws = Workspace{}) {
    gemm_status_t st = validate(in, M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc);
    if (st != GEMM_OK) return st;
    if (ws.ptr != nullptr && !aligned(ws.ptr, 16)) return GEMM_ERR_INVALID_VALUE;
    const bool f32 = in == In::F32;
    switch (algo) {
        case GEMM_ALGO_AUTO: case GEMM_ALGO_MFMA: break;
        case GEMM_ALGO_NAIVE_UNCOALESCED: case GEMM_ALGO_NAIVE: case GEMM_ALGO_TILED:
        case GEMM_ALGO_REGBLOCK:
            if (!f32) return GEMM_ERR_INVALID_VALUE;
            break;
        case GEMM_ALGO_MFMA_128x128: case GEMM_ALGO_MFMA_64x64: case GEMM_ALGO_SKINNY: break;
        case GEMM_ALGO_MFMA_DMA: break;
        case GEMM_ALGO_MFMA_256x256: break;
        case GEMM_ALGO_MFMA_256x128:
            if (f32) return GEMM_ERR_INVALID_VALUE;
            break;
        default: return GEMM_ERR_INVALID_VALUE;
    }
    if (M == 0 || N == 0) {
        t_last_kernel = "none";
        return GEMM_OK;
    }
    DeviceInfo dev;
    if (!device_info(dev) || !dev.supported) return GEMM_ERR_UNSUPPORTED_DEVICE;

    // Column-major C: compute C^T = B^T A^T into the same memory viewed row-major.
    Problem p{};
    if (oc == GEMM_ROW_MAJOR) {
        p = Problem{(int)M, (int)N, (int)K, A, lda, (int)oa, B, ldb, (int)ob, C, ldc};
    } else {
        p = Problem{(int)N, (int)M, (int)K, B, ldb, 1 - (int)ob, A, lda, 1 - (int)oa, C, ldc};
    }
    hipError_t err = hipSuccess;
    const char* name = "none";
    if (K == 0) {
        err = launch_zero_c(p, launch_for(p, stream));
        name = "zero_c";
    } else {
        gemm_status_t bad = GEMM_OK;
        err = dispatch(p, stream, algo, elem_of(in), dev, name, bad, ws);
        if (bad != GEMM_OK) return bad;
    }
    if (err != hipSuccess) {
        t_last_hip_error = (int)err;
        return GEMM_ERR_LAUNCH;
    }
    t_last_kernel = name;
    return GEMM_OK;
}

// Entries of a strided batch that one launch covers (the grid's z extent).
constexpr int64_t kMaxBatchLaunch = 65535;

// Whether the entries of a batched C (normalised: row-major M x N, leading dimension ldc,
// entry stride sc) are disjoint: stacked (each entry starts past the previous one's last
// element) or side by side within each row (sc >= N and all n entries inside ldc).
bool c_entries_disjoint(int64_t M, int64_t N, int64_t ldc, int64_t sc, int64_t n) {
    if (n <= 1) return true;
    if ((__int128)sc >= (__int128)(M - 1) * ldc + N) return true;
    return sc >= N && (n - 1) <= (ldc - N) / sc;
}

template <typename Elem>
gemm_status_t run_batched(In in, int64_t batch, int64_t M, int64_t N, int64_t K, const Elem* A, int64_t lda,
                          int64_t sa, gemm_order_t oa, const Elem* B, int64_t ldb, int64_t sb, gemm_order_t ob,
                          float* C, int64_t ldc, int64_t sc, gemm_order_t oc, hipStream_t stream) {
    gemm_status_t st = validate(in, M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc);
    if (st != GEMM_OK) return st;
    if (batch < 0 || sa < 0 || sb < 0 || sc < 0) return GEMM_ERR_INVALID_VALUE;
    const int64_t span = batch > 1 ? batch - 1 : 0;       // entry offsets, in bytes, fit in int64
    for (int64_t s : {sa, sb, sc})
        if (span > 0 && s > INT64_MAX / 4 / span) return GEMM_ERR_INVALID_VALUE;
    const bool row = oc == GEMM_ROW_MAJOR;
    if (M > 0 && N > 0 && !c_entries_disjoint(row ? M : N, row ? N : M, ldc, sc, batch))
        return GEMM_ERR_INVALID_VALUE;
    if (batch == 0 || M == 0 || N == 0) {
        t_last_kernel = "none";
        return GEMM_OK;
    }
    DeviceInfo dev;
    if (!device_info(dev) || !dev.supported) return GEMM_ERR_UNSUPPORTED_DEVICE;

    // Column-major C: every entry computes C^T = B^T A^T, so A and B swap strides too.
    Problem p{};
    Batch b{};
    if (row) {
        p = Problem{(int)M, (int)N, (int)K, A, lda, (int)oa, B, ldb, (int)ob, C, ldc};
        b = Batch{batch, sa, sb, sc};
    } else {
        p = Problem{(int)N, (int)M, (int)K, B, ldb, 1 - (int)ob, A, lda, 1 - (int)oa, C, ldc};
        b = Batch{batch, sb, sa, sc};
    }
    const int e = in == In::F32 ? 4 : 2;
    const char* name = "none";
    for (int64_t z0 = 0; z0 < batch; z0 += kMaxBatchLaunch) {
        Batch bz = b;
        bz.n = std::min(kMaxBatchLaunch, batch - z0);
        Problem pz = p;
        pz.A = static_cast<const char*>(p.A) + z0 * b.sa * e;
        pz.B = static_cast<const char*>(p.B) + z0 * b.sb * e;
        pz.C = p.C + z0 * b.sc;
        hipError_t err = hipSuccess;
        if (K == 0) {
            err = launch_zero_c(pz, launch_for(pz, stream, bz));
            name = "zero_c";
        } else {
            // the planner prices tiles against the CUs one entry gets
            DeviceInfo de = dev;
            de.cus = (int)std::max<int64_t>(1, dev.cus / bz.n);
            gemm_status_t bad = GEMM_OK;
            err = dispatch(pz, stream, GEMM_ALGO_AUTO, elem_of(in), de, name, bad, Workspace{}, bz);
            if (bad != GEMM_OK) return bad;
        }
        if (err != hipSuccess) {
            t_last_hip_error = (int)err;
            return GEMM_ERR_LAUNCH;
        }
    }
    t_last_kernel = name;
    return GEMM_OK;
}

// GEMM with the fused epilogue: 16-bit inputs on the direct-copy kernel, the whole of C in one
// launch (tiles overhang both edges), or the epilogue of an empty sum for K == 0.
gemm_status_t run_fused(In in, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, gemm_order_t oa,
                        const void* B, int64_t ldb, gemm_order_t ob, void* C, int64_t ldc, gemm_order_t oc,
                        const gemm_epilogue_t* epi, hipStream_t stream) {
    if (epi == nullptr) return GEMM_ERR_INVALID_VALUE;
    if (epi->activation != GEMM_ACT_NONE && epi->activation != GEMM_ACT_RELU && epi->activation != GEMM_ACT_GELU)
        return GEMM_ERR_INVALID_VALUE;
    if (epi->out_type != GEMM_OUT_F32 && epi->out_type != GEMM_OUT_BF16) return GEMM_ERR_INVALID_VALUE;
    const bool out16 = epi->out_type == GEMM_OUT_BF16;
    gemm_status_t st = validate(in, M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc, out16 ? 2 : 4);
    if (st != GEMM_OK) return st;
    if (epi->bias != nullptr && !aligned(epi->bias, 4)) return GEMM_ERR_INVALID_VALUE;
    const bool row = oc == GEMM_ROW_MAJOR;
    Problem p{};
    if (row) p = Problem{(int)M, (int)N, (int)K, A, lda, (int)oa, B, ldb, (int)ob, static_cast<float*>(C), ldc};
    else p = Problem{(int)N, (int)M, (int)K, B, ldb, 1 - (int)ob, A, lda, 1 - (int)oa, static_cast<float*>(C), ldc};
    // the direct-copy kernels' layout: k-contiguous operands (after a column-major C's swap); for
    // FP32 inputs K >= 32 and 32-row copy blocks within 32-bit offsets
    const bool f32 = in == In::F32;
    const int64_t lim = (int64_t)1 << 31;
    if (K > 0 && !f32 && !bf16_dma_applies(p, Launch{}, 256, 256)) return GEMM_ERR_INVALID_VALUE;
    if (K > 0 && f32 && (p.oa != kRow || p.ob != kCol || K < 32 || 32 * p.lda * 4 >= lim || 32 * p.ldb * 4 >= lim))
        return GEMM_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) {
        t_last_kernel = "none";
        return GEMM_OK;
    }
    DeviceInfo dev;
    if (!device_info(dev) || !dev.supported) return GEMM_ERR_UNSUPPORTED_DEVICE;

    // a column-major C's bias runs along its columns, the rows of the normalised C
    const Epilogue e{epi->alpha, epi->beta, epi->bias, row ? 0 : 1, (int)epi->activation, out16 ? 1 : 0};
    // nothing to apply: the plain kernel on the same plan (FP32 inputs: the plain call)
    const bool identity = e.alpha == 1.f && e.beta == 0.f && e.bias == nullptr && e.act == kActNone && !out16;
    if (identity && f32 && K > 0)
        return run(In::F32, GEMM_ALGO_AUTO, M, N, K, static_cast<const float*>(A), lda, oa, static_cast<const float*>(B),
                   ldb, ob, static_cast<float*>(C), ldc, oc, stream);
    hipError_t err = hipSuccess;
    const char* name = "epilogue_fill";
    if (K == 0) {
        EpiProblem ep{};
        static_cast<Problem&>(ep) = p;
        ep.e = e;
        Launch l = launch_for(p, stream);
        l.vec_c = (p.ldc % 4 == 0) && aligned(C, out16 ? 8 : 16);
        err = launch_epi_fill(ep, l);
    } else {
        // a core on one direct-copy tile and the strips that complete it, every part on the
        // direct-copy kernels (the only ones that carry the epilogue), each strip on its own
        // cheapest tile: 2048 x 11008 is 8 x 32 tiles of 256 x 256 (one round) and a 2048 x 2816
        // strip of 256 x 128 tiles (one round), against 2.7 rounds of 256 x 128 tiles
        const TileOpt* opts = f32 ? kF32DmaOpts : kBf16DmaOpts;
        const StripPricer dma_strips{opts, 2, opts, 0, dev.cus};
        Plan best;
        for (int i = 0; i < 2; ++i) {
            const Plan pl = plan_core(p, opts[i], true, true, dev.cus, dma_strips);
            if (pl.cost < best.cost) best = pl;
        }
        const int eb = out16 ? 2 : 4;
        auto part = [&](int r0, int m, int c0, int n, const TileOpt* force) {
            EpiProblem ep{};
            static_cast<Problem&>(ep) = sub_problem(p, r0, m, c0, n, f32 ? 4 : 2);
            ep.C = reinterpret_cast<float*>(static_cast<char*>(C) + ((int64_t)r0 * p.ldc + c0) * eb);
            ep.e = e;
            if (e.bias != nullptr) ep.e.bias = e.bias + (e.bias_rows ? r0 : c0);
            TileOpt o = force != nullptr ? *force : opts[0];
            if (force == nullptr) {
                double c = 1e300;
                for (int i = 0; i < 2; ++i) {
                    const double pc = plan_whole(ep, opts[i], dev.cus).cost;
                    if (pc < c) { c = pc; o = opts[i]; }
                }
            }
            Launch l = launch_for(ep, stream);
            l.vec_c = (p.ldc % 4 == 0) && aligned(ep.C, out16 ? 8 : 16);
            l.group_m = pick_group_m((m + o.bm - 1) / o.bm, (n + o.bn - 1) / o.bn);
            if (f32) return launch_f32_dma_epi(ep, l, o.bm, o.bn);
            return identity ? launch_bf16_dma(ep, l, o.bm, o.bn, in == In::F16)
                            : launch_bf16_dma_epi(ep, l, o.bm, o.bn, in == In::F16);
        };
        err = part(0, best.mc, 0, best.nc, &best.opt);
        if (err == hipSuccess && best.mc < p.M) err = part(best.mc, p.M - best.mc, 0, p.N, nullptr);
        if (err == hipSuccess && best.nc < p.N) err = part(0, best.mc, best.nc, p.N - best.nc, nullptr);
        static const char* names[2][2][2] = {{{"bf16_dma256x256_fused", "bf16_dma256x128_fused"},
                                              {"f16_dma256x256_fused", "f16_dma256x128_fused"}},
                                             {{"bf16_dma256x256", "bf16_dma256x128"},
                                              {"f16_dma256x256", "f16_dma256x128"}}};
        name = f32 ? (best.opt.bn == 256 ? "f32_dma256x256_fused" : "f32_dma128x128_fused")
                   : names[identity ? 1 : 0][in == In::F16 ? 1 : 0][best.opt.bn == 256 ? 0 : 1];
    }
    if (err != hipSuccess) {
        t_last_hip_error = (int)err;
        return GEMM_ERR_LAUNCH;
    }
    t_last_kernel = name;
    return GEMM_OK;
}

// GEMM on 8-bit floating-point inputs: the direct-copy kernel with the 8-bit matrix
// instruction over the whole of C (tiles overhang both edges), zero_c for K == 0.
gemm_status_t run_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, gemm_order_t oa, int fa,
                      const uint8_t* B, int64_t ldb, gemm_order_t ob, int fb, float* C, int64_t ldc, gemm_order_t oc,
                      hipStream_t stream) {
    for (int f : {fa, fb})
        if (f != GEMM_FP8_E4M3 && f != GEMM_FP8_E5M2) return GEMM_ERR_INVALID_VALUE;
    const gemm_status_t st = validate(In::FP8, M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc);
    if (st != GEMM_OK) return st;
    // both operands contiguous along k (the column-major-C swap keeps that)
    if (oa != GEMM_ROW_MAJOR || ob != GEMM_COL_MAJOR) return GEMM_ERR_INVALID_VALUE;
    const bool row = oc == GEMM_ROW_MAJOR;
    Problem p{};
    int f0 = fa, f1 = fb;
    if (row) {
        p = Problem{(int)M, (int)N, (int)K, A, lda, (int)oa, B, ldb, (int)ob, C, ldc};
    } else {
        p = Problem{(int)N, (int)M, (int)K, B, ldb, 1 - (int)ob, A, lda, 1 - (int)oa, C, ldc};
        std::swap(f0, f1);
    }
    if (K > 0 && !fp8_dma_applies(p)) return GEMM_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) {
        t_last_kernel = "none";
        return GEMM_OK;
    }
    DeviceInfo dev;
    if (!device_info(dev) || !dev.supported) return GEMM_ERR_UNSUPPORTED_DEVICE;
    Launch l = launch_for(p, stream);
    hipError_t err = hipSuccess;
    const char* name = "zero_c";
    if (K == 0) {
        err = launch_zero_c(p, l);
    } else {
        const Plan best = plan_fp8(p, dev.cus);
        const int bm = best.opt.bm, bn = best.opt.bn;
        l.group_m = pick_group_m((p.M + bm - 1) / bm, (p.N + bn - 1) / bn);
        name = fp8_name(best.opt);
        err = launch_fp8_dma(p, l, bm, bn, f0, f1);
    }
    if (err != hipSuccess) {
        t_last_hip_error = (int)err;
        return GEMM_ERR_LAUNCH;
    }
    t_last_kernel = name;
    return GEMM_OK;
}

// gemm_bf16_f32acc_noalloc: the _ws call with `scratch` as its workspace.  Nothing is
// allocated; a problem whose split would need more than kScratchBytes is refused.
gemm_status_t run_noalloc(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, gemm_order_t oa,
                          const uint16_t* B, int64_t ldb, gemm_order_t ob, float* C, int64_t ldc, gemm_order_t oc,
                          hipStream_t stream) {
    const gemm_status_t st = validate(In::BF16, M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc);
    if (st != GEMM_OK) return st;
    if (M == 0 || N == 0) return run(In::BF16, GEMM_ALGO_AUTO, M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc, stream);
    DeviceInfo dev;
    if (!device_info(dev) || !dev.supported) return GEMM_ERR_UNSUPPORTED_DEVICE;
    void* ptr = nullptr;
    const hipError_t e = scratch_address(ptr);
    if (e != hipSuccess) {
        t_last_hip_error = (int)e;
        return GEMM_ERR_LAUNCH;
    }
    const size_t need = K > 0 ? split_bytes(query_problem(M, N, K, oa, ob, oc), kElemBf16, dev.cus) : 0;
    if (need > kScratchBytes) return GEMM_ERR_SCRATCH_TOO_SMALL;
    // the planner uses the workspace only for a split that fits in the bytes it is given
    return run(In::BF16, GEMM_ALGO_AUTO, M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc, stream,
               Workspace{ptr, kScratchBytes});
}

}  // namespace
}  // namespace gemm

extern "C" {

gemm_status_t gemm_bf16_f32acc_noalloc(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                       gemm_order_t order_a, const uint16_t* B, int64_t ldb, gemm_order_t order_b,
                                       float* C, int64_t ldc, gemm_order_t order_c, hipStream_t stream) {
    return gemm::run_noalloc(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, stream);
}

gemm_status_t gemm_bf16_f32acc_fused(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                     gemm_order_t order_a, const uint16_t* B, int64_t ldb, gemm_order_t order_b,
                                     void* C, int64_t ldc, gemm_order_t order_c, const gemm_epilogue_t* epilogue,
                                     hipStream_t stream) {
    return gemm::run_fused(gemm::In::BF16, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, epilogue,
                           stream);
}

gemm_status_t gemm_f16_f32acc_fused(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                    gemm_order_t order_a, const uint16_t* B, int64_t ldb, gemm_order_t order_b,
                                    void* C, int64_t ldc, gemm_order_t order_c, const gemm_epilogue_t* epilogue,
                                    hipStream_t stream) {
    return gemm::run_fused(gemm::In::F16, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, epilogue,
                           stream);
}

gemm_status_t gemm_fp8_f32acc(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, gemm_order_t order_a,
                              gemm_fp8_t format_a, const uint8_t* B, int64_t ldb, gemm_order_t order_b,
                              gemm_fp8_t format_b, float* C, int64_t ldc, gemm_order_t order_c, hipStream_t stream) {
    return gemm::run_fp8(M, N, K, A, lda, order_a, (int)format_a, B, ldb, order_b, (int)format_b, C, ldc, order_c,
                         stream);
}

gemm_status_t gemm_f32_fused(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, gemm_order_t order_a,
                             const float* B, int64_t ldb, gemm_order_t order_b, void* C, int64_t ldc,
                             gemm_order_t order_c, const gemm_epilogue_t* epilogue, hipStream_t stream) {
    return gemm::run_fused(gemm::In::F32, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, epilogue,
                           stream);
}

gemm_status_t gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                       gemm_order_t order_a, const float* B, int64_t ldb, gemm_order_t order_b,
                       float* C, int64_t ldc, gemm_order_t order_c, hipStream_t stream) {
    return gemm::run(gemm::In::F32, GEMM_ALGO_AUTO, M, N, K, A, lda, order_a, B, ldb, order_b,
                     C, ldc, order_c, stream);
}

gemm_status_t gemm_bf16_f32acc(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                               gemm_order_t order_a, const uint16_t* B, int64_t ldb,
                               gemm_order_t order_b, float* C, int64_t ldc, gemm_order_t order_c,
                               hipStream_t stream) {
    return gemm::run(gemm::In::BF16, GEMM_ALGO_AUTO, M, N, K, A, lda, order_a, B, ldb, order_b,
                     C, ldc, order_c, stream);
}

gemm_status_t gemm_f32_algo(gemm_algo_t algo, int64_t M, int64_t N, int64_t K, const float* A,
                            int64_t lda, gemm_order_t order_a, const float* B, int64_t ldb,
                            gemm_order_t order_b, float* C, int64_t ldc, gemm_order_t order_c,
                            hipStream_t stream) {
    return gemm::run(gemm::In::F32, algo, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc,
                     order_c, stream);
}

gemm_status_t gemm_bf16_f32acc_algo(gemm_algo_t algo, int64_t M, int64_t N, int64_t K,
                                    const uint16_t* A, int64_t lda, gemm_order_t order_a,
                                    const uint16_t* B, int64_t ldb, gemm_order_t order_b,
                                    float* C, int64_t ldc, gemm_order_t order_c,
                                    hipStream_t stream) {
    return gemm::run(gemm::In::BF16, algo, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc,
                     order_c, stream);
}

gemm_status_t gemm_plan(int dtype, int64_t M, int64_t N, int64_t K, gemm_order_t order_a,
                        gemm_order_t order_b, gemm_order_t order_c, int cus, const char** kernel,
                        int64_t* core_rows, int64_t* core_cols, size_t* workspace_bytes) {
    if (kernel == nullptr || core_rows == nullptr || core_cols == nullptr || workspace_bytes == nullptr ||
        cus <= 0 || dtype < 0 || dtype > 3)
        return GEMM_ERR_INVALID_VALUE;
    if (M < 0 || N < 0 || K < 0 || M > INT_MAX || N > INT_MAX || K > INT_MAX) return GEMM_ERR_INVALID_VALUE;
    for (int o : {(int)order_a, (int)order_b, (int)order_c})
        if (o != GEMM_ROW_MAJOR && o != GEMM_COL_MAJOR) return GEMM_ERR_INVALID_VALUE;
    if (dtype == gemm::kElemFp8 && (order_a != GEMM_ROW_MAJOR || order_b != GEMM_COL_MAJOR))
        return GEMM_ERR_INVALID_VALUE;
    *kernel = "none";
    *core_rows = *core_cols = 0;
    *workspace_bytes = 0;
    if (M == 0 || N == 0) return GEMM_OK;
    const gemm::Problem p = gemm::query_problem(M, N, K, order_a, order_b, order_c);
    if (K == 0) {
        *kernel = "zero_c";
        *core_rows = p.M;
        *core_cols = p.N;
        return GEMM_OK;
    }
    int mc = 0, nc = 0;
    *kernel = gemm::plan_auto(p, dtype, cus, mc, nc);
    *core_rows = mc;
    *core_cols = nc;
    *workspace_bytes = gemm::split_bytes(p, dtype, cus);
    return GEMM_OK;
}

size_t gemm_workspace_size(int dtype, int64_t M, int64_t N, int64_t K, gemm_order_t order_a,
                           gemm_order_t order_b, gemm_order_t order_c) {
    if (M <= 0 || N <= 0 || K <= 0 || M > INT_MAX || N > INT_MAX || K > INT_MAX || dtype < 0 || dtype > 3) return 0;
    for (int o : {(int)order_a, (int)order_b, (int)order_c})
        if (o != GEMM_ROW_MAJOR && o != GEMM_COL_MAJOR) return 0;
    gemm::DeviceInfo dev;
    if (!gemm::device_info(dev) || !dev.supported) return 0;
    return gemm::split_bytes(gemm::query_problem(M, N, K, order_a, order_b, order_c), dtype, dev.cus);
}

gemm_status_t gemm_f32_ws(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                          gemm_order_t order_a, const float* B, int64_t ldb, gemm_order_t order_b,
                          float* C, int64_t ldc, gemm_order_t order_c, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    return gemm::run(gemm::In::F32, GEMM_ALGO_AUTO, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc,
                     order_c, stream, gemm::Workspace{workspace, workspace_bytes});
}

gemm_status_t gemm_bf16_f32acc_ws(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                  gemm_order_t order_a, const uint16_t* B, int64_t ldb,
                                  gemm_order_t order_b, float* C, int64_t ldc, gemm_order_t order_c,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return gemm::run(gemm::In::BF16, GEMM_ALGO_AUTO, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc,
                     order_c, stream, gemm::Workspace{workspace, workspace_bytes});
}

gemm_status_t gemm_f16_f32acc(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                              gemm_order_t order_a, const uint16_t* B, int64_t ldb, gemm_order_t order_b,
                              float* C, int64_t ldc, gemm_order_t order_c, hipStream_t stream) {
    return gemm::run(gemm::In::F16, GEMM_ALGO_AUTO, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc,
                     order_c, stream);
}

gemm_status_t gemm_f16_f32acc_algo(gemm_algo_t algo, int64_t M, int64_t N, int64_t K, const uint16_t* A,
                                   int64_t lda, gemm_order_t order_a, const uint16_t* B, int64_t ldb,
                                   gemm_order_t order_b, float* C, int64_t ldc, gemm_order_t order_c,
                                   hipStream_t stream) {
    return gemm::run(gemm::In::F16, algo, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, stream);
}

gemm_status_t gemm_f16_f32acc_ws(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                 gemm_order_t order_a, const uint16_t* B, int64_t ldb, gemm_order_t order_b,
                                 float* C, int64_t ldc, gemm_order_t order_c, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    return gemm::run(gemm::In::F16, GEMM_ALGO_AUTO, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc,
                     order_c, stream, gemm::Workspace{workspace, workspace_bytes});
}

gemm_status_t gemm_f32_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const float* A,
                                       int64_t lda, int64_t stride_a, gemm_order_t order_a, const float* B,
                                       int64_t ldb, int64_t stride_b, gemm_order_t order_b, float* C,
                                       int64_t ldc, int64_t stride_c, gemm_order_t order_c, hipStream_t stream) {
    return gemm::run_batched(gemm::In::F32, batch, M, N, K, A, lda, stride_a, order_a, B, ldb, stride_b, order_b,
                             C, ldc, stride_c, order_c, stream);
}

gemm_status_t gemm_bf16_f32acc_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                                               const uint16_t* A, int64_t lda, int64_t stride_a,
                                               gemm_order_t order_a, const uint16_t* B, int64_t ldb,
                                               int64_t stride_b, gemm_order_t order_b, float* C, int64_t ldc,
                                               int64_t stride_c, gemm_order_t order_c, hipStream_t stream) {
    return gemm::run_batched(gemm::In::BF16, batch, M, N, K, A, lda, stride_a, order_a, B, ldb, stride_b, order_b,
                             C, ldc, stride_c, order_c, stream);
}

gemm_status_t gemm_f16_f32acc_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                                              const uint16_t* A, int64_t lda, int64_t stride_a,
                                              gemm_order_t order_a, const uint16_t* B, int64_t ldb,
                                              int64_t stride_b, gemm_order_t order_b, float* C, int64_t ldc,
                                              int64_t stride_c, gemm_order_t order_c, hipStream_t stream) {
    return gemm::run_batched(gemm::In::F16, batch, M, N, K, A, lda, stride_a, order_a, B, ldb, stride_b, order_b,
                             C, ldc, stride_c, order_c, stream);
}

const char* gemm_status_string(gemm_status_t status) {
    switch (status) {
        case GEMM_OK: return "GEMM_OK";
        case GEMM_ERR_INVALID_VALUE: return "GEMM_ERR_INVALID_VALUE: invalid argument";
        case GEMM_ERR_UNSUPPORTED_DEVICE: return "GEMM_ERR_UNSUPPORTED_DEVICE: current device is not gfx950";
        case GEMM_ERR_LAUNCH: return "GEMM_ERR_LAUNCH: kernel launch failed";
        case GEMM_ERR_SCRATCH_TOO_SMALL:
            return "GEMM_ERR_SCRATCH_TOO_SMALL: the problem's split-K partial sums need more than the library's "
                   "static scratch (GEMM_NOALLOC_SCRATCH_BYTES); use gemm_bf16_f32acc_ws with a workspace";
    }
    return "unknown gemm_status_t";
}

int gemm_last_hip_error(void) { return gemm::t_last_hip_error; }

const char* gemm_last_kernel(void) { return gemm::t_last_kernel; }

const char* gemm_version(void) { return "0.1.0"; }

}  // extern "C"
