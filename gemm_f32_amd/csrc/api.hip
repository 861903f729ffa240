// libgemm's C ABI: argument validation, normalisation of a column-major C, kernel choice
// and launch.  The operation and its contract are documented in include/gemm.h.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "gemm.h"
#include "common.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

thread_local int t_last_hip_error = 0;
thread_local const char* t_last_kernel = "none";

enum class In { F32, BF16 };

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

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

gemm_status_t validate(In in, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                       int oa, const void* B, int64_t ldb, int ob, const void* C, int64_t ldc,
                       int oc) {
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
    const uintptr_t e = in == In::F32 ? 4 : 2;
    if (!aligned(A, e) || !aligned(B, e) || !aligned(C, 4)) return GEMM_ERR_INVALID_VALUE;
    return GEMM_OK;
}

int pick_group_m(int tiles_m, int tiles_n) {
    // Make the run of tiles that one XCD receives (total / 8 consecutive ids) cover a
    // near-square patch of C: group_m x (per_xcd / group_m) tiles.
    const int per_xcd = (tiles_m * tiles_n) / kNumXcds;
    int g = 1;
    while (2 * g <= tiles_m && (2 * g) * (2 * g) <= per_xcd) g *= 2;
    return g;
}

int64_t tiles(int64_t M, int64_t N, int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); }

// AUTO takes the small-problem kernel for few rows, or when even 64 x 64 tiles would leave
// more than half of the CUs idle (each such tile walks all of K alone).  For FP32 also when
// 128 x 128 tiles cannot give every CU one: its K split over eight wavefronts then beats
// the tile kernels, whose few tiles each wait on memory latency (1000^3: 58 -> 30 us).
bool prefer_small(const Problem& p, int cus, bool f32) {
    const int64_t c = cus > 0 ? cus : 256;
    return p.M <= kSkinnyMaxM || tiles(p.M, p.N, 64, 64) * 2 < c || (f32 && tiles(p.M, p.N, 128, 128) < c);
}

// The small-problem kernel, with 1 or 4 column blocks of 16 per workgroup.
hipError_t run_skinny(const Problem& p, const Launch& l, bool bf16, int cus, const char*& name) {
    const int fn = skinny_blocks(p, cus);
    name = bf16 ? (fn == 4 ? "bf16_skinny64" : "bf16_skinny16") : (fn == 4 ? "f32_skinny64" : "f32_skinny16");
    return launch_skinny(p, l, bf16, fn);
}

// Block-tile choice.  The grid runs in rounds of cus x per_cu resident blocks (per_cu: how
// many blocks of that kernel share a CU); a CU's round costs (blocks it holds) x (work per
// tile / relative throughput of the tile size), so estimate time as the sum over rounds and
// take the cheapest.  Relative throughputs are the kernels' measured rates at 4096^3 with full
// rounds.
struct TileOpt { int bm, bn; double eff; int per_cu; };
constexpr TileOpt kBf16Tiles[] = {{256, 256, 1.0, 1}, {256, 128, 0.78, 1}, {128, 128, 0.82, 2},
                                  {64, 64, 0.36, 4}};
// BF16 direct-copy kernel (256 x 256, 256 x 128) alone, and together with the
// register-staged kernel's smaller tiles (bm == 256 marks the direct-copy kernel)
constexpr TileOpt kBf16DmaTiles[] = {{256, 256, 1.0, 1}, {256, 128, 0.86, 1}};
constexpr TileOpt kBf16AnyTiles[] = {{256, 256, 1.0, 1}, {256, 128, 0.86, 1}, {128, 128, 0.80, 2},
                                     {64, 64, 0.35, 4}};
// FP32: the register-staged kernel (128 x 128, 64 x 64) and, where its requirements hold,
// the direct-copy kernel (256 x 256, 128 x 128) with the register-staged 64 x 64
constexpr TileOpt kF32Tiles[] = {{128, 128, 1.0, 4}, {64, 64, 0.92, 4}};
constexpr TileOpt kF32DmaTiles[] = {{256, 256, 1.0, 1}, {128, 128, 0.85, 2}, {64, 64, 0.76, 4}};

template <size_t NOPT>
void pick_tile(const TileOpt (&opts)[NOPT], int64_t M, int64_t N, int cus, int& bm, int& bn) {
    double best = 1e300;
    for (const TileOpt& o : opts) {
        const double c = cus > 0 ? cus : 256, n = (double)tiles(M, N, o.bm, o.bn);
        const double full = std::floor(n / (c * o.per_cu)), rest = n - full * c * o.per_cu;
        const double cost = (full * o.per_cu + std::ceil(rest / c)) * o.bm * o.bn / o.eff;
        if (cost < best) { best = cost; bm = o.bm; bn = o.bn; }
    }
}

// FP32 direct-copy kernel on the whole bt x bt tiles of C, the register-staged kernel on
// the partial strips along the bottom and right edges (same stream, disjoint parts of C).
hipError_t launch_f32_dma_split(const Problem& p, const Launch& l, int bt, int cus) {
    const int mf = p.M / bt * bt, nf = p.N / bt * bt;
    Problem core = p;
    core.M = mf;
    core.N = nf;
    Launch lc = l;
    lc.group_m = pick_group_m(mf / bt, nf / bt);
    hipError_t err = launch_f32_dma(core, lc, bt, bt);
    auto strip = [&](Problem s) {
        if (err != hipSuccess) return;
        int bm = 128, bn = 128;
        pick_tile(kF32Tiles, s.M, s.N, cus, bm, bn);
        Launch ls = l;
        ls.group_m = pick_group_m((s.M + bm - 1) / bm, (s.N + bn - 1) / bn);
        err = launch_f32_mfma(s, ls, bm);
    };
    const float* A = static_cast<const float*>(p.A);
    const float* B = static_cast<const float*>(p.B);
    if (mf < p.M) {          // rows mf .. M-1, all columns
        Problem s = p;
        s.M = p.M - mf;
        s.A = A + (p.oa == kRow ? (int64_t)mf * p.lda : (int64_t)mf);
        s.C = p.C + (int64_t)mf * p.ldc;
        strip(s);
    }
    if (nf < p.N) {          // rows 0 .. mf-1, columns nf .. N-1
        Problem s = p;
        s.M = mf;
        s.N = p.N - nf;
        s.B = B + (p.ob == kCol ? (int64_t)nf * p.ldb : (int64_t)nf);
        s.C = p.C + nf;
        strip(s);
    }
    return err;
}

template <typename Elem>
gemm_status_t run(In in, gemm_algo_t algo, int64_t M, int64_t N, int64_t K, const Elem* A,
                  int64_t lda, gemm_order_t oa, const Elem* B, int64_t ldb, gemm_order_t ob,
                  float* C, int64_t ldc, gemm_order_t oc, hipStream_t stream) {
    gemm_status_t st = validate(in, M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc);
    if (st != GEMM_OK) return st;
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
        case GEMM_ALGO_MFMA_256x128: case GEMM_ALGO_MFMA_PINGPONG:
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
    Launch l{};
    l.stream = stream;
    // 16-byte loads and global->LDS copies need only element alignment on gfx950
    l.vec_a = l.vec_b = true;
    l.vec_c = (p.ldc % 4 == 0) && aligned(p.C, 16);

    hipError_t err = hipSuccess;
    const char* name = "none";
    if (K == 0) {
        err = launch_zero_c(p, l);
        name = "zero_c";
    } else if (f32) {
        switch (algo) {
            case GEMM_ALGO_NAIVE_UNCOALESCED:
                err = launch_naive(p, l, false); name = "f32_naive_uncoalesced"; break;
            case GEMM_ALGO_NAIVE:
                err = launch_naive(p, l, true); name = "f32_naive"; break;
            case GEMM_ALGO_TILED:
                err = launch_tiled(p, l); name = "f32_tiled32"; break;
            case GEMM_ALGO_REGBLOCK: {
                l.group_m = pick_group_m((p.M + kRegblockBM - 1) / kRegblockBM,
                                         (p.N + kRegblockBN - 1) / kRegblockBN);
                err = launch_regblock(p, l); name = "f32_regblock128x128"; break;
            }
            case GEMM_ALGO_SKINNY:
                if (!skinny_applies(p, false)) return GEMM_ERR_INVALID_VALUE;
                err = run_skinny(p, l, false, dev.cus, name); break;
            default: {
                if (algo == GEMM_ALGO_AUTO && prefer_small(p, dev.cus, true) && skinny_applies(p, false)) {
                    err = run_skinny(p, l, false, dev.cus, name); break;
                }
                // direct-copy kernel (tiles 256 or 128) where it applies, else register-staged
                const bool dma256 = f32_dma_applies(p, l, 256, 256);
                const bool dma128 = f32_dma_applies(p, l, 128, 128);
                int bm = 128, bn = 128;
                bool dma = false;
                if (algo == GEMM_ALGO_MFMA_64x64) {
                    bm = bn = 64;
                } else if (algo == GEMM_ALGO_MFMA_128x128) {
                    bm = bn = 128;
                } else if (algo == GEMM_ALGO_MFMA_256x256) {
                    if (!dma256) return GEMM_ERR_INVALID_VALUE;
                    bm = bn = 256;
                    dma = true;
                } else if (algo == GEMM_ALGO_MFMA_DMA) {
                    if (!dma128) return GEMM_ERR_INVALID_VALUE;
                    bm = bn = 128;
                    if (dma256) pick_tile(kF32DmaTiles, p.M, p.N, dev.cus, bm, bn);
                    if (bm != 256) bm = bn = 128;
                    dma = true;
                } else if (dma128) {
                    pick_tile(kF32DmaTiles, p.M, p.N, dev.cus, bm, bn);
                    if (bm == 256 && !dma256) bm = bn = 128;
                    dma = bm >= 128;
                } else {
                    pick_tile(kF32Tiles, p.M, p.N, dev.cus, bm, bn);
                }
                if (dma) {
                    err = launch_f32_dma_split(p, l, bm, dev.cus);
                    name = bm == 256 ? "f32_dma256x256" : "f32_dma128x128";
                    break;
                }
                l.group_m = pick_group_m((p.M + bm - 1) / bm, (p.N + bn - 1) / bn);
                err = launch_f32_mfma(p, l, bm);
                name = bm == 64 ? "f32_mfma64x64" : "f32_mfma128x128";
                break;
            }
        }
    } else if (algo == GEMM_ALGO_SKINNY ||
               (algo == GEMM_ALGO_AUTO && prefer_small(p, dev.cus, false) && skinny_applies(p, true))) {
        if (!skinny_applies(p, true)) return GEMM_ERR_INVALID_VALUE;
        err = run_skinny(p, l, true, dev.cus, name);
    } else if (algo == GEMM_ALGO_MFMA_PINGPONG) {
        if (!bf16_pingpong_applies(p, l)) return GEMM_ERR_INVALID_VALUE;
        l.group_m = pick_group_m(p.M / 256, p.N / 256);
        err = launch_bf16_pingpong(p, l);
        name = "bf16_pingpong256x256";
    } else {
        int bm = 256, bn = 256;
        const bool dma = bf16_dma_applies(p, l, bm, bn);
        switch (algo) {
            case GEMM_ALGO_MFMA_256x256: bm = 256; bn = 256; break;
            case GEMM_ALGO_MFMA_256x128: bm = 256; bn = 128; break;
            case GEMM_ALGO_MFMA_128x128: bm = 128; bn = 128; break;
            case GEMM_ALGO_MFMA_64x64: bm = 64; bn = 64; break;
            case GEMM_ALGO_MFMA_DMA:
                if (!dma) return GEMM_ERR_INVALID_VALUE;
                pick_tile(kBf16DmaTiles, p.M, p.N, dev.cus, bm, bn);
                break;
            default:
                // the direct-copy kernel's tiles where it applies, else the register-staged
                // / direct kernel of bf16_mfma.hip
                if (dma) pick_tile(kBf16AnyTiles, p.M, p.N, dev.cus, bm, bn);
                else pick_tile(kBf16Tiles, p.M, p.N, dev.cus, bm, bn);
                break;
        }
        // an explicitly chosen tile runs on bf16_mfma.hip
        const bool use_dma = algo == GEMM_ALGO_MFMA_DMA || ((algo == GEMM_ALGO_AUTO || algo == GEMM_ALGO_MFMA) &&
                                                            dma && bm == 256);
        l.group_m = pick_group_m((p.M + bm - 1) / bm, (p.N + bn - 1) / bn);
        if (use_dma) {
            err = launch_bf16_dma(p, l, bm, bn);
            name = bn == 256 ? "bf16_dma256x256" : "bf16_dma256x128";
        } else {
            err = launch_bf16_mfma(p, l, bm, bn);
            static const char* names[] = {"bf16_mfma256x256", "bf16_mfma256x128", "bf16_mfma128x128",
                                          "bf16_mfma64x64"};
            name = names[bm == 256 ? (bn == 256 ? 0 : 1) : (bm == 128 ? 2 : 3)];
        }
    }
    if (err != hipSuccess) {
        t_last_hip_error = (int)err;
        return GEMM_ERR_LAUNCH;
    }
    t_last_kernel = name;
    return GEMM_OK;
}

}  // namespace
}  // namespace gemm

extern "C" {

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

const char* gemm_status_string(gemm_status_t status) {
    switch (status) {
        case GEMM_OK: return "GEMM_OK";
        case GEMM_ERR_INVALID_VALUE: return "GEMM_ERR_INVALID_VALUE: invalid argument";
        case GEMM_ERR_UNSUPPORTED_DEVICE: return "GEMM_ERR_UNSUPPORTED_DEVICE: current device is not gfx950";
        case GEMM_ERR_LAUNCH: return "GEMM_ERR_LAUNCH: kernel launch failed";
    }
    return "unknown gemm_status_t";
}

int gemm_last_hip_error(void) { return gemm::t_last_hip_error; }

const char* gemm_last_kernel(void) { return gemm::t_last_kernel; }

const char* gemm_version(void) { return "0.1.0"; }

}  // extern "C"
