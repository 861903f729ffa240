// C = 0 for an empty sum (K == 0).  A plain store kernel rather than hipMemsetAsync so
// that a strided C (ldc > N) is handled and so that the call stays a kernel node if a
// caller captures it in a graph.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

// C = 0 on an M x N block: four columns per thread (16-byte stores where `vec`), rows along
// grid y (strided when M exceeds it), strided-batch entries along grid z.
__global__ __launch_bounds__(256) void k_zero_c(float* C, int M, int N, int64_t ldc, int64_t sc, int vec) {
    C += blockIdx.z * sc;     // entry of a strided batch (0 for one problem)
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= N) return;
    for (int64_t r = blockIdx.y; r < M; r += gridDim.y) {
        float* row = C + r * ldc;
        if (vec && c + 3 < N) {
            *reinterpret_cast<float4*>(row + c) = make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            for (int e = 0; e < 4 && c + e < N; ++e) row[c + e] = 0.f;
        }
    }
}

// The fused epilogue of an empty sum (K == 0): C = act(beta * C + bias).
__global__ __launch_bounds__(256) void k_epi_fill(EpiProblem p) {
    const int64_t total = (int64_t)p.M * p.N;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(e / p.N), c = (int)(e % p.N);
        const int64_t off = (int64_t)r * p.ldc + c;
        epi_store(p.e, p.C, off, epi_value(p.e, 0.f, p.C, off, r, c));
    }
}

// The second step of split-K: C += slab 0 + slab 1 + ... + slab S-1, added in that order (every
// call sums the same way, so results are identical from call to call).  The slabs are dense
// M x N; four columns per thread, 16-byte accesses when C's rows allow them (vec).
__global__ __launch_bounds__(256) void k_add_slabs(float* C, int64_t ldc, int M, int N, const float* part, int S,
                                                   int vec) {
    const int64_t groups = (N + 3) / 4, total = (int64_t)M * groups, slab = (int64_t)M * N;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(t / groups), c = 4 * (int)(t % groups);
        const int64_t off = (int64_t)r * N + c;
        float* dst = C + (int64_t)r * ldc + c;
        if (vec && c + 3 < N) {
            float4 acc = *reinterpret_cast<const float4*>(dst);
            for (int z = 0; z < S; ++z) {
                const float4 v = *reinterpret_cast<const float4*>(part + z * slab + off);
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
            }
            *reinterpret_cast<float4*>(dst) = acc;
        } else {
            for (int e = 0; e < 4 && c + e < N; ++e) {
                float acc = dst[e];
                for (int z = 0; z < S; ++z) acc += part[z * slab + off + e];
                dst[e] = acc;
            }
        }
    }
}

}  // namespace

hipError_t launch_add_slabs(float* C, int64_t ldc, int M, int N, const float* part, int slabs, const Launch& l) {
    if (slabs <= 0 || M == 0 || N == 0) return hipSuccess;
    const int64_t total = (int64_t)M * ((N + 3) / 4);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    const int vec = l.vec_c && (N % 4) == 0;
    hipLaunchKernelGGL(k_add_slabs, dim3((unsigned)blocks), dim3(256), 0, l.stream, C, ldc, M, N, part, slabs, vec);
    return hipGetLastError();
}

hipError_t launch_epi_fill(const EpiProblem& p, const Launch& l) {
    const int64_t total = (int64_t)p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_epi_fill, dim3((unsigned)blocks), dim3(256), 0, l.stream, p);
    return hipGetLastError();
}

hipError_t launch_zero_c(const Problem& p, const Launch& l) {
    if (p.M <= 0 || p.N <= 0) return hipSuccess;
    const unsigned gx = (unsigned)(((int64_t)p.N + 1023) / 1024);
    const unsigned gy = (unsigned)std::min<int64_t>(p.M, 1024);
    hipLaunchKernelGGL(k_zero_c, dim3(gx, gy, (unsigned)l.batch), dim3(256), 0, l.stream, p.C, p.M, p.N, p.ldc,
                       l.batch > 1 ? l.sc : (int64_t)0, (int)l.vec_c);
    return hipGetLastError();
}

}  // namespace gemm
