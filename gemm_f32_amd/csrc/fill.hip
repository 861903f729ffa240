// C = 0 for an empty sum (K == 0).  A plain store kernel rather than hipMemsetAsync so
// that a strided C (ldc > N) is handled and so that the call stays a kernel node if a
// caller captures it in a graph.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace gemm {
namespace {

__global__ __launch_bounds__(256) void k_zero_c(float* C, int M, int N, int64_t ldc, int64_t sc) {
    C += blockIdx.y * sc;     // entry of a strided batch (0 for one problem)
    const int64_t total = (int64_t)M * N;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = e / N, c = e % N;
        C[r * ldc + c] = 0.f;
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

}  // namespace

hipError_t launch_epi_fill(const EpiProblem& p, const Launch& l) {
    const int64_t total = (int64_t)p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_epi_fill, dim3((unsigned)blocks), dim3(256), 0, l.stream, p);
    return hipGetLastError();
}

hipError_t launch_zero_c(const Problem& p, const Launch& l) {
    const int64_t total = (int64_t)p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (l.batch > 1 && blocks > 64) blocks = 64;     // the batch fills the grid along y
    hipLaunchKernelGGL(k_zero_c, dim3((unsigned)blocks, (unsigned)l.batch), dim3(256), 0, l.stream, p.C, p.M, p.N,
                       p.ldc, l.batch > 1 ? l.sc : (int64_t)0);
    return hipGetLastError();
}

}  // namespace gemm
