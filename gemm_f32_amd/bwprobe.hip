// Read and write patterns of the few-row product, timed on their own (no arithmetic beyond a
// running sum that keeps the loads live).  Measurement tooling: not part of libgemm.
//
// The few-row product C[16 x N] = A[16 x K] B[K x N] is bound by reading B once.  How fast that
// read can go depends on the pattern the product imposes on it, not only on the bytes:
//   * plain:  the whole buffer by a grid-stride loop of 16-byte loads, 1024 workgroups
//             (the best case for these sizes);
//   * slab16: a row-major B read 16 columns (64 bytes of each row) per workgroup, 256
//             workgroups on neighbouring slabs per XCD -- what one 16-column block of C needs;
//   * skinny: the same slabs with the small-problem FP32 kernel's loads (lane l reads column
//             l % 16 of rows 4 (l / 16) + e, e = 0..3: 4-byte loads; 8 wavefronts dealing 16-row
//             k-steps in turn, 8 in flight), with or without the lane's 16 bytes of A per k-step
//             (A: 16 x K row-major, read from L2 by every workgroup);
//   * w32h:   32 columns (128 bytes of each row, 8-byte loads along N) and half of K per
//             workgroup, 256 workgroups, with or without A -- the pattern of the library's
//             two-halves mode for few FP32 rows (which adds the two halves' sums into a zeroed
//             C);
//   * chunk:  one contiguous chunk per workgroup (a column-major B, 16 columns of K elements
//             per workgroup), 256 workgroups;
//   * write:  a grid-stride loop of 16-byte stores (a C written once).
// Each entry point checks its geometry against the element count it is given and returns
// hipErrorInvalidValue instead of launching past it.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

constexpr int kSteps = 8;                 // k-steps (or rows of 16-byte loads) in flight per lane

// keeps every loaded value live without writing more than one value per lane (never, in fact,
// for finite data: the sum is compared with a constant no sum of the probe's inputs reaches)
__device__ inline void sink(float s, float* out) {
    if (s == 1.2345e30f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_plain(const float4* __restrict__ p, int64_t n4, float* out) {
    float s = 0.f;
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    for (int64_t base = (int64_t)blockIdx.x * 256 * 4 + threadIdx.x; base < n4; base += stride) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            v[u] = i < n4 ? p[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) s += v[u].x + v[u].y + v[u].z + v[u].w;
    }
    sink(s, out);
}

// slab = 32 x (block % 8) + block / 8: the 32 workgroups one XCD receives read neighbouring slabs
__device__ inline int xcd_slab(int b) { return (b % 8) * 32 + b / 8; }

__global__ __launch_bounds__(256) void k_slab16(const float* __restrict__ p, int rows, int ld, float* out) {
    const int col = xcd_slab(blockIdx.x) * 16 + (threadIdx.x & 3) * 4;
    float s = 0.f;
    for (int r0 = threadIdx.x >> 2; r0 < rows; r0 += 64 * kSteps) {
        float4 v[kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int r = r0 + 64 * u;
            v[u] = r < rows ? *reinterpret_cast<const float4*>(p + (int64_t)r * ld + col) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) s += v[u].x + v[u].y + v[u].z + v[u].w;
    }
    sink(s, out);
}

template <bool RA>
__global__ __launch_bounds__(512) void k_skinny(const float* __restrict__ b, int K, int ld, const float* __restrict__ a,
                                               float* out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, lq = lane >> 4;
    const float* col = b + xcd_slab(blockIdx.x) * 16 + li;
    const int steps = K / 16;
    float s = 0.f;
    for (int ks = wave * kSteps; ks < steps; ks += 8 * kSteps) {
        float v[kSteps][4];
        float4 av[kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int k0 = (ks + u) * 16 + 4 * lq;      // ks + u < steps: steps % kSteps == 0
#pragma unroll
            for (int e = 0; e < 4; ++e) v[u][e] = col[(int64_t)(k0 + e) * ld];
            if (RA) av[u] = *reinterpret_cast<const float4*>(a + (int64_t)li * K + k0);
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            s += v[u][0] + v[u][1] + v[u][2] + v[u][3];
            if (RA) s += av[u].x * av[u].y + av[u].z * av[u].w;
        }
    }
    sink(s, out);
}

// 32-column block cb = block % (N / 32), K half = block / (N / 32)
template <bool RA>
__global__ __launch_bounds__(512) void k_w32h(const float* __restrict__ b, int K, int ld, int nblocks,
                                             const float* __restrict__ a, float* out) {
    const int cb = blockIdx.x % nblocks, half = blockIdx.x / nblocks;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, lq = lane >> 4;
    const float* col = b + cb * 32 + 2 * li;
    const int steps = K / 32;                   // k-steps of 16 rows in one half
    float s = 0.f;
    for (int ks = wave * kSteps; ks < steps; ks += 8 * kSteps) {
        float2 v[kSteps][4];
        float4 av[kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int k0 = (half * steps + ks + u) * 16 + 4 * lq;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[u][e] = *reinterpret_cast<const float2*>(col + (int64_t)(k0 + e) * ld);
            if (RA) av[u] = *reinterpret_cast<const float4*>(a + (int64_t)li * K + k0);
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s += v[u][e].x * v[u][e].y;
            if (RA) s += av[u].x * av[u].y + av[u].z * av[u].w;
        }
    }
    sink(s, out);
}

__global__ __launch_bounds__(256) void k_chunk(const float4* __restrict__ p, int64_t chunk, float* out) {
    const float4* q = p + (int64_t)blockIdx.x * chunk;
    float s = 0.f;
    for (int64_t base = threadIdx.x; base < chunk; base += 256 * kSteps) {
        float4 v[kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            v[u] = i < chunk ? q[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) s += v[u].x + v[u].y + v[u].z + v[u].w;
    }
    sink(s, out);
}

__global__ __launch_bounds__(256) void k_write(float4* __restrict__ p, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) p[i] = make_float4(1.f, 1.f, 1.f, 1.f);
}

hipError_t done() { return hipGetLastError(); }

}  // namespace

// `out` holds at least bwprobe_out_floats() floats; `n` counts the floats of the buffer read.
extern "C" int64_t bwprobe_out_floats(void) { return 1024 * 512; }

extern "C" int bwprobe_plain(const float* p, int64_t n, float* out, hipStream_t st) {
    if (n % 4 != 0 || n <= 0) return (int)hipErrorInvalidValue;
    k_plain<<<1024, 256, 0, st>>>(reinterpret_cast<const float4*>(p), n / 4, out);
    return (int)done();
}

// B: K x N row-major floats, N == 4096 (256 slabs of 16), ld >= N
extern "C" int bwprobe_slab16(const float* b, int64_t n, int K, int N, int ld, float* out, hipStream_t st) {
    if (N != 4096 || ld < N || K <= 0 || (int64_t)K * ld > n) return (int)hipErrorInvalidValue;
    k_slab16<<<256, 256, 0, st>>>(b, K, ld, out);
    return (int)done();
}

// B as above; A: 16 x K row-major floats (na of them); K a multiple of 16 kSteps
extern "C" int bwprobe_skinny(const float* b, int64_t n, int K, int N, int ld, const float* a, int64_t na, float* out,
                              hipStream_t st) {
    if (N != 4096 || ld < N || K <= 0 || K % (16 * kSteps) != 0 || (int64_t)K * ld > n) return (int)hipErrorInvalidValue;
    if (a && na < 16 * (int64_t)K) return (int)hipErrorInvalidValue;
    if (a) k_skinny<true><<<256, 512, 0, st>>>(b, K, ld, a, out);
    else k_skinny<false><<<256, 512, 0, st>>>(b, K, ld, nullptr, out);
    return (int)done();
}

// B as above with N a multiple of 32 and 2 N / 32 workgroups; K a multiple of 32 kSteps
extern "C" int bwprobe_w32h(const float* b, int64_t n, int K, int N, int ld, const float* a, int64_t na, float* out,
                            hipStream_t st) {
    if (N <= 0 || N % 32 != 0 || N / 16 > 1024 || ld < N || K <= 0 || K % (32 * kSteps) != 0 || (int64_t)K * ld > n)
        return (int)hipErrorInvalidValue;
    if (a && na < 16 * (int64_t)K) return (int)hipErrorInvalidValue;
    if (a) k_w32h<true><<<N / 16, 512, 0, st>>>(b, K, ld, N / 32, a, out);
    else k_w32h<false><<<N / 16, 512, 0, st>>>(b, K, ld, N / 32, nullptr, out);
    return (int)done();
}

// 256 contiguous chunks of n / 256 floats (n a multiple of 1024)
extern "C" int bwprobe_chunk(const float* p, int64_t n, float* out, hipStream_t st) {
    if (n <= 0 || n % 1024 != 0) return (int)hipErrorInvalidValue;
    k_chunk<<<256, 256, 0, st>>>(reinterpret_cast<const float4*>(p), n / 1024, out);
    return (int)done();
}

extern "C" int bwprobe_write(float* p, int64_t n, hipStream_t st) {
    if (n % 4 != 0 || n <= 0) return (int)hipErrorInvalidValue;
    k_write<<<256, 256, 0, st>>>(reinterpret_cast<float4*>(p), n / 4);
    return (int)done();
}
