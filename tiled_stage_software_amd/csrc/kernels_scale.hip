// kernels_scale.hip -- C = beta*C, the BLAS quick return when K == 0 or alpha == 0
// (beta == 0 writes zeros without reading C).
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace gemm {

__global__ __launch_bounds__(256) void scale_kernel(const GemmParams p) {
    const int64_t total = (int64_t)p.M * p.N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t m = e / p.N;
        const int n = (int)(e - m * p.N);
        const int64_t off = m * p.ldc + n;
        if (p.out_type == DT_F32) {
            float* c = reinterpret_cast<float*>(p.C) + off;
            *c = p.beta == 0.0f ? 0.0f : p.beta * *c;
        } else {
            uint16_t* c = reinterpret_cast<uint16_t*>(p.C) + off;
            const bool bf = p.out_type == DT_BF16;
            float v = 0.0f;
            if (p.beta != 0.0f) v = p.beta * (bf ? bf16_bits_to_f32(*c) : f16_bits_to_f32(*c));
            *c = bf ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
        }
    }
}

hipError_t launch_scale(const GemmParams& p, hipStream_t st) {
    const int64_t total = (int64_t)p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(scale_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p);
    return hipGetLastError();
}

int num_compute_units() {
    // One atomic per device, so that first calls from several host threads do not race:
    // each may query, and all store the same value.
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace gemm
