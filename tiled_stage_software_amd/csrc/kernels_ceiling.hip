// kernels_ceiling.hip -- the compute-bound control: matrix instructions on operands held in
// registers, with no memory traffic inside the loop.  The streaming copy (kernels_copy.hip)
// shows what the card's memory delivers; this kernel shows what its matrix cores sustain at
// the clock the card's power limit allows for a given operand distribution (random values
// switch more of the multiplier arrays than zeros, so the card clocks lower on them).  A
// GEMM kernel's fraction of this figure, on operands of the same distribution, separates
// what its feed and overlap lose from what the card itself cannot give.
//
// A workgroup is 8 waves, two per SIMD, as the GEMM kernels run.  Each wave loads R k-steps
// of WA first-operand and WB second-operand fragments once, then repeats `iters` times the
// inner product of a GEMM k-loop: for each k-step, WA x WB instructions into WA x WB
// independent accumulators.  Both instruction shapes do 2^20 FLOPs per wave and iteration
// (16x16x32: R 4, 4 x 4 accumulators; 32x32x16: R 8, 2 x 2).  At the end every lane writes
// the sum of all its accumulator values in a fixed order, so no instruction can be dropped
// and small-integer operands give exact sums.
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"

namespace gemm {

template <int MI>
struct CeilShape;
template <>
struct CeilShape<16> {
    static constexpr int R = 4, WA = 4, WB = 4;
};
template <>
struct CeilShape<32> {
    static constexpr int R = 8, WA = 2, WB = 2;
};

template <typename T, int MI>
__global__ __launch_bounds__(kCeilThreads) void mfma_ceiling_kernel(const uint16_t* __restrict__ frags,
                                                                     float* __restrict__ sums, int64_t iters) {
    typedef Mfma<T, MI> Op;
    typedef typename Op::frag F;
    typedef typename Op::acc Acc;
    constexpr int R = CeilShape<MI>::R, WA = CeilShape<MI>::WA, WB = CeilShape<MI>::WB;
    static_assert(R * (WA + WB) == kCeilFrags, "every shape reads the whole fragment set");
    static_assert(R * WA * WB * 2 * MI * MI * (512 / MI) == (1 << 20), "2^20 FLOPs per wave and iteration");
    const int lane = lane_id();
    F a[R][WA], b[R][WB];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int i = 0; i < WA; ++i)
            a[r][i] = *reinterpret_cast<const F*>(frags + ((r * (WA + WB) + i) * 64 + lane) * 8);
#pragma unroll
        for (int j = 0; j < WB; ++j)
            b[r][j] = *reinterpret_cast<const F*>(frags + ((r * (WA + WB) + WA + j) * 64 + lane) * 8);
    }
    Acc acc[WA][WB];
#pragma unroll
    for (int i = 0; i < WA; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j) acc[i][j] = Acc{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < WA; ++i)
#pragma unroll
                for (int j = 0; j < WB; ++j) acc[i][j] = Op::run(a[r][i], b[r][j], acc[i][j]);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < WA; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j)
#pragma unroll
            for (int e = 0; e < MI * MI / 64; ++e) s += acc[i][j][e];
    sums[((int64_t)blockIdx.x * (kCeilThreads / 64) + wave_id()) * 64 + lane] = s;
}

hipError_t launch_mfma_ceiling(int in_type, int mi, const uint16_t* frags, float* sums, int64_t grid, int64_t iters,
                               hipStream_t st) {
    const dim3 g((unsigned)grid), b(kCeilThreads);
    if (in_type == DT_BF16 && mi == 16)
        hipLaunchKernelGGL((mfma_ceiling_kernel<__bf16, 16>), g, b, 0, st, frags, sums, iters);
    else if (in_type == DT_BF16 && mi == 32)
        hipLaunchKernelGGL((mfma_ceiling_kernel<__bf16, 32>), g, b, 0, st, frags, sums, iters);
    else if (in_type == DT_F16 && mi == 16)
        hipLaunchKernelGGL((mfma_ceiling_kernel<_Float16, 16>), g, b, 0, st, frags, sums, iters);
    else if (in_type == DT_F16 && mi == 32)
        hipLaunchKernelGGL((mfma_ceiling_kernel<_Float16, 32>), g, b, 0, st, frags, sums, iters);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gemm
