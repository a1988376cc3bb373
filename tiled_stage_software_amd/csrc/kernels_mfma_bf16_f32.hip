// kernels_mfma_bf16_f32.hip -- the matrix-core kernels for bf16 inputs and a f32 C
// (explicit instantiation of the launch tables in mfma.hpp).
#include "mfma.hpp"

namespace gemm {
template hipError_t ring_dispatch<__bf16, DT_F32>(int tile, int S, const GemmParams& p, hipStream_t st);
template hipError_t staged_dispatch<__bf16, DT_F32>(int tile, int S, const GemmParams& p, hipStream_t st);
}  // namespace gemm
