// kernels_mfma.hip -- dispatch of the matrix-core GEMM on the input / output type pair.
// The kernels themselves are in mfma.hpp, instantiated once per pair by the
// kernels_mfma_<in>_<out>.hip units.
#include "common.hpp"
#include "launch.hpp"

namespace gemm {

template <typename T, int OUT>
hipError_t ring_dispatch(int tile, int S, const GemmParams& p, hipStream_t st);
template <typename T, int OUT>
hipError_t staged_dispatch(int tile, int S, const GemmParams& p, hipStream_t st);

extern template hipError_t ring_dispatch<__bf16, DT_BF16>(int, int, const GemmParams&, hipStream_t);
extern template hipError_t ring_dispatch<__bf16, DT_F32>(int, int, const GemmParams&, hipStream_t);
extern template hipError_t ring_dispatch<_Float16, DT_F16>(int, int, const GemmParams&, hipStream_t);
extern template hipError_t ring_dispatch<_Float16, DT_F32>(int, int, const GemmParams&, hipStream_t);
extern template hipError_t staged_dispatch<__bf16, DT_BF16>(int, int, const GemmParams&, hipStream_t);
extern template hipError_t staged_dispatch<__bf16, DT_F32>(int, int, const GemmParams&, hipStream_t);
extern template hipError_t staged_dispatch<_Float16, DT_F16>(int, int, const GemmParams&, hipStream_t);
extern template hipError_t staged_dispatch<_Float16, DT_F32>(int, int, const GemmParams&, hipStream_t);

// C is fp32 or the input type.
hipError_t launch_mfma_ring(int in_type, int tile, int nstage, const GemmParams& p, hipStream_t st) {
    if (in_type == DT_BF16)
        return p.out_type == DT_F32 ? ring_dispatch<__bf16, DT_F32>(tile, nstage, p, st)
                                    : ring_dispatch<__bf16, DT_BF16>(tile, nstage, p, st);
    return p.out_type == DT_F32 ? ring_dispatch<_Float16, DT_F32>(tile, nstage, p, st)
                                : ring_dispatch<_Float16, DT_F16>(tile, nstage, p, st);
}
hipError_t launch_mfma_staged(int in_type, int tile, int nstage, const GemmParams& p, hipStream_t st) {
    if (in_type == DT_BF16)
        return p.out_type == DT_F32 ? staged_dispatch<__bf16, DT_F32>(tile, nstage, p, st)
                                    : staged_dispatch<__bf16, DT_BF16>(tile, nstage, p, st);
    return p.out_type == DT_F32 ? staged_dispatch<_Float16, DT_F32>(tile, nstage, p, st)
                                : staged_dispatch<_Float16, DT_F16>(tile, nstage, p, st);
}

}  // namespace gemm
