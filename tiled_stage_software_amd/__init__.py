"""libgemm for AMD MI355X (gfx950): tiled, software-pipelined GEMM with hand-written HIP
kernels behind a C ABI (include/libgemm.h).  This package holds the HIP sources
(csrc/), the in-tree build (build.py), the ctypes binding (libgemm.py) and the seeded
input generators (inputs.py)."""
from .libgemm import (GEMM_OK, GEMM_ERR_INVALID_ARG, GEMM_ERR_UNSUPPORTED, GEMM_ERR_HIP,  # noqa: F401
                      GEMM_ROW_MAJOR, GEMM_COL_MAJOR, GEMM_F32, GEMM_BF16, GEMM_F16,
                      GEMM_KERNEL_AUTO, GEMM_KERNEL_VALU_RING, GEMM_KERNEL_VALU_STAGED,
                      GEMM_KERNEL_MFMA_RING, GEMM_KERNEL_MFMA_STAGED, GEMM_KERNEL_SCALE,
                      GemmError, GemmOpts, GemmPlan, matmul, load)
