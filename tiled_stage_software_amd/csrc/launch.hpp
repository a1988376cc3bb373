// launch.hpp -- host-side launchers of the kernel families (internal to the library).
#pragma once

#include "common.hpp"

namespace gemm {

// Each launcher enqueues one kernel on `st` and returns hipGetLastError() (or
// hipErrorInvalidValue for a tile / stage combination that is not instantiated).
hipError_t launch_valu_ring(int tile, int nstage, const GemmParams& p, hipStream_t st);
hipError_t launch_valu_staged(int tile, int nstage, const GemmParams& p, hipStream_t st);
hipError_t launch_mfma_ring(int in_type, int tile, int nstage, const GemmParams& p, hipStream_t st);
hipError_t launch_mfma_staged(int in_type, int tile, int nstage, const GemmParams& p, hipStream_t st);
hipError_t launch_scale(const GemmParams& p, hipStream_t st);

// Compute units of the current device (cached per device in an atomic, so concurrent
// first calls are safe; 256 when no device can be queried, e.g. planning on a host
// without a GPU).
int num_compute_units();

// Pipelined streaming copy (the bandwidth-bound control): `slabs` slabs of kCopySlab
// bytes, per_wg consecutive slabs per workgroup.
constexpr int kCopySlab = 16384;
constexpr int kCopyThreads = 256;
struct CopyParams {
    const char* src;
    char* dst;
    int64_t slabs;
    int64_t per_wg;
};
hipError_t launch_pipe_copy(int nstage, const CopyParams& p, int64_t grid, hipStream_t st);

// Matrix instructions on register operands (the compute-bound control): `grid` workgroups
// of kCeilThreads; frags holds kCeilFrags fragments of 64 lanes x 8 16-bit values; sums one
// float per thread.  mi = 16 or 32, in_type DT_BF16 or DT_F16.
constexpr int kCeilThreads = 512;
constexpr int kCeilFrags = 32;
hipError_t launch_mfma_ceiling(int in_type, int mi, const uint16_t* frags, float* sums, int64_t grid, int64_t iters,
                               hipStream_t st);

// Operand repacking for the direct ring: dst is rows x len_pad 16-bit elements,
// row-major, 16-byte aligned (len_pad a multiple of 64); dst[r][c] = src(r, c) for
// c < len, +0 beyond, with src(r, c) = src[r*ld + c] (trans = 0) or src[c*ld + r]
// (trans = 1).  A job with rows == 0 is skipped.  tiles_c / ntiles / blocks are filled
// by the launcher.
constexpr int kPackThreads = 256;
struct PackJob {
    const uint16_t* src;
    uint16_t* dst;
    int64_t ld;
    int rows, len, len_pad, trans;
    int tiles_c, ntiles, blocks;
};
struct PackParams {
    PackJob job[2];
};
hipError_t launch_pack(PackParams p, hipStream_t st);

// The library's own workspace for gemm_ws_static: a static device array of
// kStaticWsBytes per GPU (256-byte aligned), for callers that cannot allocate.  *ptr =
// its device address on the current device (looked up once per device).
constexpr int64_t kStaticWsBytes = int64_t(32) << 20;
hipError_t static_workspace(void** ptr);

}  // namespace gemm
