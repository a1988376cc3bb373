// kernels_copy.hip -- an nStage-pipelined streaming copy, the bandwidth-bound control of
// software pipelining ("Software Pipelining and Double Buffering", "When it pays": more
// stages change nothing once a kernel already saturates memory bandwidth).
//
// Each workgroup streams a contiguous run of 16 KiB slabs through the same LDS ring and
// the same K-loop template (schedule.hpp) as the GEMM kernels: a slab is copied
// global->LDS by LDS-DMA loads into ring slot (slab mod S), and written out from LDS to
// the destination in two halves -- the "fragment read" of a half is its LDS read, the
// "math" its global store.  Nothing but the stage count differs between variants.
#include "common.hpp"
#include "loaders.hpp"
#include "launch.hpp"
#include "schedule.hpp"

namespace gemm {

template <int S>
struct CopyRingOps {
    static constexpr int KS = 2;                                  // halves written per slab
    static constexpr int NW = kCopyThreads / 64;
    static constexpr int L = kCopySlab / 1024 / NW;               // 1 KiB copies per wave per slab
    static_assert(L == 4, "one M0 value and immediates 0..3 KiB per wave and slab");
    static constexpr int HALF = kCopySlab / KS;
    static constexpr int PER_T = HALF / 16 / kCopyThreads;        // 16-byte vectors per thread per half

    LDS_AS char* smem;
    const char* src;       // this workgroup's first source slab
    char* dst;             // and destination slab
    uint32_t voff;         // lane's byte within its wave's 4 KiB band
    int band;              // wave's band offset in a slab
    u32x4 r[2][PER_T];     // one half of a slab, double-buffered like MFMA fragments
    char* d[2];

    __device__ __forceinline__ void issue(int slab, int slot, int part, int parts) {
        const int c0 = part * L / parts, c1 = (part + 1) * L / parts;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(src + (int64_t)slab * kCopySlab), (short)0, -1, kBufferFlags);
        LDS_AS char* m0 = smem + slot * kCopySlab + band;
        if (c0 <= 0 && 0 < c1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, m0, 16, voff, 0, 0, 0);
        if (c0 <= 1 && 1 < c1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, m0, 16, voff, 0, 1024, 0);
        if (c0 <= 2 && 2 < c1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, m0, 16, voff, 0, 2048, 0);
        if (c0 <= 3 && 3 < c1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, m0, 16, voff, 0, 3072, 0);
    }
    template <int N>
    __device__ __forceinline__ void wait_slabs() { wait_vm<N * L>(); }
    __device__ __forceinline__ void wait_lds() { wait_lgkm0(); }
    __device__ __forceinline__ void barrier() { gemm::barrier(); }
    // LDS read of half `ks` of slab `kt` (in ring slot `slot`) into buffer BUF.
    template <int BUF>
    __device__ __forceinline__ void frag(int kt, int slot, int ks) {
        LDS_AS const char* h = smem + slot * kCopySlab + ks * HALF + threadIdx.x * 16;
#pragma unroll
        for (int j = 0; j < PER_T; ++j) r[BUF][j] = *reinterpret_cast<LDS_AS const u32x4*>(h + j * kCopyThreads * 16);
        d[BUF] = dst + (int64_t)kt * kCopySlab + ks * HALF + threadIdx.x * 16;
    }
    // Global store of the half held in buffer BUF.
    template <int BUF, int HAS, int PARTS>
    __device__ __forceinline__ void math(int) {
#pragma unroll
        for (int j = 0; j < PER_T; ++j) *reinterpret_cast<u32x4*>(d[BUF] + j * kCopyThreads * 16) = r[BUF][j];
    }
};

template <int S>
__global__ __launch_bounds__(kCopyThreads) void pipe_copy_kernel(const CopyParams p) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[S * kCopySlab];
    const int64_t first = (int64_t)blockIdx.x * p.per_wg;
    int64_t n = p.slabs - first;
    if (n > p.per_wg) n = p.per_wg;
    if (n <= 0) return;
    CopyRingOps<S> ops;
    ops.smem = (LDS_AS char*)(smem_raw);
    ops.src = p.src + first * kCopySlab;
    ops.dst = p.dst + first * kCopySlab;
    ops.band = wave_id() * (CopyRingOps<S>::L * 1024);
    ops.voff = (uint32_t)(ops.band + lane_id() * 16);
    gemm_sched::ring_mainloop<S, CopyRingOps<S>::KS, 0>(ops, (int)n);
}

hipError_t launch_pipe_copy(int nstage, const CopyParams& p, int64_t grid, hipStream_t st) {
    switch (nstage) {
        case 1: hipLaunchKernelGGL(pipe_copy_kernel<1>, dim3((unsigned)grid), dim3(kCopyThreads), 0, st, p); break;
        case 2: hipLaunchKernelGGL(pipe_copy_kernel<2>, dim3((unsigned)grid), dim3(kCopyThreads), 0, st, p); break;
        case 3: hipLaunchKernelGGL(pipe_copy_kernel<3>, dim3((unsigned)grid), dim3(kCopyThreads), 0, st, p); break;
        case 4: hipLaunchKernelGGL(pipe_copy_kernel<4>, dim3((unsigned)grid), dim3(kCopyThreads), 0, st, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gemm
