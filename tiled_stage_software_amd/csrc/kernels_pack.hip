// kernels_pack.hip -- repack 16-bit GEMM operands into the layout the direct-to-LDS ring
// reads: K-contiguous rows, 16-byte aligned, K zero-padded to a whole number of slabs.
//
// The ring copies 16-byte chunks straight from global memory into LDS, so it needs both
// operands K-contiguous with 16-byte aligned rows and K a multiple of the slab depth (the
// staged kernels take anything, at the cost of a trip through registers).  An operand
// that breaks one of these -- an N-contiguous B, a row pitch that is not a multiple of 8
// elements, a K tail -- is rewritten once per call into a workspace; the multiply then
// runs on the copies.  Zero padding along K adds products 0*0 = +0 to every sum, so the
// result is that of the unpadded problem.
//
// One launch handles up to two jobs (A and B).  Each workgroup owns two consecutive 64 x 64
// tiles of one job's output.  Output row r, column c (c < len_pad, a multiple of 64):
//   trans = 0: src[r*ld + c]   (the source is already contiguous along K): rows are
//              copied 16 bytes per lane, coalesced on both sides;
//   trans = 1: src[c*ld + r]   (contiguous along the other index): the tile goes through
//              LDS, read along r and written along c, so both global sides stay coalesced
//              (LDS chunks XOR-swizzled, free of bank conflicts on both sides).
// Columns c >= len are written as zeros.  The pass is bound by HBM bandwidth.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace gemm {

namespace {

constexpr int kPackTile = 64;

// LDS tile of the transposing job: row c (64 elements, 8 chunks of 16 bytes) holds the
// source line c; its chunk q (elements 8q .. 8q+7 along r) sits at chunk position
// q ^ ((c >> 3) & 7).  The loads write whole rows (8 lanes per 128-byte row); the stores
// gather one element from 8 consecutive rows per lane, with the 8 lane groups 8 rows
// apart: the swizzle puts those groups on 8 different chunks, so the 64 lanes hit 32
// distinct banks.
__device__ __forceinline__ int tile_at(int c, int r) {
    return c * kPackTile + 8 * ((r >> 3) ^ ((c >> 3) & 7)) + (r & 7);
}

// 8 consecutive 16-bit source elements starting at element `idx` (any alignment: the
// target allows unaligned 16-byte global loads).
__device__ __forceinline__ u32x4 load8(const uint16_t* src, int64_t idx) {
    u32x4 t;
    __builtin_memcpy(&t, src + idx, 16);
    return t;
}

// Elements idx + e*stride for e < n (the rest +0), packed two per word.
__device__ __forceinline__ u32x4 load8_partial(const uint16_t* src, int64_t idx, int64_t stride, int n) {
    u32x4 t = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (e < n) t[e >> 1] |= (uint32_t)src[idx + e * stride] << ((e & 1) * 16);
    return t;
}

// A workgroup packs kTilesPerWg consecutive 64 x 64 tiles of one job.  Every lane issues
// all of its loads (for all its tiles) before its first store: the compiler cannot move a
// load of src above a store to dst (they might alias), so interleaving them would leave
// one load in flight per lane.
constexpr int kTilesPerWg = 2;

__device__ __forceinline__ void tile_origin(const PackJob& j, int t, int& r0, int& c0) {
    r0 = (t / j.tiles_c) * kPackTile;
    c0 = (t % j.tiles_c) * kPackTile;
}

__device__ __forceinline__ void pack_rows(const PackJob& j, int t0, int ntiles) {
    const int t = threadIdx.x;
    u32x4 v[kTilesPerWg][2];
#pragma unroll
    for (int u = 0; u < kTilesPerWg; ++u) {
        int r0, c0;
        tile_origin(j, t0 + u, r0, c0);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int r = r0 + (t >> 3) + 32 * pass;
            const int c = c0 + 8 * (t & 7);
            const int64_t idx = (int64_t)r * j.ld + c;
            if (u >= ntiles || r >= j.rows) v[u][pass] = u32x4{0u, 0u, 0u, 0u};
            else if (c + 8 <= j.len) v[u][pass] = load8(j.src, idx);
            else v[u][pass] = load8_partial(j.src, idx, 1, j.len - c);  // K tail (n <= 0: all zeros)
        }
    }
#pragma unroll
    for (int u = 0; u < kTilesPerWg; ++u) {
        int r0, c0;
        tile_origin(j, t0 + u, r0, c0);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int r = r0 + (t >> 3) + 32 * pass;
            const int c = c0 + 8 * (t & 7);
            if (u < ntiles && r < j.rows) *reinterpret_cast<u32x4*>(j.dst + (int64_t)r * j.len_pad + c) = v[u][pass];
        }
    }
}

__device__ __forceinline__ void pack_trans(const PackJob& j, int t0, int ntiles, uint16_t* tiles) {
    const int t = threadIdx.x;
    // Load: source line c (contiguous along r), 8 consecutive r per lane; then store the
    // 8 values as one 16-byte LDS row chunk of the tile.
    u32x4 in[kTilesPerWg][2];
#pragma unroll
    for (int u = 0; u < kTilesPerWg; ++u) {
        int r0, c0;
        tile_origin(j, t0 + u, r0, c0);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int c = c0 + (t >> 3) + 32 * pass, r = r0 + 8 * (t & 7);
            const int64_t idx = (int64_t)c * j.ld + r;
            if (u >= ntiles || c >= j.len) in[u][pass] = u32x4{0u, 0u, 0u, 0u};
            else if (r + 8 <= j.rows) in[u][pass] = load8(j.src, idx);
            else in[u][pass] = load8_partial(j.src, idx, 1, j.rows - r);
        }
    }
#pragma unroll
    for (int u = 0; u < kTilesPerWg; ++u)
#pragma unroll
        for (int pass = 0; pass < 2; ++pass)
            *reinterpret_cast<u32x4*>(tiles + u * kPackTile * kPackTile + tile_at((t >> 3) + 32 * pass, 8 * (t & 7))) =
                in[u][pass];
    __syncthreads();
    // Store: output row r, 8 consecutive c per lane, gathered from 8 LDS rows.
#pragma unroll
    for (int u = 0; u < kTilesPerWg; ++u) {
        int r0, c0;
        tile_origin(j, t0 + u, r0, c0);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int rl = (t >> 3) + 32 * pass;
            const int cl = 8 * (t & 7);
            const int r = r0 + rl;
            if (u >= ntiles || r >= j.rows) continue;
            u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e >> 1] |= (uint32_t)tiles[u * kPackTile * kPackTile + tile_at(cl + e, rl)] << ((e & 1) * 16);
            *reinterpret_cast<u32x4*>(j.dst + (int64_t)r * j.len_pad + c0 + cl) = v;
        }
    }
}

__global__ __launch_bounds__(kPackThreads) void pack_kernel(PackParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t tiles[kTilesPerWg * kPackTile * kPackTile];
    int b = blockIdx.x;
    const int which = b < p.job[0].blocks ? 0 : 1;
    if (which) b -= p.job[0].blocks;
    const PackJob& j = p.job[which];
    const int t0 = b * kTilesPerWg;
    const int ntiles = min(kTilesPerWg, j.ntiles - t0);
    if (j.trans) pack_trans(j, t0, ntiles, tiles);
    else pack_rows(j, t0, ntiles);
}

}  // namespace

hipError_t launch_pack(PackParams p, hipStream_t st) {
    int64_t total = 0;
    for (int i = 0; i < 2; ++i) {
        PackJob& j = p.job[i];
        if (j.rows <= 0) { j.blocks = 0; j.ntiles = 0; j.tiles_c = 1; continue; }
        if (j.len_pad % kPackTile || j.len > j.len_pad) return hipErrorInvalidValue;
        j.tiles_c = j.len_pad / kPackTile;
        const int64_t ntiles = (int64_t)((j.rows + kPackTile - 1) / kPackTile) * j.tiles_c;
        const int64_t blocks = (ntiles + kTilesPerWg - 1) / kTilesPerWg;
        if (ntiles > INT32_MAX) return hipErrorInvalidValue;
        j.ntiles = (int)ntiles;
        j.blocks = (int)blocks;
        total += blocks;
    }
    if (total == 0) return hipSuccess;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)total), dim3(kPackThreads), 0, st, p);
    return hipGetLastError();
}

// Workspace of gemm_ws_static: the rewritten operands of a call that may not allocate go
// here.  Each GPU holds its own copy for the life of the process; every call on a GPU
// reuses it (the pack writes every byte a multiply then reads, zero padding included, so
// nothing needs clearing between calls).  In host code `scratch` names only a host-side
// stand-in: kernels get the device address that hipGetSymbolAddress returns.
static __device__ __align__(256) char scratch[kStaticWsBytes];

hipError_t static_workspace(void** ptr) {
    // one address per device, looked up with that device current the first time a call
    // needs it (atomics: concurrent first calls look it up twice and agree)
    static std::atomic<void*> addr[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace gemm
