// common.hpp -- device helpers shared by the GEMM kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "schedule.hpp"

namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// Arguments every kernel receives (by value, in the kernarg segment).
struct GemmParams {
    const char* A;
    const char* B;
    char* C;
    int64_t lda, ldb, ldc;  // elements
    int M, N, K;
    float alpha, beta;
    int a_col, b_col;       // 1 = column-major operand (staged kernels read this at run time)
    int out_type;           // DT_* of C
    int tiles_m, tiles_n;   // C tiles along M and N
    int group_m;            // tile rows per rasterisation group
    int xcd_remap;          // 1 = spread consecutive tiles onto one XCD
    int a_vec, b_vec;       // staged kernels: 16-byte vector loads are legal for A / B
    int lds_pad;            // host only: extra dynamic LDS bytes per workgroup (equal-occupancy runs)
    int poison;             // host only: 1 = launch the LDS-poisoning debug variant of the kernel
};

// ---------------------------------------------------------------- waits and barriers
// s_waitcnt immediate for the gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14].
__device__ __forceinline__ constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 15));
}
// All of this wave's LDS reads and writes have completed (also a compiler barrier for
// memory, so that no LDS access is moved across it).
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Workgroup barrier that keeps outstanding global->LDS copies of the ring in flight (a
// __syncthreads() fence would wait for all of them).  The asm statement clobbers
// "memory" so that the compiler moves no LDS access across it; the hardware ordering
// (this wave's own LDS / copy traffic completed) is the explicit s_waitcnt before it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Debugging wrapper of a ring kernel's K-loop operations.  Right after the barrier that
// releases a ring slot (every wave has finished reading the slab in it; nothing has been
// copied into it yet) each thread of the workgroup overwrites its share of the slot with
// all-ones bits -- NaN as bf16, f16 and fp32 -- waits for its writes, and meets the others
// at a second barrier before anything can be issued into the slot.  A fragment read of a
// released slot, or one that runs ahead of the copy it should wait for, then reads NaN
// instead of a stale slab, and the result shows it whatever the inputs (all-ones or
// identity operands included).  The protocol calls release() through the K-loop template's
// hook; kernels built without this wrapper contain no trace of it.
template <class Base>
struct PoisonOps : Base {
    __device__ __forceinline__ void release(int slot) {
        LDS_AS char* st = this->smem + slot * Base::STAGE;
        for (int i = (int)threadIdx.x * 16; i < Base::STAGE; i += (int)blockDim.x * 16)
            *reinterpret_cast<LDS_AS u32x4*>(st + i) = u32x4{~0u, ~0u, ~0u, ~0u};
        wait_lgkm0();
        barrier();
    }
};
template <bool POISON, class O>
using MaybePoison = typename std::conditional<POISON, PoisonOps<O>, O>::type;

// Waves per SIMD that the LDS footprint allows (4 SIMDs per CU, 160 KiB of LDS),
// clamped to [1, cap]; used as the kernels' amdgpu_waves_per_eu so that the compiler
// budgets registers for the occupancy the ring actually permits.
constexpr int occupancy_waves(int threads, int lds_bytes, int cap) {
    const int wg = lds_bytes > 0 ? 163840 / lds_bytes : 32;
    const int need = (threads + 255) / 256;  // one workgroup alone puts this many waves on a SIMD
    int w = wg * (threads / 64) / 4;
    if (w > cap) w = cap;
    if (w < need) w = need;
    if (w < 1) w = 1;
    return w;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------- LDS swizzle
// 16-byte chunk c of LDS row r lives at chunk position c ^ swz(r).  For CPR = 8
// (128-byte rows) and CPR = 4 (64-byte rows) the functions make any 8 or 16 consecutive
// rows read at one logical chunk hit distinct banks, for both 128- and 256-byte LDS
// phases; both have period 16 in r.  CPR = 32 (512-byte rows: a [k][n] tile of 256
// 16-bit columns) serves the transposing fragment reads, each of which takes two
// neighbouring chunks from each of four consecutive rows per 16 lanes: the XOR values
// 0, 4, 10, 14 for r mod 4 = 0..3 put those 4 x 2 chunks (and the next 16 lanes' 4 x 2
// chunks, two chunks further on) on distinct banks in both 128- and 256-byte phases;
// period 4 in r.  Other CPR: no swizzle.
template <int CPR>
__host__ __device__ __forceinline__ constexpr int swz(int r) {
    if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
    else if constexpr (CPR == 4) return ((r >> 1) ^ (r >> 2)) & 3;
    else if constexpr (CPR == 32) return (4 * (r & 3)) ^ (r & 2);
    else return 0;
}
// Row period of swz<CPR> (the swizzle phases a loader must tell apart).
template <int CPR>
__host__ __device__ __forceinline__ constexpr int swz_period() {
    return CPR == 32 ? 4 : 16;
}

// ---------------------------------------------------------------- tile order
// Workgroup id -> (tile_m, tile_n).  Workgroups are dispatched round-robin over the 8
// XCDs, each with its own L2; the remap gives each XCD a contiguous run of the grouped
// order so that the tiles resident on one XCD share A row-panels and B column-panels.
// wg: the workgroup index (a persistent workgroup passes the index of the tile slot it
// is working on: its own id plus a multiple of the grid size, a multiple of 8, so the
// slot stays on the workgroup's XCD).
__device__ __forceinline__ void tile_coords_of(const GemmParams& p, int wg, int& tm, int& tn) {
    const int total = p.tiles_m * p.tiles_n;
    if (p.xcd_remap && (total & 7) == 0) wg = (wg & 7) * (total >> 3) + (wg >> 3);
    const int per_group = p.group_m * p.tiles_n;
    const int g = wg / per_group;
    const int first_m = g * p.group_m;
    const int gsize = min(p.tiles_m - first_m, p.group_m);
    const int r = wg - g * per_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}
__device__ __forceinline__ void tile_coords(const GemmParams& p, int& tm, int& tn) {
    tile_coords_of(p, blockIdx.x, tm, tn);
}

// ---------------------------------------------------------------- epilogue helpers
// out = alpha*acc (beta == 0: C not read) or fmaf(alpha, acc, beta*c).
__device__ __forceinline__ float epi(float acc, float alpha, float beta, float c) {
    return beta == 0.0f ? alpha * acc : __builtin_fmaf(alpha, acc, beta * c);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    _Float16 h = (_Float16)x;  // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Old values of 4 consecutive C elements (row-major, column n..n+3) as fp32, for an
// epilogue with beta != 0; elements outside [lo, N) are not read (0).  Kept separate from
// the store so that an epilogue can issue the loads of several quads before any store:
// a load cannot be moved above a store to C that might alias it.
template <int OUT>
__device__ __forceinline__ f32x4 load_c4(const GemmParams& p, int64_t m, int n, int lo) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    const bool full = n >= lo && n + 3 < p.N;
    if constexpr (OUT == DT_F32) {
        const float* c = reinterpret_cast<const float*>(p.C) + m * p.ldc + n;
        if (full && (reinterpret_cast<uintptr_t>(c) & 15) == 0) {
            o = *reinterpret_cast<const f32x4*>(c);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n + j >= lo && n + j < p.N) o[j] = c[j];
        }
    } else {
        constexpr bool bf = OUT == DT_BF16;
        const uint16_t* c = reinterpret_cast<const uint16_t*>(p.C) + m * p.ldc + n;
        if (full && (reinterpret_cast<uintptr_t>(c) & 7) == 0) {
            const u32x2 w = *reinterpret_cast<const u32x2*>(c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint16_t b = (uint16_t)(w[j >> 1] >> ((j & 1) * 16));
                o[j] = bf ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n + j >= lo && n + j < p.N) o[j] = bf ? bf16_bits_to_f32(c[j]) : f16_bits_to_f32(c[j]);
        }
    }
    return o;
}

// Store out = epi(v, old) for 4 consecutive C elements (columns n..n+3 within [lo, N));
// `old` holds the values load_c4 read (ignored when beta == 0).
template <int OUT>
__device__ __forceinline__ void store_c4(const GemmParams& p, int64_t m, int n, f32x4 v, f32x4 old, int lo) {
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = epi(v[j], p.alpha, p.beta, old[j]);
    const bool full = n >= lo && n + 3 < p.N;
    if constexpr (OUT == DT_F32) {
        float* c = reinterpret_cast<float*>(p.C) + m * p.ldc + n;
        if (full && (reinterpret_cast<uintptr_t>(c) & 15) == 0) {
            *reinterpret_cast<f32x4*>(c) = r;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n + j >= lo && n + j < p.N) c[j] = r[j];
        }
    } else {
        constexpr bool bf = OUT == DT_BF16;
        uint16_t* c = reinterpret_cast<uint16_t*>(p.C) + m * p.ldc + n;
        uint16_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = bf ? f32_to_bf16_bits(r[j]) : f32_to_f16_bits(r[j]);
        if (full && (reinterpret_cast<uintptr_t>(c) & 7) == 0) {
            u32x2 pk;
            pk[0] = (uint32_t)w[0] | ((uint32_t)w[1] << 16);
            pk[1] = (uint32_t)w[2] | ((uint32_t)w[3] << 16);
            *reinterpret_cast<u32x2*>(c) = pk;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n + j >= lo && n + j < p.N) c[j] = w[j];
        }
    }
}

// C rows start on the boundary a whole quad needs (16 bytes for fp32, 8 for 16-bit), so
// any quad at a column multiple of 4 can move as one vector.
template <int OUT>
__device__ __forceinline__ bool c_quads_aligned(const GemmParams& p) {
    constexpr int QB = OUT == DT_F32 ? 16 : 8;
    return (reinterpret_cast<uintptr_t>(p.C) % QB) == 0 && (p.ldc * (OUT == DT_F32 ? 4 : 2)) % QB == 0;
}

// Unpredicated forms for quads known to lie inside C, at a column multiple of 4, with
// c_quads_aligned(p).
template <int OUT>
__device__ __forceinline__ f32x4 load_c4_vec(const GemmParams& p, int64_t m, int n) {
    if constexpr (OUT == DT_F32) {
        return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.C) + m * p.ldc + n);
    } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(p.C) + m * p.ldc + n);
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint16_t b = (uint16_t)(w[j >> 1] >> ((j & 1) * 16));
            o[j] = OUT == DT_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
        }
        return o;
    }
}
template <int OUT>
__device__ __forceinline__ void store_c4_vec(const GemmParams& p, int64_t m, int n, f32x4 v, f32x4 old) {
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = epi(v[j], p.alpha, p.beta, old[j]);
    if constexpr (OUT == DT_F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C) + m * p.ldc + n) = r;
    } else {
        uint16_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = OUT == DT_BF16 ? f32_to_bf16_bits(r[j]) : f32_to_f16_bits(r[j]);
        u32x2 pk;
        pk[0] = (uint32_t)w[0] | ((uint32_t)w[1] << 16);
        pk[1] = (uint32_t)w[2] | ((uint32_t)w[3] << 16);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.C) + m * p.ldc + n) = pk;
    }
}

// Store 4 consecutive C elements (row-major, column n..n+3) of type OUT, with a
// per-element column predicate when the quad straddles N or the first column `lo` this
// tile owns (an edge tile shifted inward starts at a column that need not be a multiple
// of 4).  Reads C when beta != 0.
template <int OUT>
__device__ __forceinline__ void store4(const GemmParams& p, int64_t m, int n, f32x4 v, int lo = 0) {
    const bool full = n >= lo && n + 3 < p.N;
    if constexpr (OUT == DT_F32) {
        float* c = reinterpret_cast<float*>(p.C) + m * p.ldc + n;
        const bool vec = full && ((reinterpret_cast<uintptr_t>(c) & 15) == 0);
        if (vec) {
            f32x4 old = {0.f, 0.f, 0.f, 0.f};
            if (p.beta != 0.0f) old = *reinterpret_cast<const f32x4*>(c);
            f32x4 r;
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] = epi(v[j], p.alpha, p.beta, old[j]);
            *reinterpret_cast<f32x4*>(c) = r;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n + j >= lo && n + j < p.N) c[j] = epi(v[j], p.alpha, p.beta, p.beta != 0.0f ? c[j] : 0.0f);
        }
    } else {
        constexpr bool bf = OUT == DT_BF16;
        uint16_t* c = reinterpret_cast<uint16_t*>(p.C) + m * p.ldc + n;
        const bool vec = full && ((reinterpret_cast<uintptr_t>(c) & 7) == 0);
        if (vec) {
            u32x2 old = {0u, 0u};
            if (p.beta != 0.0f) old = *reinterpret_cast<const u32x2*>(c);
            uint16_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint16_t ob = (uint16_t)(old[j >> 1] >> ((j & 1) * 16));
                const float o = bf ? bf16_bits_to_f32(ob) : f16_bits_to_f32(ob);
                const float r = epi(v[j], p.alpha, p.beta, o);
                w[j] = bf ? f32_to_bf16_bits(r) : f32_to_f16_bits(r);
            }
            u32x2 pk;
            pk[0] = (uint32_t)w[0] | ((uint32_t)w[1] << 16);
            pk[1] = (uint32_t)w[2] | ((uint32_t)w[3] << 16);
            *reinterpret_cast<u32x2*>(c) = pk;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (n + j >= lo && n + j < p.N) {
                    float o = 0.0f;
                    if (p.beta != 0.0f) o = bf ? bf16_bits_to_f32(c[j]) : f16_bits_to_f32(c[j]);
                    const float r = epi(v[j], p.alpha, p.beta, o);
                    c[j] = bf ? f32_to_bf16_bits(r) : f32_to_f16_bits(r);
                }
            }
        }
    }
}

}  // namespace gemm
