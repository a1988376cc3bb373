// loaders.hpp -- global -> LDS slab loaders.
//
// Every kernel keeps, per ring slot, one LDS tile per operand made of LR "LDS rows" of
// ROWB bytes.  A 16-byte chunk c of LDS row r sits at chunk position c ^ swz(r) when
// the operand is swizzled (the swizzled shared-memory layout of section 5.2 of the
// multi-stage page, here as an XOR on 16-byte chunks so that the MFMA / FMA fragment
// reads of consecutive rows spread over all LDS banks).
//
//  * DirectLoader: buffer_load_dwordx4 ... lds -- each lane's 16 bytes go from HBM straight
//    into LDS without passing through registers (the role of the asynchronous copy of
//    "Matrix multiplication" and of cp.async in the other pages).  The LDS destination
//    of one wave instruction is 1 KiB contiguous, so the swizzle is produced by choosing
//    which global chunk each lane fetches.  Requires the global operand to be
//    contiguous along the LDS row, 16-byte aligned rows, and the whole tile in bounds.
//  * StagedLoader: ordinary loads into registers, then ds_write.  Handles any layout
//    (transposing when the global operand is contiguous across LDS rows), any
//    alignment (element loads when 16-byte vectors are not legal) and ragged edges
//    (out-of-range elements are written as zero, so they add +0 to every sum).
#pragma once

#include "common.hpp"

namespace gemm {

// Byte offset of element column `col` (in elements of size ES) of LDS row `r`.
template <int ROWB, int ES, bool SWZ>
__device__ __forceinline__ int lds_offset(int r, int col) {
    constexpr int CPR = ROWB / 16;
    const int byte = col * ES;
    const int chunk = byte >> 4;
    const int pc = SWZ ? (chunk ^ swz<CPR>(r)) : chunk;
    return r * ROWB + (pc << 4) + (byte & 15);
}

// Word 3 of a raw (stride 0) buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle, no index stride.
constexpr int kBufferFlags = 0x00020000;

// ------------------------------------------------------------------------------------
// LR rows of ROWB bytes, loaded by NW waves, IPW copies of 1 KiB per wave per slab.
//
// Wave w fills the contiguous band of LDS rows [w*IPW*RPI, (w+1)*IPW*RPI), copy i the
// i-th KiB of that band.  The LDS destination of a DMA copy is M0 + the instruction's
// immediate offset + 16*lane, and the same immediate is added to the global address;
// so GROUP consecutive copies share one M0 value and step through the band with
// immediates 0, 1 KiB, ...  (rewriting M0 between DMA copies stalls the issuing wave,
// and that wave is the one that feeds the matrix cores).
//
// The global address of lane l in copy i splits into a wave-uniform part -- the copy's
// first row times the row pitch, less its immediate -- passed as the scalar offset, and a
// per-lane part that depends only on the lane and on the swizzle phase of the copy's
// first row (NP phases), so a handful of lane-offset registers serve all copies.
template <int LR, int ROWB, int NW, bool SWZ, bool ASM = false>
struct DirectLoader {
    static constexpr int CPR = ROWB / 16;
    static constexpr int RPI = 64 / CPR;            // LDS rows per copy instruction
    static constexpr int IPW = LR / (RPI * NW);     // copies per wave per slab
    static constexpr int GROUP = 4;                 // copies per M0 value (immediates < 4 KiB)
    // swizzle phases of a copy's first row (the swizzle's period in the row index)
    static constexpr int PERIOD = swz_period<CPR>();
    static constexpr int NP = SWZ ? (RPI >= PERIOD ? 1 : PERIOD / RPI) : 1;
    static_assert(ROWB % 16 == 0 && CPR >= 1 && CPR <= 64 && 64 % CPR == 0, "row bytes");
    static_assert(IPW >= 1 && IPW * RPI * NW == LR, "rows must split evenly over the waves");
    static_assert(RPI * ROWB == 1024, "one copy fills 1 KiB of LDS");
    static_assert(IPW % NP == 0, "the phase of copy i must not depend on the wave");

    const char* base;      // uniform: address of LDS row 0, chunk 0 of slab 0
    int64_t slab_step;     // uniform: bytes between consecutive slabs
    uint32_t vpat[NP];     // per lane: row-in-copy * pitch + swizzled chunk, per phase
    uint32_t soff[IPW];    // uniform: first row of copy i * pitch - copy i's immediate
    int lds_wave;          // uniform: LDS byte offset of this wave's band

    // row_origin: global address of LDS row 0 / chunk 0 in slab 0; ld_bytes: bytes
    // between consecutive LDS rows in global memory (ld_bytes >= ROWB, and the host keeps
    // LR*ld_bytes < 2^31, so every offset fits 32 bits; copy i starts at row >= i*RPI,
    // so its scalar offset is never negative).
    // w: index of this wave among the NW loading waves (default: its index in the workgroup).
    __device__ __forceinline__ void init(const char* row_origin, int64_t ld_bytes, int64_t slab_bytes, int w = -1) {
        if (w < 0) w = wave_id();
        const int lane = lane_id();
        const int lr = lane / CPR;
        const int pc = lane % CPR;
        base = row_origin;
        slab_step = slab_bytes;
#pragma unroll
        for (int ph = 0; ph < NP; ++ph) {
            const int c = SWZ ? (pc ^ swz<CPR>(ph * RPI + lr)) : pc;
            vpat[ph] = (uint32_t)((int64_t)lr * ld_bytes + c * 16);
        }
#pragma unroll
        for (int i = 0; i < IPW; ++i)
            soff[i] = (uint32_t)((int64_t)((w * IPW + i) * RPI) * ld_bytes - (i % GROUP) * 1024);
        lds_wave = w * IPW * 1024;
    }
    // The copies are buffer loads with the LDS bit (a buffer resource based at the slab,
    // unbounded range): unlike the flat-encoded global form they do not count against the
    // LDS counter, so waits for fragment reads stay exact.
    template <int IMM>
    static __device__ __forceinline__ void copy(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t so, LDS_AS char* m0) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, m0, 16, voff, so, IMM, 0);
    }
    // Copies [i0, i1) of this wave's IPW copies of slab `slab` (compile-time range
    // after unrolling).
    __device__ __forceinline__ void issue(int slab, LDS_AS char* lds_tile, int i0, int i1) const {
        issue_at(base + (int64_t)slab * slab_step, lds_tile, i0, i1);
    }
    // Same, for the slab whose LDS row 0 / chunk 0 is at global address g (another tile's
    // slab in a persistent kernel; same row pitch).
    __device__ __forceinline__ void issue_at(const char* g, LDS_AS char* lds_tile, int i0, int i1) const {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)g, (short)0, -1, kBufferFlags);
#pragma unroll
        for (int i = 0; i < IPW; ++i)
            if (i >= i0 && i < i1) copy_one(i, g, rs, lds_tile);
    }
    // Copy i of a slab whose LDS row 0 / chunk 0 is at global address g (rs: the same as a
    // buffer resource).
    __device__ __forceinline__ void copy_one(int i, const char* g, __amdgpu_buffer_rsrc_t rs, LDS_AS char* lds_tile) const {
        LDS_AS char* m0 = lds_tile + lds_wave + (i / GROUP) * (GROUP * 1024);
        const uint32_t vo = vpat[i % NP];
        if constexpr (ASM) {
            const char* sa = g + soff[i];
            switch (i % GROUP) {
                case 0: copy_g<0>(sa, vo, m0); break;
                case 1: copy_g<1024>(sa, vo, m0); break;
                case 2: copy_g<2048>(sa, vo, m0); break;
                default: copy_g<3072>(sa, vo, m0); break;
            }
        } else {
            switch (i % GROUP) {
                case 0: copy<0>(rs, vo, soff[i], m0); break;
                case 1: copy<1024>(rs, vo, soff[i], m0); break;
                case 2: copy<2048>(rs, vo, soff[i], m0); break;
                default: copy<3072>(rs, vo, soff[i], m0); break;
            }
        }
    }
    // Copies [i0, i1) of slab `slab` when only its first `rows` LDS rows exist in global
    // memory (a partial last slab): lanes whose row lies beyond copy as usual (their
    // lanes of the instruction are switched off), the others write +0 into their 16 bytes
    // of LDS instead, so the slab's missing rows add nothing to any sum.  The zero writes
    // go through the LDS counter; the caller drains it before the barrier.
    __device__ __forceinline__ void issue_rows(int slab, LDS_AS char* lds_tile, int i0, int i1, int rows) const {
        const char* g = base + (int64_t)slab * slab_step;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)g, (short)0, -1, kBufferFlags);
        const int w = lds_wave / (IPW * 1024);
        const int lr = lane_id() / CPR;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            if (i >= i0 && i < i1) {
                if ((w * IPW + i) * RPI + lr < rows) {
                    copy_one(i, g, rs, lds_tile);
                } else {
                    LDS_AS char* m0 = lds_tile + lds_wave + (i / GROUP) * (GROUP * 1024);
                    *reinterpret_cast<LDS_AS u32x4*>(m0 + (i % GROUP) * 1024 + lane_id() * 16) = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    }
    // The global form of the same copy: LDS[M0 + IMM + 16*lane] = global[sa + voff + IMM],
    // 16 bytes per lane.  Written as inline asm so that the compiler neither waits on the LDS
    // counter for it nor moves other M0 users between the M0 write and the copy; completion
    // is tracked by the explicit vmcnt waits of the ring protocol.  One wait state after
    // the M0 write before the copy reads it.
    template <int IMM>
    static __device__ __forceinline__ void copy_g(const char* sa, uint32_t voff, LDS_AS char* m0) {
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3"
                     :: "v"(voff), "s"(sa), "s"((uint32_t)(uintptr_t)m0), "n"(IMM) : "m0");
    }
};

// ------------------------------------------------------------------------------------
// Register-staged loader.  LDS tile: LR rows x LC elements (ES bytes each), row pitch
// ROWB = LC*ES.  Global element (LDS row r, LDS col c) of slab s is at
//   aligned    (TRANS = false, contiguous along LDS cols): X[(r0 + r)*ld + c0 + c]
//   transposed (TRANS = true, contiguous along LDS rows):  X[(c0 + c)*ld + r0 + r]
// where slab s advances c0 by LC, or -- for an operand whose slabs advance along the LDS
// rows (`slab_rows`: the VALU B tile, LDS rows = k) -- r0 by LR.  Row indices are valid
// below r_lim, column indices below c_lim.
//
// Per slab the loader takes one of two paths, chosen uniformly for the workgroup:
// interior slabs use one 16-byte load per vector (unaligned when the operand's rows are
// not 16-byte aligned); edge slabs load whole vectors where they lie inside along the
// contiguous direction (lines beyond the edge read the last valid line and become +0)
// and element by element only where a vector straddles the end, an out-of-range
// element reading element 0 of the operand and being replaced by +0, so ragged edges
// and the K tail contribute exactly zero.
template <int LR, int LC, int ES, int NT, bool SWZ, bool TRANS>
struct StagedLoader {
    static constexpr int VE = 16 / ES;               // elements per 16-byte vector
    static constexpr int ROWB = LC * ES;
    // aligned mode: chunks of VE along an LDS row
    static constexpr int CH = LR * LC / VE / NT;     // vectors per thread per slab
    static_assert(CH >= 1 && CH * VE * NT == LR * LC, "slab must split evenly over the threads");
    // transposed mode: VE consecutive LDS rows x CHT consecutive LDS cols per thread
    static constexpr int G = LR / VE;
    static constexpr int CHT = LC * G / NT;
    static_assert(!TRANS || CHT == CH, "both modes move the same number of vectors");
    static_assert(!TRANS || (CHT * ES <= 16 && (16 % (CHT * ES)) == 0), "a transposed write must fit in one chunk");

    u32x4 v[CH];
    const char* X;
    int64_t ld;          // elements
    int r0, c0;          // tile origin (LDS row 0 / col 0 of slab 0), in the operand's index space
    int r_lim, c_lim;    // valid extents
    bool vec;            // 16-byte vectors are 16-byte aligned (else unaligned loads)
    bool slab_rows;      // slabs advance along LDS rows (else along LDS cols)

    __device__ __forceinline__ void init(const char* X_, int64_t ld_, int r0_, int c0_, int r_lim_, int c_lim_,
                                         bool vec_, bool slab_rows_) {
        X = X_; ld = ld_; r0 = r0_; c0 = c0_; r_lim = r_lim_; c_lim = c_lim_;
        vec = vec_; slab_rows = slab_rows_;
    }

    __device__ __forceinline__ uint32_t ld_elem(int64_t idx) const {
        if constexpr (ES == 4) return reinterpret_cast<const uint32_t*>(X)[idx];
        else return reinterpret_cast<const uint16_t*>(X)[idx];
    }

    // Thread's j-th vector: LDS row / col of its first element and the global index.
    __device__ __forceinline__ void coords(int j, int rs, int cs, int& gr, int& gc, int64_t& idx) const {
        const int tid = threadIdx.x;
        if constexpr (!TRANS) {
            const int q = tid + j * NT;
            gr = rs + q / (LC / VE);
            gc = cs + (q % (LC / VE)) * VE;
            idx = (int64_t)gr * ld + gc;
        } else {
            gr = rs + (tid % G) * VE;
            gc = cs + (tid / G) * CHT + j;
            idx = (int64_t)gc * ld + gr;
        }
    }

    // One 16-byte vector at element index idx: a plain vector load when the operand's
    // rows are 16-byte aligned, else an unaligned one (the target allows unaligned
    // global accesses; elements are always naturally aligned).
    __device__ __forceinline__ u32x4 ld_vec(int64_t idx) const {
        if (vec) return *reinterpret_cast<const u32x4*>(X + idx * ES);
        u32x4 t;
        __builtin_memcpy(&t, X + idx * ES, 16);
        return t;
    }

    __device__ __forceinline__ void load(int slab) {
        const int rs = slab_rows ? r0 + slab * LR : r0;
        const int cs = slab_rows ? c0 : c0 + slab * LC;
        const bool interior = rs + LR <= r_lim && cs + LC <= c_lim;
        if (interior) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                int gr, gc;
                int64_t idx;
                coords(j, rs, cs, gr, gc, idx);
                v[j] = ld_vec(idx);
            }
        } else {
            // Edge slab.  A vector whose elements all lie inside along the contiguous
            // direction is loaded whole, from the last valid line when its own line is
            // outside (then replaced by zeros); only vectors that straddle the end of
            // the contiguous direction (the K tail, a ragged N / M edge) go element by
            // element, reading element 0 for anything outside and selecting +0.
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                int gr, gc;
                int64_t idx;
                coords(j, rs, cs, gr, gc, idx);
                const bool whole = TRANS ? gr + VE <= r_lim : gc + VE <= c_lim;
                const bool line_ok = TRANS ? gc < c_lim : gr < r_lim;
                u32x4 t = {0u, 0u, 0u, 0u};
                if (whole) {
                    const int64_t cidx = TRANS ? (int64_t)(line_ok ? gc : c_lim - 1) * ld + gr
                                               : (int64_t)(line_ok ? gr : r_lim - 1) * ld + gc;
                    const u32x4 x = ld_vec(cidx);
                    if (line_ok) t = x;
                } else {
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        const bool ok = TRANS ? (gc < c_lim && gr + e < r_lim) : (gr < r_lim && gc + e < c_lim);
                        uint32_t x = ld_elem(ok ? idx + e : 0);
                        x = ok ? x : 0u;
                        if constexpr (ES == 4) t[e] = x;
                        else t[e >> 1] |= x << ((e & 1) * 16);
                    }
                }
                v[j] = t;
            }
        }
    }

    __device__ __forceinline__ uint32_t elem(int j, int e) const {
        if constexpr (ES == 4) return v[j][e];
        else return (v[j][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
    }

    __device__ __forceinline__ void write(LDS_AS char* lds_tile) const {
        const int tid = threadIdx.x;
        if constexpr (!TRANS) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int q = tid + j * NT;
                const int r = q / (LC / VE);
                const int c = (q % (LC / VE)) * VE;
                *reinterpret_cast<LDS_AS u32x4*>(lds_tile + lds_offset<ROWB, ES, SWZ>(r, c)) = v[j];
            }
        } else {
            const int grp = tid % G;
            const int cb = (tid / G) * CHT;
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                const int r = grp * VE + e;
                LDS_AS char* dst = lds_tile + lds_offset<ROWB, ES, SWZ>(r, cb);
                if constexpr (CHT * ES == 16) {
                    u32x4 w;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if constexpr (ES == 4) w[q] = elem(q, e);
                        else w[q] = elem(2 * q, e) | (elem(2 * q + 1, e) << 16);
                    }
                    *reinterpret_cast<LDS_AS u32x4*>(dst) = w;
                } else if constexpr (CHT * ES == 8) {
                    u32x2 w;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        if constexpr (ES == 4) w[q] = elem(q, e);
                        else w[q] = elem(2 * q, e) | (elem(2 * q + 1, e) << 16);
                    }
                    *reinterpret_cast<LDS_AS u32x2*>(dst) = w;
                } else if constexpr (CHT * ES == 4) {
                    uint32_t w;
                    if constexpr (ES == 4) w = elem(0, e);
                    else w = elem(0, e) | (elem(1, e) << 16);
                    *reinterpret_cast<LDS_AS uint32_t*>(dst) = w;
                } else {
                    *reinterpret_cast<LDS_AS uint16_t*>(dst) = (uint16_t)elem(0, e);
                }
            }
        }
    }
};

// ------------------------------------------------------------------------------------
// Register-staged loader for a K-contiguous 16-bit operand of any alignment: LR rows of LC
// k per slab, each thread moving CH 16-byte vectors.  Every vector is one buffer load of
// 16 bytes at the element's own (2- or 4-byte aligned) offset, which the hardware serves
// whole (checked on the GPU), with no branch on alignment or position: the loads of one
// slab never wait for those of the previous one, and they leave the issuing wave at once.
// The buffer range ends at the operand's last element, so nothing beyond it is read (a
// dword that crosses that end comes back as zero: the last element of each row is loaded
// again on its own for the partial last slab, and put back).  In the partial last slab the
// columns beyond K are cleared in registers before the write, so they add +0 to every sum.
template <int LR, int LC, int NT>
struct RowLoader {
    static constexpr int VE = 8;              // 16-bit elements per vector
    static constexpr int VPR = LC / VE;       // vectors per row
    static constexpr int CH = LR * VPR / NT;  // vectors per thread per slab
    static constexpr int ROWB = LC * 2;       // bytes per LDS row
    static_assert(CH >= 1 && CH * NT == LR * VPR, "slab must split evenly over the threads");
    u32x4 v[CH];
    uint32_t last[CH];    // partial slab: element K-1 of each vector's row
    const char* base;     // row 0, column 0 of the tile (slab 0)
    int64_t ld;           // elements
    int K;                // columns that exist
    int64_t end;          // bytes from `base` to the end of the operand's last element

    // X: the operand; rows r0 .. r0+LR-1 of its M rows are this tile's (r0 + LR <= M).
    __device__ __forceinline__ void init(const char* X, int64_t ld_, int r0, int K_, int M) {
        base = X + (int64_t)r0 * ld_ * 2;
        ld = ld_;
        K = K_;
        end = ((int64_t)(M - 1 - r0) * ld_ + K_) * 2;
    }
    __device__ __forceinline__ void coords(int j, int& r, int& c) const {
        const int q = (int)threadIdx.x + j * NT;
        r = q / VPR;
        c = (q % VPR) * VE;
    }
    // Issue the loads of slab `slab` (partial: the slab holds column K-1 and ends past it).
    __device__ __forceinline__ void load(int slab, bool partial) {
        const int64_t s0 = (int64_t)slab * ROWB;
        const int64_t left = end - s0;
        const uint32_t nrec = left > 0x7fffffff ? 0x7fffffffu : (uint32_t)left;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(base + s0), (short)0, (int)nrec, kBufferFlags);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            int r, c;
            coords(j, r, c);
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(((int64_t)r * ld + c) * 2), 0, 0);
        }
        if (partial) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                int r, c;
                coords(j, r, c);
                last[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, (uint32_t)(((int64_t)r * ld + (K - 1) - slab * LC) * 2), 0, 0);
            }
        }
    }
    // Write the registers of slab `slab` into an LDS tile ([row][k], rows of ROWB bytes,
    // 16-byte chunks swizzled by swz<ROWB / 16>); the loads must have completed.
    __device__ __forceinline__ void write(LDS_AS char* lds_tile, int slab, bool partial) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            int r, c;
            coords(j, r, c);
            u32x4 x = v[j];
            if (partial) {
                const int k0 = slab * LC + c;       // column of element 0
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const uint32_t sh = (e & 1) * 16;
                    uint32_t w = x[e >> 1];
                    if (k0 + e == K - 1) w = (w & ~(0xffffu << sh)) | ((last[j] & 0xffffu) << sh);
                    else if (k0 + e >= K) w &= ~(0xffffu << sh);
                    x[e >> 1] = w;
                }
            }
            *reinterpret_cast<LDS_AS u32x4*>(lds_tile + lds_offset<ROWB, 2, true>(r, c)) = x;
        }
    }
};

}  // namespace gemm
