// kernels_valu.hip -- fp32 GEMM on the vector ALUs, register-blocked.
//
// Thread tile (section 4, "Thread Tile", of "CUTLASS-Cute 初步(6)：CUDA GEMM 计算优化、
// Multi-Stage 与软流水"): every thread owns TM x TN accumulators and, per k, forms the
// outer product of TM values of A and TN values of B held in registers, so each value
// read from LDS feeds TN (or TM) fused multiply-adds.  The fragments of the next pair of
// k are read from LDS while the current pair is multiplied (warp-scope register double
// buffering of "Matrix multiplication" / section 6 of the multi-stage page).
//
// Every accumulator is ONE fp32 fma chain in ascending k starting from +0, whatever the
// tile, the stage count, the k-step width or the loader: results are bit-identical
// across variants and equal to a sequential fmaf() loop.
//
// A k-step covers KW = 4 consecutive k: each lane reads its A rows as whole 16-byte
// chunks (4 k), which the chunk swizzle spreads over distinct banks for any 8
// consecutive rows.  With KW = 2 (8-byte halves of a chunk) the 16 rows a wave reads
// share half the banks, a two-way conflict on every A read (kept as a tile for the
// comparison).
//
// LDS tiles per ring slot: A as [BM rows = m][BK floats = k] (XOR-swizzled 16-byte
// chunks), B as [BK rows = k][BN floats = n].
//
// Thread (tr, tc), tr = tid mod (BM/TM), tc = tid / (BM/TM):
//   rows    m = tr + (BM/TM)*i,                 i < TM
//   columns n = 4*tc + 4*(BN/TN)*h + j,         h < TN/4, j < 4
// so the lanes of a wave read consecutive rows (conflict-free through the swizzle) and
// consecutive 16-byte column groups of B.
#include <type_traits>

#include "common.hpp"
#include "loaders.hpp"
#include "launch.hpp"

namespace gemm {

template <int BM, int BN, int BK, int TM, int TN, int KW = 4>
struct ValuCompute {
    static constexpr int TGM = BM / TM;  // thread rows
    static constexpr int TGN = BN / TN;  // thread cols
    static constexpr int NT = TGM * TGN;
    static constexpr int KS = BK / KW;   // k-steps (KW k each) per slab
    static constexpr int CH = BK / 4;    // 16-byte chunks per A row
    static_assert(KW == 2 || KW == 4, "k-step of 2 or 4 k");
    static constexpr int A_ROWB = BK * 4;
    static constexpr int B_ROWB = BN * 4;
    static constexpr int A_BYTES = BM * A_ROWB;
    static constexpr int B_BYTES = BK * B_ROWB;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_CPR = A_ROWB / 16;
    static_assert(TN % 4 == 0 && BK % 4 == 0, "column quads and an even number of k-steps");
    static_assert(NT % 64 == 0, "whole waves");

    // Rows of one thread are tr + TGM*i; the XOR swizzle has period 16 in the row, so
    // they fall into NQ = 16/gcd(16, TGM) swizzle classes (i mod NQ).
    static constexpr int NQ = (TGM % 16 == 0) ? 1 : (TGM % 8 == 0 ? 2 : (TGM % 4 == 0 ? 4 : 16));
    static_assert(TM % NQ == 0 || NQ == 1, "rows per thread must cover the swizzle classes evenly");

    typedef typename std::conditional<KW == 4, f32x4, f32x2>::type fa_t;
    float acc[TM][TN];
    fa_t fa[2][TM];           // fa[buf][i] = A[m_i][KW*ks .. KW*ks + KW)
    f32x4 fb[2][KW][TN / 4];  // fb[buf][kk][h] = B[KW*ks + kk][n_h .. n_h+3]
    uint32_t a_addr[NQ][CH];  // LDS byte offset of (row tr + TGM*q, 16-byte chunk c)
    uint32_t b_col;               // LDS byte offset of column 4*tc of B row 0
    LDS_AS char* smem;

    __device__ __forceinline__ void init(LDS_AS char* smem_) {
        smem = smem_;
        const int tid = threadIdx.x;
        const int tr = tid % TGM, tc = tid / TGM;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int m = tr + TGM * q;
                a_addr[q][c] = (uint32_t)(m * A_ROWB + ((c ^ swz<A_CPR>(m)) << 4));
            }
        b_col = (uint32_t)(A_BYTES + tc * 16);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;
    }

    template <int BUF>
    __device__ __forceinline__ void frag(int slot, int ks) {
        LDS_AS const char* st = smem + slot * STAGE;
        // k = KW*ks .. KW*ks + KW - 1 sit in 16-byte chunk (KW*ks)/4 of the A row, at byte
        // 4*(KW*ks mod 4); row tr + TGM*i = (row tr + TGM*(i mod NQ)) + TGM*NQ*(i / NQ)
        // rows, whose swizzle is the same (TGM*NQ is a multiple of 16).
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[BUF][i] = *reinterpret_cast<LDS_AS const fa_t*>(
                st + a_addr[i % NQ][(KW * ks) / 4] + ((KW * ks) % 4) * 4 + (i / NQ) * (TGM * NQ * A_ROWB));
#pragma unroll
        for (int kk = 0; kk < KW; ++kk)
#pragma unroll
            for (int h = 0; h < TN / 4; ++h)
                fb[BUF][kk][h] = *reinterpret_cast<LDS_AS const f32x4*>(
                    st + b_col + (KW * ks + kk) * B_ROWB + h * (TGN * 16));
    }

    template <int BUF>
    __device__ __forceinline__ void math() {
#pragma unroll
        for (int kk = 0; kk < KW; ++kk)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int h = 0; h < TN / 4; ++h)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][4 * h + j] = __builtin_fmaf(fa[BUF][i][kk], fb[BUF][kk][h][j], acc[i][4 * h + j]);
        // keep the k-step structure: the fragment loads issued before this math stay
        // ahead of it and the next k-step's loads are not hoisted above it
        __builtin_amdgcn_sched_barrier(0);
    }

    __device__ __forceinline__ void epilogue(const GemmParams& p, int m0, int n0, int m_keep, int n_keep) {
        const int tid = threadIdx.x;
        const int tr = tid % TGM, tc = tid / TGM;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + tr + TGM * i;
            if (m < m_keep || m >= p.M) continue;
#pragma unroll
            for (int h = 0; h < TN / 4; ++h) {
                const int n = n0 + 4 * tc + 4 * TGN * h;
                if (n + 3 < n_keep || n >= p.N) continue;
                f32x4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = acc[i][4 * h + j];
                store4<DT_F32>(p, m, n, v, n_keep);
            }
        }
    }
};

// ---------------------------------------------------------------- direct ring kernel
template <int BM, int BN, int BK, int TM, int TN, int S, int KW>
struct ValuRingOps : ValuCompute<BM, BN, BK, TM, TN, KW> {
    typedef ValuCompute<BM, BN, BK, TM, TN, KW> C;
    static constexpr int NW = C::NT / 64;
    typedef DirectLoader<BM, C::A_ROWB, NW, true> LA;    // rows m, k along the row
    typedef DirectLoader<BK, C::B_ROWB, NW, false> LB;   // rows k, n along the row
    static constexpr int L = LA::IPW + LB::IPW;
    LA la;
    LB lb;

    // Part `part` of `parts` of the copy of slab `slab` into ring slot `slot`: the L
    // copies of this wave (A's first, then B's) are split into equal consecutive runs.
    __device__ __forceinline__ void issue(int slab, int slot, int part, int parts) {
        LDS_AS char* st = this->smem + slot * C::STAGE;
        const int c0 = part * L / parts, c1 = (part + 1) * L / parts;
        constexpr int LA_N = decltype(la)::IPW;
        la.issue(slab, st, c0, c1 < LA_N ? c1 : LA_N);
        lb.issue(slab, st + C::A_BYTES, c0 > LA_N ? c0 - LA_N : 0, c1 - LA_N);
    }
    template <int N>
    __device__ __forceinline__ void wait_slabs() { wait_vm<N * L>(); }
    __device__ __forceinline__ void wait_lds() { wait_lgkm0(); }
    __device__ __forceinline__ void barrier() { gemm::barrier(); }
    template <int BUF>
    __device__ __forceinline__ void frag(int, int slot, int ks) { C::template frag<BUF>(slot, ks); }
    template <int BUF, int HAS, int PARTS>
    __device__ __forceinline__ void math(int) { C::template math<BUF>(); }
};

template <int BM, int BN, int BK, int TM, int TN, int S, int KW, bool POISON>
__global__ __launch_bounds__((BM / TM) * (BN / TN)) __attribute__((amdgpu_waves_per_eu(
    occupancy_waves((BM / TM) * (BN / TN), S * ValuCompute<BM, BN, BK, TM, TN>::STAGE,
                    TM * TN >= 64 ? (KW == 4 ? 2 : 3) : (TM * TN >= 32 ? 3 : 4)))))
void valu_ring_kernel(const GemmParams p) {
    typedef MaybePoison<POISON, ValuRingOps<BM, BN, BK, TM, TN, S, KW>> Ops;
    __shared__ __attribute__((aligned(1024))) char smem_raw[S * Ops::STAGE];
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m_keep = tm * BM, n_keep = tn * BN;
    const int m0 = min(m_keep, p.M - BM);
    const int n0 = min(n_keep, p.N - BN);
    Ops ops;
    ops.init((LDS_AS char*)(smem_raw));
    // A row-major: LDS row m <- A[m][k0 .. k0+BK); B row-major: LDS row k <- B[k][n0 .. n0+BN).
    ops.la.init(p.A + (int64_t)m0 * p.lda * 4, p.lda * 4, BK * 4);
    ops.lb.init(p.B + (int64_t)n0 * 4, p.ldb * 4, (int64_t)BK * p.ldb * 4);
    gemm_sched::ring_mainloop<S, Ops::KS, 0>(ops, p.K / BK);
    ops.epilogue(p, m0, n0, m_keep, n_keep);
}

// ---------------------------------------------------------------- staged kernel
// AT: A column-major (contiguous across its LDS rows m); BT: B column-major (contiguous
// across its LDS rows k).  Such operands are transposed on their way into LDS.
template <int BM, int BN, int BK, int TM, int TN, int S, bool AT, bool BT>
struct ValuStagedOps : ValuCompute<BM, BN, BK, TM, TN, 2> {  // 2-k steps: the staged loads hold registers too
    typedef ValuCompute<BM, BN, BK, TM, TN, 2> C;
    StagedLoader<BM, BK, 4, C::NT, true, AT> la;    // LDS rows m, cols k
    StagedLoader<BK, BN, 4, C::NT, false, BT> lb;   // LDS rows k, cols n

    __device__ __forceinline__ void load(int slab) {
        la.load(slab);
        lb.load(slab);
    }
    __device__ __forceinline__ void write(int, int slot) {
        LDS_AS char* st = this->smem + slot * C::STAGE;
        la.write(st);
        lb.write(st + C::A_BYTES);
    }
    __device__ __forceinline__ void wait_lds() { wait_lgkm0(); }
    __device__ __forceinline__ void barrier() { gemm::barrier(); }
    template <int BUF>
    __device__ __forceinline__ void frag(int, int slot, int ks) { C::template frag<BUF>(slot, ks); }
    template <int BUF, int HAS, int PARTS>
    __device__ __forceinline__ void math(int) { C::template math<BUF>(); }
};

template <int BM, int BN, int BK, int TM, int TN, int S, bool AT, bool BT>
__global__ __launch_bounds__((BM / TM) * (BN / TN)) __attribute__((amdgpu_waves_per_eu(
    occupancy_waves((BM / TM) * (BN / TN), S * ValuCompute<BM, BN, BK, TM, TN>::STAGE, TM * TN >= 64 ? 2 : 4))))
void valu_staged_kernel(const GemmParams p) {
    typedef ValuStagedOps<BM, BN, BK, TM, TN, S, AT, BT> Ops;
    __shared__ __attribute__((aligned(1024))) char smem_raw[S * Ops::STAGE];
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    Ops ops;
    ops.init((LDS_AS char*)(smem_raw));
    // A: LDS rows m, cols k.  B: LDS rows k, cols n; its slabs advance along the LDS rows.
    ops.la.init(p.A, p.lda, m0, 0, p.M, p.K, p.a_vec != 0, false);
    ops.lb.init(p.B, p.ldb, 0, n0, p.K, p.N, p.b_vec != 0, true);
    gemm_sched::staged_mainloop<S, Ops::KS>(ops, (p.K + BK - 1) / BK);
    ops.epilogue(p, m0, n0, m0, n0);
}

// ---------------------------------------------------------------- launch tables
template <int BM, int BN, int BK, int TM, int TN, int S, int KW>
static hipError_t launch_ring(const GemmParams& p, hipStream_t st) {
    hipLaunchKernelGGL((valu_ring_kernel<BM, BN, BK, TM, TN, S, KW, false>), dim3(p.tiles_m * p.tiles_n),
                       dim3((BM / TM) * (BN / TN)), p.lds_pad, st, p);
    return hipGetLastError();
}
// The LDS-poisoning debug variant (built for the default fp32 tile only).
template <int BM, int BN, int BK, int TM, int TN, int S, int KW>
static hipError_t launch_ring_poison(const GemmParams& p, hipStream_t st) {
    hipLaunchKernelGGL((valu_ring_kernel<BM, BN, BK, TM, TN, S, KW, true>), dim3(p.tiles_m * p.tiles_n),
                       dim3((BM / TM) * (BN / TN)), p.lds_pad, st, p);
    return hipGetLastError();
}
template <int BM, int BN, int BK, int TM, int TN, int S>
static hipError_t launch_staged(const GemmParams& p, hipStream_t st) {
    const dim3 grid(p.tiles_m * p.tiles_n), block((BM / TM) * (BN / TN));
    const bool at = p.a_col != 0, bt = p.b_col != 0;
    if (!at && !bt) hipLaunchKernelGGL((valu_staged_kernel<BM, BN, BK, TM, TN, S, false, false>), grid, block, p.lds_pad, st, p);
    else if (!at && bt) hipLaunchKernelGGL((valu_staged_kernel<BM, BN, BK, TM, TN, S, false, true>), grid, block, p.lds_pad, st, p);
    else if (at && !bt) hipLaunchKernelGGL((valu_staged_kernel<BM, BN, BK, TM, TN, S, true, false>), grid, block, p.lds_pad, st, p);
    else hipLaunchKernelGGL((valu_staged_kernel<BM, BN, BK, TM, TN, S, true, true>), grid, block, p.lds_pad, st, p);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int TM, int TN, int KW = 4>
static hipError_t ring_stages(int S, const GemmParams& p, hipStream_t st) {
    switch (S) {
        case 1: return launch_ring<BM, BN, BK, TM, TN, 1, KW>(p, st);
        case 2: return launch_ring<BM, BN, BK, TM, TN, 2, KW>(p, st);
        case 3: return launch_ring<BM, BN, BK, TM, TN, 3, KW>(p, st);
        case 4: return launch_ring<BM, BN, BK, TM, TN, 4, KW>(p, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_valu_ring(int tile, int nstage, const GemmParams& p, hipStream_t st) {
    if (p.poison && tile == 5) {
        switch (nstage) {
            case 1: return launch_ring_poison<128, 64, 16, 8, 4, 1, 4>(p, st);
            case 2: return launch_ring_poison<128, 64, 16, 8, 4, 2, 4>(p, st);
            case 3: return launch_ring_poison<128, 64, 16, 8, 4, 3, 4>(p, st);
            case 4: return launch_ring_poison<128, 64, 16, 8, 4, 4, 4>(p, st);
        }
        return hipErrorInvalidValue;
    }
    if (p.poison && tile == 10) {
        switch (nstage) {
            case 1: return launch_ring_poison<128, 128, 32, 8, 8, 1, 4>(p, st);
            case 2: return launch_ring_poison<128, 128, 32, 8, 8, 2, 4>(p, st);
            case 3: return launch_ring_poison<128, 128, 32, 8, 8, 3, 4>(p, st);
            case 4: return launch_ring_poison<128, 128, 32, 8, 8, 4, 4>(p, st);
        }
        return hipErrorInvalidValue;
    }
    switch (tile) {
        case 1: return ring_stages<128, 64, 16, 8, 8, 2>(nstage, p, st);  // 128 threads, 2-k steps (8-byte A reads)
        case 2: return ring_stages<64, 64, 16, 4, 4>(nstage, p, st);   // 256 threads
        case 3: return ring_stages<32, 32, 16, 4, 4>(nstage, p, st);   // 64 threads
        case 4: return ring_stages<128, 64, 16, 8, 8>(nstage, p, st);  // tile 1 with 4-k steps
        case 5: return ring_stages<128, 64, 16, 8, 4>(nstage, p, st);  // 256 threads, 8x4 per thread
        case 6: return ring_stages<128, 64, 16, 4, 8>(nstage, p, st);  // 256 threads, 4x8 per thread
        case 7: return ring_stages<32, 32, 32, 4, 4>(nstage, p, st);   // tile 3 with 32-deep slabs
        case 8: return ring_stages<128, 64, 32, 8, 4>(nstage, p, st);  // tile 5 with 32-deep slabs
        case 9: return ring_stages<16, 16, 32, 1, 4>(nstage, p, st);   // 64 threads of 1x4
        case 10: return ring_stages<128, 128, 32, 8, 8>(nstage, p, st); // 256 threads, 8x8 per thread
        case 11: return ring_stages<128, 128, 16, 8, 4>(nstage, p, st); // 512 threads, 8x4 per thread
    }
    return hipErrorInvalidValue;
}

hipError_t launch_valu_staged(int tile, int nstage, const GemmParams& p, hipStream_t st) {
    switch (tile) {
        case 1:
            if (nstage == 1) return launch_staged<128, 64, 16, 8, 8, 1>(p, st);
            if (nstage == 2) return launch_staged<128, 64, 16, 8, 8, 2>(p, st);
            break;
        case 3:
            if (nstage == 1) return launch_staged<32, 32, 16, 4, 4, 1>(p, st);
            if (nstage == 2) return launch_staged<32, 32, 16, 4, 4, 2>(p, st);
            break;
    }
    return hipErrorInvalidValue;
}

}  // namespace gemm
