// mfma.hpp -- bf16 / f16 GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x16 or
// v_mfma_f32_16x16x32): the kernel templates and their launch tables.  Each
// kernels_mfma_<in>_<out>.hip instantiates the tables for one input / output type pair
// (four translation units that compile in parallel); kernels_mfma.hip dispatches.
//
// Hierarchy (sections 1-3 of "CUTLASS-Cute 初步(6)：CUDA GEMM 计算优化、Multi-Stage 与软流水"):
//   workgroup tile BM x BN of C, looped over K in slabs of BK;
//   WM x WN waves, each owning a disjoint (BM/WM) x (BN/WN) block of accumulators;
//   per wave and per k-step (16 deep for 32x32x16, 32 deep for 16x16x32), (BM/WM/MI) A
//   fragments and (BN/WN/MI) B fragments are read from LDS and combined by MI x MI
//   MFMAs -- waves in one row of the tile read the same A fragments, waves in one column
//   the same B fragments.
//
// Operand fragments (one 16-byte LDS read per lane): lane l holds 8 consecutive k of
// row (l mod MI) of the MI-row block, k-chunk l/MI of the k-step; A and B lanes of one
// lane group carry the same k, so each product term meets its partner.  The MFMA is fed
// (B fragment, A fragment), so the MI x MI result it returns is C transposed: for
// MI = 32, lane l, register 4g+j holds C[m = l mod 32][n = 8g + 4*(l/32) + j]; for
// MI = 16, lane l, register j holds C[m = l mod 16][n = 4*(l/16) + j] -- 4 consecutive
// columns per lane and register group, which the epilogue stores as one vector.
#pragma once

#include "common.hpp"
#include "loaders.hpp"
#include "launch.hpp"

namespace gemm {

// MI x MI x KI matrix instruction: MI = 32 (32x32x16, 16 f32 results per lane) or
// MI = 16 (16x16x32, 4 f32 results per lane); both take 8 16-bit values per lane and
// operand and run at the same peak rate.
template <typename T, int MI>
struct Mfma;
template <>
struct Mfma<__bf16, 32> {
    typedef bf16x8 frag;
    typedef f32x16 acc;
    static __device__ __forceinline__ acc run(frag a, frag b, acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mfma<_Float16, 32> {
    typedef f16x8 frag;
    typedef f32x16 acc;
    static __device__ __forceinline__ acc run(frag a, frag b, acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mfma<__bf16, 16> {
    typedef bf16x8 frag;
    typedef f32x4 acc;
    static __device__ __forceinline__ acc run(frag a, frag b, acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mfma<_Float16, 16> {
    typedef f16x8 frag;
    typedef f32x4 acc;
    static __device__ __forceinline__ acc run(frag a, frag b, acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// Shared compute state: accumulators and double-buffered fragments of one wave.
template <typename T, int BM, int BN, int BK, int WM, int WN, int MI = 32>
struct MfmaCompute {
    static constexpr int ROWB = BK * 2;
    static constexpr int CPR = ROWB / 16;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / MI, TN = WTN / MI;
    static constexpr int KI = 512 / MI;             // k per instruction: 16 or 32
    static constexpr int LG = 64 / MI;              // lane groups = 16-byte k-chunks per k-step
    static constexpr int NR = MI * MI / 64;         // f32 results per lane and instruction
    static constexpr int KS = BK / KI;
    static constexpr int A_BYTES = BM * ROWB;
    static constexpr int B_BYTES = BN * ROWB;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static_assert(MI == 16 || MI == 32, "instruction shape");
    static_assert(BK % (2 * KI) == 0, "two k-steps per slab at least");
    static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile is made of MI x MI blocks");

    typedef typename Mfma<T, MI>::frag frag_t;
    typedef typename Mfma<T, MI>::acc acc_t;
    acc_t acc[TM][TN];
    frag_t fa[2][TM];
    frag_t fb[2][TN];
    uint32_t a_off[KS];  // per lane LDS byte offsets within a stage (wave tile row 0)
    uint32_t b_off[KS];
    LDS_AS char* smem;

    __device__ __forceinline__ void init(LDS_AS char* smem_) {
        smem = smem_;
        const int w = wave_id();
        const int wm = w / WN, wn = w % WN;
        const int lane = lane_id();
        const int r = lane % MI;
        const int g = lane / MI;
        // k-chunk of lane group g within the k-step.  The instruction sums over all of its
        // k, so any one-to-one assignment works as long as A and B use the same one (each
        // accumulator still sees a fixed k order).  16x16x32: groups 0..3 take chunks
        // 0, 2, 1, 3 -- with chunks 0..3 in lane order every 16-byte fragment read met a
        // bank conflict on the 128-byte swizzled rows (lanes 0..31 then read two adjacent
        // chunks of 16 rows; a probe of the patterns measured 100% conflicts for that and
        // none for this order, as for the 32x32x16 reads).
        const int kc = MI == 16 ? (g & 1) * 2 + (g >> 1) : g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = LG * ks + kc;
            const int sw = c ^ swz<CPR>(r);  // wave-tile rows are multiples of 16: swz period 16
            a_off[ks] = (uint32_t)((wm * WTM + r) * ROWB + (sw << 4));
            b_off[ks] = (uint32_t)(A_BYTES + (wn * WTN + r) * ROWB + (sw << 4));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < NR; ++e) acc[i][j][e] = 0.0f;
    }

    template <int BUF>
    __device__ __forceinline__ void frag(int slot, int ks) {
        LDS_AS const char* st = smem + slot * STAGE;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[BUF][i] = *reinterpret_cast<LDS_AS const frag_t*>(st + a_off[ks] + i * MI * ROWB);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb[BUF][j] = *reinterpret_cast<LDS_AS const frag_t*>(st + b_off[ks] + j * MI * ROWB);
    }

    // The MFMAs of one k-step.  The next k-step's TM+TN fragment reads and COPIES
    // global->LDS copies were issued in program order just before; the scheduling groups
    // place one fragment read after each of the first TM+TN MFMAs and the copies evenly
    // among all the MFMAs, so that their latency runs under the remaining MFMAs and the
    // copies reach the texture path at the rate it drains them.
    template <int BUF, int COPIES>
    __device__ __forceinline__ void math() {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = Mfma<T, MI>::run(fb[BUF][j], fa[BUF][i], acc[i][j]);
        constexpr int NF = TM + TN;
        constexpr int NM = TM * TN;
        static_assert(NM >= NF, "at least one MFMA per fragment read");
        constexpr int STRIDE = COPIES > 0 ? (NM / COPIES > 0 ? NM / COPIES : 1) : NM + 1;
        constexpr int PER = COPIES > NM ? (COPIES + NM - 1) / NM : 1;
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
            if (i < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
            if (COPIES > 0 && i % STRIDE == 0 && (i / STRIDE) * PER < COPIES)
                __builtin_amdgcn_sched_group_barrier(0x010, PER, 0);            // VMEM (the DMA copies)
        }
        // keep the k-step structure: nothing of the next k-step is hoisted above here
        __builtin_amdgcn_sched_barrier(0);
    }

    // Store the wave's accumulators.  (m0, n0): C coordinates of the tile computed;
    // rows below m_keep / columns below n_keep belong to another tile (edge tiles are
    // shifted inward to stay in bounds) and are not stored here.
    template <int OUT>
    __device__ __forceinline__ void epilogue(const GemmParams& p, int m0, int n0, int m_keep, int n_keep) {
        const int w = wave_id();
        const int wm = w / WN, wn = w % WN;
        const int lane = lane_id();
        // Per batch of quads (a block row's JB column blocks: all of them when that is at
        // most 8 quads, else one, to bound the registers held): with beta != 0, first the
        // old C of the batch (the loads then overlap), then the stores.  A tile inside C
        // (not shifted, not cut) with vector-aligned rows takes unpredicated vectors (a
        // wave-uniform choice): the per-element edge branches would otherwise make the
        // compiler wait between quads.
        constexpr int JB = TN * (NR / 4) <= 8 ? TN : 1;
        if (m0 == m_keep && n0 == n_keep && m0 + BM <= p.M && n0 + BN <= p.N && c_quads_aligned<OUT>(p)) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int m = m0 + wm * WTM + i * MI + (lane % MI);
#pragma unroll
                for (int j0 = 0; j0 < TN; j0 += JB) {
                    f32x4 old[JB][NR / 4];
#pragma unroll
                    for (int j = 0; j < JB; ++j)
#pragma unroll
                        for (int g = 0; g < NR / 4; ++g) old[j][g] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (p.beta != 0.0f) {  // one branch around the batch: its loads issue back to back
#pragma unroll
                        for (int j = 0; j < JB; ++j)
#pragma unroll
                            for (int g = 0; g < NR / 4; ++g)
                                old[j][g] = load_c4_vec<OUT>(p, m, n0 + wn * WTN + (j0 + j) * MI + g * 8 + (lane / MI) * 4);
                    }
#pragma unroll
                    for (int j = 0; j < JB; ++j)
#pragma unroll
                        for (int g = 0; g < NR / 4; ++g) {
                            const int n = n0 + wn * WTN + (j0 + j) * MI + g * 8 + (lane / MI) * 4;
                            f32x4 v;
                            v[0] = acc[i][j0 + j][4 * g + 0];
                            v[1] = acc[i][j0 + j][4 * g + 1];
                            v[2] = acc[i][j0 + j][4 * g + 2];
                            v[3] = acc[i][j0 + j][4 * g + 3];
                            store_c4_vec<OUT>(p, m, n, v, old[j][g]);
                        }
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + wm * WTM + i * MI + (lane % MI);
            const bool mok = m >= m_keep && m < p.M;
#pragma unroll
            for (int j0 = 0; j0 < TN; j0 += JB) {
                f32x4 old[JB][NR / 4];
#pragma unroll
                for (int j = 0; j < JB; ++j)
#pragma unroll
                    for (int g = 0; g < NR / 4; ++g) {
                        // MI = 32: register group g covers n = 8g + 4*(lane/32) + 0..3;
                        // MI = 16: the single group covers n = 4*(lane/16) + 0..3
                        const int n = n0 + wn * WTN + (j0 + j) * MI + g * 8 + (lane / MI) * 4;
                        old[j][g] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (p.beta != 0.0f && mok && n + 3 >= n_keep && n < p.N) old[j][g] = load_c4<OUT>(p, m, n, n_keep);
                    }
#pragma unroll
                for (int j = 0; j < JB; ++j) {
#pragma unroll
                    for (int g = 0; g < NR / 4; ++g) {
                        const int n = n0 + wn * WTN + (j0 + j) * MI + g * 8 + (lane / MI) * 4;
                        if (mok && n + 3 >= n_keep && n < p.N) {
                            f32x4 v;
                            v[0] = acc[i][j0 + j][4 * g + 0];
                            v[1] = acc[i][j0 + j][4 * g + 1];
                            v[2] = acc[i][j0 + j][4 * g + 2];
                            v[3] = acc[i][j0 + j][4 * g + 3];
                            store_c4<OUT>(p, m, n, v, old[j][g], n_keep);
                        }
                    }
                }
            }
        }
    }
    // Workgroup-wide epilogue through LDS for a 16-bit C with beta == 0 on a tile inside C
    // whose rows start 16-byte aligned (every wave of the workgroup calls it; the ring's
    // LDS is free once the K loop is done).  Each lane rounds alpha*acc and writes its
    // quads into a BM x 256 tile in LDS -- row r, 16-byte chunk q at chunk position
    // q ^ (r mod 32) of the row, so the 32 rows a write instruction touches spread over
    // the banks -- then the workgroup stores whole 512-byte rows, 16 bytes per lane.  The
    // lane layout of the accumulators would otherwise store 8-byte pieces of 32 rows per
    // instruction.  Same values as epilogue(): RNE(alpha * acc).
    template <int OUT, int NT>
    __device__ __forceinline__ void epilogue_lds(const GemmParams& p, int m0, int n0) {
        static_assert(OUT != DT_F32 && BN == 256, "16-bit rows of 256 columns");
        constexpr int RB = BN * 2;   // bytes per tile row
        constexpr int CPR_C = RB / 16;
        wait_lgkm0();
        gemm::barrier();             // every wave's last fragment reads are done
        const int w = wave_id();
        const int wm = w / WN, wn = w % WN;
        const int lane = lane_id();
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * WTM + i * MI + (lane % MI);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < NR / 4; ++g) {
                    const int c = wn * WTN + j * MI + g * 8 + (lane / MI) * 4;
                    uint16_t h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = p.alpha * acc[i][j][4 * g + e];
                        h[e] = OUT == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
                    }
                    u32x2 pk;
                    pk[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                    pk[1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
                    const int off = r * RB + (((c >> 3) ^ (r & (CPR_C - 1))) << 4) + (c & 7) * 2;
                    *reinterpret_cast<LDS_AS u32x2*>(smem + off) = pk;
                }
        }
        wait_lgkm0();
        gemm::barrier();
        const int t = threadIdx.x;
#pragma unroll
        for (int k = 0; k < BM * CPR_C / NT; ++k) {
            const int idx = t + NT * k;
            const int r = idx / CPR_C, q = idx % CPR_C;
            const u32x4 v = *reinterpret_cast<LDS_AS const u32x4*>(smem + r * RB + ((q ^ (r & (CPR_C - 1))) << 4));
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.C) + (int64_t)(m0 + r) * p.ldc + n0 + q * 8) = v;
        }
    }
};

// ---------------------------------------------------------------- direct ring kernel
// PIN = false: fragment reads and copies are issued where the K-loop schedule asks for
//   them and the compiler interleaves them with the MFMAs (scheduling-group hints).
// PIN = true: frag() and issue() only note what is asked; the next math() issues it,
//   one fragment read after each of the first TM+TN MFMAs and the k-step's copies evenly
//   spaced over all its MFMAs, each MFMA group closed by a scheduling barrier so the
//   order is exactly that.  Reads for the buffer math() is about to consume (the first
//   k-step of the loop) are issued before its MFMAs; copies noted before a wait (the
//   prologue) or before another request are issued at once.
template <typename T, int BM, int BN, int BK, int WM, int WN, int S, int MI, bool PIN>
struct MfmaRingOps : MfmaCompute<T, BM, BN, BK, WM, WN, MI> {
    typedef MfmaCompute<T, BM, BN, BK, WM, WN, MI> C;
    static constexpr int NW = WM * WN;
    DirectLoader<BM, C::ROWB, NW, true> la;
    DirectLoader<BN, C::ROWB, NW, true> lb;
    static constexpr int LA_N = DirectLoader<BM, C::ROWB, NW, true>::IPW;
    static constexpr int L = LA_N + DirectLoader<BN, C::ROWB, NW, true>::IPW;

    // deferred work (PIN): fragment LDS addresses per buffer, copy run [cp0, cp1)
    LDS_AS const char* fpa[2];
    LDS_AS const char* fpb[2];
    bool fpend[2] = {false, false};
    int cp_slab = 0, cp0 = 0, cp1 = 0;
    LDS_AS char* cp_tile = nullptr;

    // Copies [c0, c1) of this wave's L copies of slab `slab` (A's first, then B's).
    __device__ __forceinline__ void copies(int slab, LDS_AS char* st, int c0, int c1) {
        la.issue(slab, st, c0, c1 < LA_N ? c1 : LA_N);
        lb.issue(slab, st + C::A_BYTES, c0 > LA_N ? c0 - LA_N : 0, c1 - LA_N);
    }
    // Part `part` of `parts` of the copy of slab `slab` into ring slot `slot`: the L
    // copies of this wave are split into equal consecutive runs.
    __device__ __forceinline__ void issue(int slab, int slot, int part, int parts) {
        LDS_AS char* st = this->smem + slot * C::STAGE;
        const int c0 = part * L / parts, c1 = (part + 1) * L / parts;
        if (PIN) {
            flush();   // a second request before any math (the prologue): issue the first now
            cp_slab = slab; cp_tile = st; cp0 = c0; cp1 = c1;
        } else {
            copies(slab, st, c0, c1);
        }
    }
    // Issue noted copies that no math() took (before a wait that counts them).
    __device__ __forceinline__ void flush() {
        if (cp0 < cp1) copies(cp_slab, cp_tile, cp0, cp1);
        cp0 = cp1 = 0;
    }
    template <int N>
    __device__ __forceinline__ void wait_slabs() {
        if (PIN) flush();
        wait_vm<N * L>();
    }
    __device__ __forceinline__ void wait_lds() { wait_lgkm0(); }
    __device__ __forceinline__ void barrier() { gemm::barrier(); }
    template <int BUF>
    __device__ __forceinline__ void frag(int, int slot, int ks) {
        if (PIN) {
            LDS_AS const char* st = this->smem + slot * C::STAGE;
            fpa[BUF] = st + this->a_off[ks];
            fpb[BUF] = st + this->b_off[ks];
            fpend[BUF] = true;
        } else {
            C::template frag<BUF>(slot, ks);
        }
    }
    template <int BUF>
    __device__ __forceinline__ void read_now(int f) {
        if (f < C::TM) this->fa[BUF][f] = *reinterpret_cast<LDS_AS const typename C::frag_t*>(fpa[BUF] + f * MI * C::ROWB);
        else this->fb[BUF][f - C::TM] = *reinterpret_cast<LDS_AS const typename C::frag_t*>(fpb[BUF] + (f - C::TM) * MI * C::ROWB);
    }
    // HAS: this k-step issued one part of PARTS of a slab copy (L copies per slab).
    template <int BUF, int HAS, int PARTS>
    __device__ __forceinline__ void math(int) {
        if (!PIN) {
            C::template math<BUF, HAS ? (L + PARTS - 1) / PARTS : 0>();
            return;
        }
        constexpr int NB = BUF ^ 1;
        constexpr int NM = C::TM * C::TN, NF = C::TM + C::TN;
        constexpr int NC = HAS ? (L + PARTS - 1) / PARTS : 0;   // copies noted for this k-step (at most)
        if (fpend[BUF]) {
#pragma unroll
            for (int f = 0; f < NF; ++f) read_now<BUF>(f);
            fpend[BUF] = false;
        }
#pragma unroll
        for (int t = 0; t < NM; ++t) {
            const int i = t / C::TN, j = t % C::TN;
            this->acc[i][j] = Mfma<T, MI>::run(this->fb[BUF][j], this->fa[BUF][i], this->acc[i][j]);
            // the MFMA first: its operand wait must not also cover the reads issued next
            __builtin_amdgcn_sched_barrier(0);
            if (t < NF && fpend[NB]) read_now<NB>(t);
#pragma unroll
            for (int q = 0; q < NC; ++q)
                if (t == (q * NM) / NC + NM / (2 * NC) && cp0 + q < cp1) copies(cp_slab, cp_tile, cp0 + q, cp0 + q + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        fpend[NB] = false;
        if (cp0 + NC < cp1) copies(cp_slab, cp_tile, cp0 + NC, cp1);   // not reached by the schedule
        cp0 = cp1 = 0;
    }
};

template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S, bool SPREAD, int MI, bool PIN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(
    occupancy_waves(WM * WN * 64, S * MfmaCompute<T, BM, BN, BK, WM, WN>::STAGE, (BM / WM) * (BN / WN) > 64 * 64 ? 1 : 2))))
void mfma_ring_kernel(const GemmParams p) {
    typedef MfmaRingOps<T, BM, BN, BK, WM, WN, S, MI, PIN> Ops;
    __shared__ __attribute__((aligned(1024))) char smem_raw[S * Ops::STAGE];
    int tm, tn;
    tile_coords(p, tm, tn);
    // Edge tiles are shifted inward so that every copy stays inside the matrix
    // (the host guarantees M >= BM and N >= BN for this kernel).
    const int m_keep = tm * BM, n_keep = tn * BN;
    const int m0 = min(m_keep, p.M - BM);
    const int n0 = min(n_keep, p.N - BN);
    Ops ops;
    ops.init((LDS_AS char*)(smem_raw));
    ops.la.init(p.A + (int64_t)m0 * p.lda * 2, p.lda * 2, BK * 2);
    ops.lb.init(p.B + (int64_t)n0 * p.ldb * 2, p.ldb * 2, BK * 2);
    gemm_sched::ring_mainloop<S, Ops::KS, SPREAD ? Ops::KS : 0>(ops, p.K / BK);
    ops.template epilogue<OUT>(p, m0, n0, m_keep, n_keep);
}

// ---------------------------------------------------------------- split-copy ring
// Eight waves, two per SIMD, all multiplying (a 256x256 tile, so a quarter fewer copied
// bytes per FLOP than the 256x128 producer / consumer tile); only the first NC waves --
// one per SIMD -- issue and wait for the copies, so when one of them stalls on a copy the
// other wave of its SIMD keeps the matrix core busy.  Both kinds run the same K-loop
// template and meet at the same barriers.
template <typename T, int BM, int BN, int BK, int WM, int WN, int S, int NC, bool COPY, int MI = 32>
struct SplitCopyOps : MfmaCompute<T, BM, BN, BK, WM, WN, MI> {
    typedef MfmaCompute<T, BM, BN, BK, WM, WN, MI> C;
    DirectLoader<BM, C::ROWB, NC, true> la;
    DirectLoader<BN, C::ROWB, NC, true> lb;
    static constexpr int L = DirectLoader<BM, C::ROWB, NC, true>::IPW + DirectLoader<BN, C::ROWB, NC, true>::IPW;
    // part `part` of `parts` of the slab's L copies (A's first, then B's)
    __device__ __forceinline__ void issue(int slab, int slot, int part, int parts) {
        if (!COPY) return;
        LDS_AS char* st = this->smem + slot * C::STAGE;
        constexpr int LA_N = decltype(la)::IPW;
        const int c0 = part * L / parts, c1 = (part + 1) * L / parts;
        la.issue(slab, st, c0, c1 < LA_N ? c1 : LA_N);
        lb.issue(slab, st + C::A_BYTES, c0 > LA_N ? c0 - LA_N : 0, c1 - LA_N);
    }
    template <int N>
    __device__ __forceinline__ void wait_slabs() { if (COPY) wait_vm<N * L>(); }
    __device__ __forceinline__ void wait_lds() { wait_lgkm0(); }
    __device__ __forceinline__ void barrier() { gemm::barrier(); }
    template <int BUF>
    __device__ __forceinline__ void frag(int, int slot, int ks) { C::template frag<BUF>(slot, ks); }
    template <int BUF, int HAS, int PARTS>
    __device__ __forceinline__ void math(int) { C::template math<BUF, (COPY && HAS) ? (L + PARTS - 1) / PARTS : 0>(); }
};

template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S, int NC, int PARTS, bool POISON,
          int MI>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_split_kernel(const GemmParams p) {
    constexpr int KS = MfmaCompute<T, BM, BN, BK, WM, WN, MI>::KS;
    static constexpr int STAGE = (BM + BN) * BK * 2;
    // a 16-bit C tile of 256 columns leaves through LDS after the K loop (epilogue_lds):
    // at least that much LDS whatever the ring (one workgroup per CU either way)
    static constexpr int EPI = (OUT != DT_F32 && BN == 256) ? BM * BN * 2 : 0;
    static constexpr int SMEM = S * STAGE > EPI ? S * STAGE : EPI;
    __shared__ __attribute__((aligned(1024))) char smem_raw[SMEM];
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m_keep = tm * BM, n_keep = tn * BN;
    const int m0 = min(m_keep, p.M - BM);
    const int n0 = min(n_keep, p.N - BN);
    // 16-bit C, beta == 0, the tile inside C, rows 16-byte aligned: the C tile goes out
    // through the (then idle) LDS ring as whole rows; the same test in every wave
    // (an fp32 C through LDS, in two passes of raw sums, measured 3% slower on the
    // irregular-tail workload than the quad stores, so fp32 keeps those)
    constexpr bool LDS_EPI = EPI > 0;
    const bool lds_epi = LDS_EPI && p.beta == 0.0f && m0 == m_keep && n0 == n_keep && m0 + BM <= p.M &&
                         n0 + BN <= p.N && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 && (p.ldc * 2) % 16 == 0;
    if (wave_id() < NC) {
        MaybePoison<POISON, SplitCopyOps<T, BM, BN, BK, WM, WN, S, NC, true, MI>> ops;
        ops.init((LDS_AS char*)(smem_raw));
        ops.la.init(p.A + (int64_t)m0 * p.lda * 2, p.lda * 2, BK * 2);
        ops.lb.init(p.B + (int64_t)n0 * p.ldb * 2, p.ldb * 2, BK * 2);
        gemm_sched::ring_mainloop<S, KS, PARTS>(ops, p.K / BK);
        if constexpr (LDS_EPI) {
            if (lds_epi) { ops.template epilogue_lds<OUT, WM * WN * 64>(p, m0, n0); return; }
        }
        ops.template epilogue<OUT>(p, m0, n0, m_keep, n_keep);
    } else {
        MaybePoison<POISON, SplitCopyOps<T, BM, BN, BK, WM, WN, S, NC, false, MI>> ops;
        ops.init((LDS_AS char*)(smem_raw));
        gemm_sched::ring_mainloop<S, KS, PARTS>(ops, p.K / BK);
        if constexpr (LDS_EPI) {
            if (lds_epi) { ops.template epilogue_lds<OUT, WM * WN * 64>(p, m0, n0); return; }
        }
        ops.template epilogue<OUT>(p, m0, n0, m_keep, n_keep);
    }
}

// Persistent form of the split-copy ring: one workgroup per compute unit walks the tile
// slots wg, wg + G, wg + 2G, ... (G, the grid, a multiple of 8, so a slot stays on its
// workgroup's XCD) through ONE ring whose slab index g runs over all its tiles' K-slabs.
// The copy of the next tile's first slab is issued while the current tile's last slab is
// multiplied, and the current tile's C is stored between the two (after_slab): the
// stores drain while the next tile computes, and no tile waits for the ring to fill.
template <typename T, int BM, int BN, int BK, int WM, int WN, int S, int NC, bool COPY>
struct SplitPersistOps : SplitCopyOps<T, BM, BN, BK, WM, WN, S, NC, COPY> {
    typedef SplitCopyOps<T, BM, BN, BK, WM, WN, S, NC, COPY> Base;
    typedef MfmaCompute<T, BM, BN, BK, WM, WN, 32> C;
    const GemmParams* gp;
    int numK, wg, G;
    __device__ __forceinline__ void tile_origin(int j, int& m_keep, int& n_keep, int& m0, int& n0) const {
        int tm, tn;
        tile_coords_of(*gp, wg + j * G, tm, tn);
        m_keep = tm * BM;
        n_keep = tn * BN;
        m0 = min(m_keep, gp->M - BM);
        n0 = min(n_keep, gp->N - BN);
    }
    // part `part` of `parts` of the copies of slab g (tile g / numK, K-slab g mod numK)
    __device__ __forceinline__ void issue(int g, int slot, int part, int parts) {
        if (!COPY) return;
        const int j = g / numK, kt = g - j * numK;
        int mk, nk, m0, n0;
        tile_origin(j, mk, nk, m0, n0);
        LDS_AS char* st = this->smem + slot * C::STAGE;
        constexpr int LA_N = decltype(this->la)::IPW;
        const int c0 = part * Base::L / parts, c1 = (part + 1) * Base::L / parts;
        this->la.issue_at(gp->A + ((int64_t)m0 * gp->lda + (int64_t)kt * BK) * 2, st, c0, c1 < LA_N ? c1 : LA_N);
        this->lb.issue_at(gp->B + ((int64_t)n0 * gp->ldb + (int64_t)kt * BK) * 2, st + C::A_BYTES,
                          c0 > LA_N ? c0 - LA_N : 0, c1 - LA_N);
    }
    // after the last k-step of slab g: if g ends a tile, store it and start the next one
    template <int OUT>
    __device__ __forceinline__ void finish_tile(int g) {
        const int j = g / numK;
        if (g - j * numK != numK - 1) return;
        int mk, nk, m0, n0;
        tile_origin(j, mk, nk, m0, n0);
        this->template epilogue<OUT>(*gp, m0, n0, mk, nk);
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int q = 0; q < C::TN; ++q)
#pragma unroll
                for (int e = 0; e < C::NR; ++e) this->acc[i][q][e] = 0.0f;
    }
};
template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S, int NC, bool COPY>
struct SplitPersistOpsOut : SplitPersistOps<T, BM, BN, BK, WM, WN, S, NC, COPY> {
    __device__ __forceinline__ void after_slab(int g) { this->template finish_tile<OUT>(g); }
};

template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S, int NC>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_splitp_kernel(const GemmParams p) {
    static constexpr int STAGE = (BM + BN) * BK * 2;
    __shared__ __attribute__((aligned(1024))) char smem_raw[S * STAGE];
    const int G = gridDim.x, wg = blockIdx.x;
    const int total = p.tiles_m * p.tiles_n;
    const int ntiles = wg < total ? (total - wg + G - 1) / G : 0;
    const int numK = p.K / BK;
    const int nslabs = ntiles * numK;
    if (wave_id() < NC) {
        SplitPersistOpsOut<T, OUT, BM, BN, BK, WM, WN, S, NC, true> ops;
        ops.init((LDS_AS char*)(smem_raw));
        ops.gp = &p; ops.numK = numK; ops.wg = wg; ops.G = G;
        ops.la.init(p.A, p.lda * 2, BK * 2);
        ops.lb.init(p.B, p.ldb * 2, BK * 2);
        gemm_sched::ring_mainloop<S, BK / 16, 0>(ops, nslabs);
    } else {
        SplitPersistOpsOut<T, OUT, BM, BN, BK, WM, WN, S, NC, false> ops;
        ops.init((LDS_AS char*)(smem_raw));
        ops.gp = &p; ops.numK = numK; ops.wg = wg; ops.G = G;
        gemm_sched::ring_mainloop<S, BK / 16, 0>(ops, nslabs);
    }
}

template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S, int NC>
static hipError_t launch_splitp(const GemmParams& p, hipStream_t st) {
    const int total = p.tiles_m * p.tiles_n;
    // one workgroup per CU (the ring takes most of the LDS); a multiple of 8 keeps each
    // tile slot on its workgroup's XCD
    int grid = num_compute_units();
    grid -= grid & 7;
    if (grid < 8) grid = 8;
    if (grid > total) grid = total;
    hipLaunchKernelGGL((mfma_splitp_kernel<T, OUT, BM, BN, BK, WM, WN, S, NC>), dim3(grid), dim3(WM * WN * 64),
                       p.lds_pad, st, p);
    return hipGetLastError();
}

template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S, int NC, int PARTS = 0,
          bool POISON = false, int MI = 32>
static hipError_t launch_split(const GemmParams& p, hipStream_t st) {
    const int grid = p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL((mfma_split_kernel<T, OUT, BM, BN, BK, WM, WN, S, NC, PARTS, POISON, MI>), dim3(grid), dim3(WM * WN * 64),
                       p.lds_pad, st, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------- row-major B in place
// B (K x N) row-major is N-contiguous.  Its K-slab is copied into LDS as it lies -- BK rows
// (one per k) of BN elements, 16-byte chunk c of row r at chunk position c ^ swz<BN/8>(r)
// -- and each lane gathers its B fragment (8 consecutive k of one column) with two
// transposing LDS reads, ds_read_b64_tr_b16: within each group of 16 lanes the instruction
// treats the 8-byte pieces the 16 lanes address as a 16 x 4 block and hands lane i
// element i mod 4 of the pieces addressed by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.  Lane j
// of a group therefore points at row kb + j/4, columns nb + 4(j mod 4) .. +3, and lane i
// receives B[kb .. kb+3][nb + i]; rows kb + 4 .. kb + 7 give the other half.  The fragment
// a lane of the 32x32x16 instruction needs -- column l mod 32, k-chunk l / 32 -- sets
// kb = 8 (g / 2) and nb = 16 (g mod 2) for lane group g = l / 16.  (Layout checked on the
// GPU with a one-wave probe.)  A keeps the K-contiguous [m][k] tile.
template <typename T, int BM, int BN, int BK, int WM, int WN>
struct MfmaKnCompute : MfmaCompute<T, BM, BN, BK, WM, WN, 32> {
    typedef MfmaCompute<T, BM, BN, BK, WM, WN, 32> C;
    static constexpr int ROWB_B = BN * 2;   // bytes per k-row of the B tile
    static constexpr int CPR_B = ROWB_B / 16;
    static_assert(CPR_B == 32, "the transposing reads are laid out for 256-column B tiles");
    static_assert(C::B_BYTES == BK * ROWB_B, "same B bytes per slot in either layout");
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    uint32_t btr[C::TN];   // per lane: byte offset of the piece it addresses for fragment j
                           // (k-step 0, rows kb .. kb+3), relative to the slot

    __device__ __forceinline__ void init(LDS_AS char* smem_) {
        C::init(smem_);
        const int wn = wave_id() % WN;
        const int lane = lane_id();
        const int g = lane / 16, j16 = lane % 16;
        // the k row this lane addresses: rows of one read differ by multiples of 4 from it,
        // so its swizzle phase (row mod 4) is the same for every k-step and half
        const int r = 8 * (g / 2) + j16 / 4;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int n = wn * C::WTN + j * 32 + 16 * (g % 2) + 4 * (j16 % 4);
            btr[j] = (uint32_t)(C::A_BYTES + r * ROWB_B + (((n >> 3) ^ swz<CPR_B>(r)) << 4) + (n & 7) * 2);
        }
    }

    template <int BUF>
    __device__ __forceinline__ void frag(int slot, int ks) {
        LDS_AS const char* st = this->smem + slot * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
            this->fa[BUF][i] = *reinterpret_cast<LDS_AS const typename C::frag_t*>(st + this->a_off[ks] + i * 32 * C::ROWB);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            LDS_AS const char* b = st + btr[j] + ks * 16 * ROWB_B;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(b));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(b + 4 * ROWB_B));
            this->fb[BUF][j] = __builtin_bit_cast(typename C::frag_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    }
};

// Split-copy ring over a row-major A of any alignment and a row-major B read in place.
// The copying waves (one per SIMD) bring each K-slab in two ways: B's BK rows by direct
// global->LDS copies (16-byte aligned rows, one part per k-step of the slab: the part
// count moves this kernel by under half a percent); A's BM rows through registers, with 16-byte loads of any alignment issued as
// soon as the slot is free and written into it just before the barrier that publishes the
// slab (the staged half of the protocol).  A K tail needs no padding: A's columns beyond K
// are cleared in registers, and in the last, partial slab the lanes of B's copies whose
// rows lie beyond K write +0 into LDS instead of copying, so those k add +0 to every sum,
// as in zero-padded operands.  The B copies are issued as inline asm (the global form of
// the LDS-bound load), out of the compiler's sight: it would otherwise make every
// transposing fragment read wait for all copies in flight; the protocol's own vmcnt waits
// and barriers order them.
template <typename T, int BM, int BN, int BK, int WM, int WN, int NC, bool COPY>
struct KnSplitOps : MfmaKnCompute<T, BM, BN, BK, WM, WN> {
    typedef MfmaKnCompute<T, BM, BN, BK, WM, WN> C;
    static constexpr int NTC = NC * 64;                        // copying threads (waves 0..NC-1)
    RowLoader<BM, BK, NTC> la;                                 // A: [m][k] rows, any alignment
    DirectLoader<BK, BN * 2, NC, true, true> lb;               // B: [k][n] rows
    static constexpr int LB = DirectLoader<BK, BN * 2, NC, true, true>::IPW;
    int numK = 0;
    int k_last = BK;          // rows (k) of the last slab that exist
    int pend_slot = 0;        // slot the register-staged A of the next slab goes to
    int pend_slab = 0;

    __device__ __forceinline__ bool partial(int slab) const { return slab == numK - 1 && k_last < BK; }
    __device__ __forceinline__ void issue(int slab, int slot, int part, int parts) {
        if (!COPY) return;
        if (part == 0) {
            la.load(slab, partial(slab));
            pend_slot = slot;
            pend_slab = slab;
        }
        LDS_AS char* st = this->smem + slot * C::STAGE + C::A_BYTES;
        const int i0 = part * LB / parts, i1 = (part + 1) * LB / parts;
        if (partial(slab)) lb.issue_rows(slab, st, i0, i1, k_last);
        else lb.issue(slab, st, i0, i1);
    }
    // Two slots at most: every copy and load in flight belongs to the next slab, which the
    // wait completes; A's registers are then written into its slot (their loads have had
    // the whole slab to arrive: writing them earlier, mid-slab, measured slower), and the
    // LDS counter drained so the barrier that follows publishes them.
    template <int N>
    __device__ __forceinline__ void wait_slabs() {
        static_assert(N == 0, "one slab in flight at most");
        if (!COPY) return;
        wait_vm<0>();
        la.write(this->smem + pend_slot * C::STAGE, pend_slab, partial(pend_slab));
        wait_lgkm0();
    }
    __device__ __forceinline__ void wait_lds() { wait_lgkm0(); }
    __device__ __forceinline__ void barrier() { gemm::barrier(); }
    template <int BUF>
    __device__ __forceinline__ void frag(int, int slot, int ks) { C::template frag<BUF>(slot, ks); }
    template <int BUF, int HAS, int PARTS>
    __device__ __forceinline__ void math(int) { C::template math<BUF, (COPY && HAS) ? (LB + PARTS - 1) / PARTS : 0>(); }
};

template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S, int NC, bool POISON>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_kn_kernel(const GemmParams p) {
    static_assert(S == 1 || S == 2, "the staged half of the protocol holds one slab in registers");
    static constexpr int STAGE = (BM + BN) * BK * 2;
    static constexpr int EPI = (OUT != DT_F32 && BN == 256) ? BM * BN * 2 : 0;
    static constexpr int SMEM = S * STAGE > EPI ? S * STAGE : EPI;
    __shared__ __attribute__((aligned(1024))) char smem_raw[SMEM];
    int tm, tn;
    tile_coords(p, tm, tn);
    // edge tiles shifted inward, as in the other ring kernels (the host guarantees M >= BM,
    // N >= BN); the K range is covered whole, the last slab possibly partial
    const int m_keep = tm * BM, n_keep = tn * BN;
    const int m0 = min(m_keep, p.M - BM);
    const int n0 = min(n_keep, p.N - BN);
    const int numK = (p.K + BK - 1) / BK;
    const int k_last = p.K - (numK - 1) * BK;
    constexpr bool LDS_EPI = EPI > 0;
    const bool lds_epi = LDS_EPI && p.beta == 0.0f && m0 == m_keep && n0 == n_keep && m0 + BM <= p.M &&
                         n0 + BN <= p.N && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 && (p.ldc * 2) % 16 == 0;
    constexpr int KS = BK / 16;
    if (wave_id() < NC) {
        MaybePoison<POISON, KnSplitOps<T, BM, BN, BK, WM, WN, NC, true>> ops;
        ops.init((LDS_AS char*)(smem_raw));
        ops.numK = numK;
        ops.k_last = k_last;
        ops.la.init(p.A, p.lda, m0, p.K, p.M);
        ops.lb.init(p.B + (int64_t)n0 * 2, p.ldb * 2, (int64_t)BK * p.ldb * 2);
        gemm_sched::ring_mainloop<S, KS, S == 1 ? 0 : KS>(ops, numK);
        if constexpr (LDS_EPI) {
            if (lds_epi) { ops.template epilogue_lds<OUT, WM * WN * 64>(p, m0, n0); return; }
        }
        ops.template epilogue<OUT>(p, m0, n0, m_keep, n_keep);
    } else {
        MaybePoison<POISON, KnSplitOps<T, BM, BN, BK, WM, WN, NC, false>> ops;
        ops.init((LDS_AS char*)(smem_raw));
        ops.numK = numK;
        gemm_sched::ring_mainloop<S, KS, S == 1 ? 0 : KS>(ops, numK);
        if constexpr (LDS_EPI) {
            if (lds_epi) { ops.template epilogue_lds<OUT, WM * WN * 64>(p, m0, n0); return; }
        }
        ops.template epilogue<OUT>(p, m0, n0, m_keep, n_keep);
    }
}

template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S, int NC, bool POISON = false>
static hipError_t launch_kn(const GemmParams& p, hipStream_t st) {
    const int grid = p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL((mfma_kn_kernel<T, OUT, BM, BN, BK, WM, WN, S, NC, POISON>), dim3(grid), dim3(WM * WN * 64),
                       p.lds_pad, st, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------- wave-specialised ring
// Producer / consumer split of the same ring: NP producer waves issue every global->LDS
// copy and wait for it; 4 consumer waves (2x2, wave tile (BM/2) x (BN/2)) only read
// fragments and run MFMAs, so a copy never blocks the wave that feeds a matrix core.
// Both roles run the same K-loop template (schedule.hpp) with their half of the work
// and no-ops for the other half, so they meet at exactly the same barriers: a slab is
// published by the barrier after the producers' wait, and a slot is overwritten only
// after the barrier that follows the consumers' last reads of it.
template <typename T, int BM, int BN, int BK, int S, int NP>
struct WsProducerOps {
    static constexpr int ROWB = BK * 2;
    static constexpr int A_BYTES = BM * ROWB;
    static constexpr int STAGE = (BM + BN) * ROWB;
    static constexpr int KS = BK / 16;
    DirectLoader<BM, ROWB, NP, true> la;
    DirectLoader<BN, ROWB, NP, true> lb;
    static constexpr int L = DirectLoader<BM, ROWB, NP, true>::IPW + DirectLoader<BN, ROWB, NP, true>::IPW;
    LDS_AS char* smem;
    __device__ __forceinline__ void issue(int slab, int slot, int, int) {
        LDS_AS char* st = smem + slot * STAGE;
        la.issue(slab, st, 0, decltype(la)::IPW);
        lb.issue(slab, st + A_BYTES, 0, decltype(lb)::IPW);
    }
    template <int N>
    __device__ __forceinline__ void wait_slabs() { wait_vm<N * L>(); }
    __device__ __forceinline__ void wait_lds() {}
    __device__ __forceinline__ void barrier() { gemm::barrier(); }
    template <int BUF>
    __device__ __forceinline__ void frag(int, int, int) {}
    template <int BUF, int HAS, int PARTS>
    __device__ __forceinline__ void math(int) {}
};

template <typename T, int BM, int BN, int BK>
struct WsConsumerOps : MfmaCompute<T, BM, BN, BK, 2, 2, 32> {
    typedef MfmaCompute<T, BM, BN, BK, 2, 2, 32> C;
    __device__ __forceinline__ void issue(int, int, int, int) {}
    template <int N>
    __device__ __forceinline__ void wait_slabs() {}
    __device__ __forceinline__ void wait_lds() { wait_lgkm0(); }
    __device__ __forceinline__ void barrier() { gemm::barrier(); }
    template <int BUF>
    __device__ __forceinline__ void frag(int, int slot, int ks) { C::template frag<BUF>(slot, ks); }
    template <int BUF, int HAS, int PARTS>
    __device__ __forceinline__ void math(int) { C::template math<BUF, 0>(); }
};

template <typename T, int OUT, int BM, int BN, int BK, int S, int NP>
__global__ __launch_bounds__((4 + NP) * 64) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_ws_kernel(const GemmParams p) {
    static constexpr int STAGE = (BM + BN) * BK * 2;
    __shared__ __attribute__((aligned(1024))) char smem_raw[S * STAGE];
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m_keep = tm * BM, n_keep = tn * BN;
    const int m0 = min(m_keep, p.M - BM);
    const int n0 = min(n_keep, p.N - BN);
    const int numK = p.K / BK;
    if (wave_id() >= 4) {
        WsProducerOps<T, BM, BN, BK, S, NP> ops;
        ops.smem = (LDS_AS char*)(smem_raw);
        ops.la.init(p.A + (int64_t)m0 * p.lda * 2, p.lda * 2, BK * 2, wave_id() - 4);
        ops.lb.init(p.B + (int64_t)n0 * p.ldb * 2, p.ldb * 2, BK * 2, wave_id() - 4);
        gemm_sched::ring_mainloop<S, BK / 16, 0>(ops, numK);
    } else {
        WsConsumerOps<T, BM, BN, BK> ops;
        ops.init((LDS_AS char*)(smem_raw));
        gemm_sched::ring_mainloop<S, BK / 16, 0>(ops, numK);
        ops.template epilogue<OUT>(p, m0, n0, m_keep, n_keep);
    }
}

template <typename T, int OUT, int BM, int BN, int BK, int S, int NP>
static hipError_t launch_ws(const GemmParams& p, hipStream_t st) {
    const int grid = p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL((mfma_ws_kernel<T, OUT, BM, BN, BK, S, NP>), dim3(grid), dim3((4 + NP) * 64), p.lds_pad, st, p);
    return hipGetLastError();
}

// Persistent form: one workgroup per CU walks tile slots wg, wg + G, wg + 2G, ... (G =
// grid size) and runs ONE ring over the concatenation of their K-slabs (slab g = tile
// g / numK, K-slab g mod numK).  The producers stream the next tile's first slabs while
// the consumers finish the current tile and store it, so no tile pays the ring's fill.
template <typename T, int BM, int BN, int BK, int S, int NP>
struct WspProducerOps : WsProducerOps<T, BM, BN, BK, S, NP> {
    typedef WsProducerOps<T, BM, BN, BK, S, NP> P;
    const GemmParams* gp;
    int numK, wg, G;
    __device__ __forceinline__ void issue(int g, int slot, int, int) {
        const int j = g / numK, kt = g - j * numK;
        int tm, tn;
        tile_coords_of(*gp, wg + j * G, tm, tn);
        const int m0 = min(tm * BM, gp->M - BM), n0 = min(tn * BN, gp->N - BN);
        LDS_AS char* st = this->smem + slot * P::STAGE;
        this->la.issue_at(gp->A + ((int64_t)m0 * gp->lda + (int64_t)kt * BK) * 2, st, 0, decltype(this->la)::IPW);
        this->lb.issue_at(gp->B + ((int64_t)n0 * gp->ldb + (int64_t)kt * BK) * 2, st + P::A_BYTES, 0,
                          decltype(this->lb)::IPW);
    }
};

template <typename T, int OUT, int BM, int BN, int BK>
struct WspConsumerOps : WsConsumerOps<T, BM, BN, BK> {
    typedef MfmaCompute<T, BM, BN, BK, 2, 2, 32> C;
    const GemmParams* gp;
    int numK, wg, G;
    // after the last k-step of slab g: if g ends a tile, store the tile and start the next
    __device__ __forceinline__ void after_slab(int g) {
        const int j = g / numK;
        if (g - j * numK != numK - 1) return;
        int tm, tn;
        tile_coords_of(*gp, wg + j * G, tm, tn);
        const int m_keep = tm * BM, n_keep = tn * BN;
        this->template epilogue<OUT>(*gp, min(m_keep, gp->M - BM), min(n_keep, gp->N - BN), m_keep, n_keep);
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int q = 0; q < C::TN; ++q)
#pragma unroll
                for (int e = 0; e < C::NR; ++e) this->acc[i][q][e] = 0.0f;
    }
};

template <typename T, int OUT, int BM, int BN, int BK, int S, int NP>
__global__ __launch_bounds__((4 + NP) * 64) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_wsp_kernel(const GemmParams p) {
    static constexpr int STAGE = (BM + BN) * BK * 2;
    __shared__ __attribute__((aligned(1024))) char smem_raw[S * STAGE];
    const int G = gridDim.x, wg = blockIdx.x;
    const int total = p.tiles_m * p.tiles_n;
    const int ntiles = wg < total ? (total - wg + G - 1) / G : 0;
    const int numK = p.K / BK;
    const int nslabs = ntiles * numK;
    if (wave_id() >= 4) {
        WspProducerOps<T, BM, BN, BK, S, NP> ops;
        ops.smem = (LDS_AS char*)(smem_raw);
        ops.gp = &p; ops.numK = numK; ops.wg = wg; ops.G = G;
        ops.la.init(p.A, p.lda * 2, BK * 2, wave_id() - 4);
        ops.lb.init(p.B, p.ldb * 2, BK * 2, wave_id() - 4);
        gemm_sched::ring_mainloop<S, BK / 16, 0>(ops, nslabs);
    } else {
        WspConsumerOps<T, OUT, BM, BN, BK> ops;
        ops.init((LDS_AS char*)(smem_raw));
        ops.gp = &p; ops.numK = numK; ops.wg = wg; ops.G = G;
        gemm_sched::ring_mainloop<S, BK / 16, 0>(ops, nslabs);
    }
}

template <typename T, int OUT, int BM, int BN, int BK, int S, int NP>
static hipError_t launch_wsp(const GemmParams& p, hipStream_t st) {
    const int total = p.tiles_m * p.tiles_n;
    // one workgroup per CU (the ring takes most of the LDS); a multiple of 8 keeps each
    // tile slot on its workgroup's XCD
    int grid = num_compute_units();
    grid -= grid & 7;
    if (grid < 8) grid = 8;
    if (grid > total) grid = total;
    hipLaunchKernelGGL((mfma_wsp_kernel<T, OUT, BM, BN, BK, S, NP>), dim3(grid), dim3((4 + NP) * 64), p.lds_pad, st, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------- staged kernel
// AT / BT: the operand is contiguous across the LDS rows (A column-major, B row-major)
// and is transposed on its way into the K-contiguous LDS tile.
template <typename T, int BM, int BN, int BK, int WM, int WN, int S, bool AT, bool BT>
struct MfmaStagedOps : MfmaCompute<T, BM, BN, BK, WM, WN> {
    typedef MfmaCompute<T, BM, BN, BK, WM, WN> C;
    static constexpr int NT = WM * WN * 64;
    StagedLoader<BM, BK, 2, NT, true, AT> la;
    StagedLoader<BN, BK, 2, NT, true, BT> lb;

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
    __device__ __forceinline__ void math(int) { C::template math<BUF, 0>(); }
};

template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S, bool AT, bool BT>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(
    occupancy_waves(WM * WN * 64, S * MfmaCompute<T, BM, BN, BK, WM, WN>::STAGE, 2))))
void mfma_staged_kernel(const GemmParams p) {
    typedef MfmaStagedOps<T, BM, BN, BK, WM, WN, S, AT, BT> Ops;
    __shared__ __attribute__((aligned(1024))) char smem_raw[S * Ops::STAGE];
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    Ops ops;
    ops.init((LDS_AS char*)(smem_raw));
    // LDS rows of A are m (k along the row); of B, n.
    ops.la.init(p.A, p.lda, m0, 0, p.M, p.K, p.a_vec != 0, false);
    ops.lb.init(p.B, p.ldb, n0, 0, p.N, p.K, p.b_vec != 0, false);
    gemm_sched::staged_mainloop<S, Ops::KS>(ops, (p.K + BK - 1) / BK);
    ops.template epilogue<OUT>(p, m0, n0, m0, n0);
}

// ---------------------------------------------------------------- launch tables
template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S, bool SPREAD = false, int MI = 32, bool PIN = false>
static hipError_t launch_ring(const GemmParams& p, hipStream_t st) {
    const int grid = p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL((mfma_ring_kernel<T, OUT, BM, BN, BK, WM, WN, S, SPREAD, MI, PIN>), dim3(grid), dim3(WM * WN * 64), p.lds_pad, st, p);
    return hipGetLastError();
}
template <typename T, int OUT, int BM, int BN, int BK, int WM, int WN, int S>
static hipError_t launch_staged(const GemmParams& p, hipStream_t st) {
    const dim3 grid(p.tiles_m * p.tiles_n), block(WM * WN * 64);
    const bool at = p.a_col != 0, bt = p.b_col == 0;  // contiguous across the LDS rows
    if (!at && !bt)
        hipLaunchKernelGGL((mfma_staged_kernel<T, OUT, BM, BN, BK, WM, WN, S, false, false>), grid, block, p.lds_pad, st, p);
    else if (!at && bt)
        hipLaunchKernelGGL((mfma_staged_kernel<T, OUT, BM, BN, BK, WM, WN, S, false, true>), grid, block, p.lds_pad, st, p);
    else if (at && !bt)
        hipLaunchKernelGGL((mfma_staged_kernel<T, OUT, BM, BN, BK, WM, WN, S, true, false>), grid, block, p.lds_pad, st, p);
    else
        hipLaunchKernelGGL((mfma_staged_kernel<T, OUT, BM, BN, BK, WM, WN, S, true, true>), grid, block, p.lds_pad, st, p);
    return hipGetLastError();
}

template <typename T, int OUT>
hipError_t ring_dispatch(int tile, int S, const GemmParams& p, hipStream_t st) {
    switch (tile) {
        case 1:  // 256x256x64, 2x2 waves of 128x128
            if (S == 1) return launch_ring<T, OUT, 256, 256, 64, 2, 2, 1>(p, st);
            if (S == 2) return launch_ring<T, OUT, 256, 256, 64, 2, 2, 2>(p, st);
            break;
        case 2:  // 256x256x32, 2x2 waves of 128x128
            if (S == 1) return launch_ring<T, OUT, 256, 256, 32, 2, 2, 1>(p, st);
            if (S == 2) return launch_ring<T, OUT, 256, 256, 32, 2, 2, 2>(p, st);
            if (S == 3) return launch_ring<T, OUT, 256, 256, 32, 2, 2, 3>(p, st);
            if (S == 4) return launch_ring<T, OUT, 256, 256, 32, 2, 2, 4>(p, st);
            break;
        case 3:  // 128x128x64, 2x2 waves of 64x64
            if (S == 1) return launch_ring<T, OUT, 128, 128, 64, 2, 2, 1>(p, st);
            if (S == 2) return launch_ring<T, OUT, 128, 128, 64, 2, 2, 2>(p, st);
            if (S == 3) return launch_ring<T, OUT, 128, 128, 64, 2, 2, 3>(p, st);
            if (S == 4) return launch_ring<T, OUT, 128, 128, 64, 2, 2, 4>(p, st);
            break;
        case 18:  // 256x128x64, 4 consumer waves + 2 producer waves
            if (S == 1) return launch_ws<T, OUT, 256, 128, 64, 1, 2>(p, st);
            if (S == 2) return launch_ws<T, OUT, 256, 128, 64, 2, 2>(p, st);
            if (S == 3) return launch_ws<T, OUT, 256, 128, 64, 3, 2>(p, st);
            break;
        case 19:  // tile 18 (4 consumer + 2 producer waves), persistent
            if (S == 2) return launch_wsp<T, OUT, 256, 128, 64, 2, 2>(p, st);
            if (S == 3) return launch_wsp<T, OUT, 256, 128, 64, 3, 2>(p, st);
            break;
        case 23:  // 256x256x64, 2x4 waves of 128x64, copies by waves 0-3 only
            if (S == 1) return launch_split<T, OUT, 256, 256, 64, 2, 4, 1, 4>(p, st);
            if (S == 2) return launch_split<T, OUT, 256, 256, 64, 2, 4, 2, 4>(p, st);
            break;
        case 24:  // tile 23 with each slab's copies spread over its 4 k-steps (S = 1: one slot,
                  // the slab's copies go out together, as in tile 23)
            if (S == 1) return launch_split<T, OUT, 256, 256, 64, 2, 4, 1, 4, 4>(p, st);
            if (S == 2) return launch_split<T, OUT, 256, 256, 64, 2, 4, 2, 4, 4>(p, st);
            break;
        case 25:  // 256x256x32, 2x4 waves, copies by waves 0-3 spread, deeper ring
            if (S == 3) return launch_split<T, OUT, 256, 256, 32, 2, 4, 3, 4, 2>(p, st);
            if (S == 4) return launch_split<T, OUT, 256, 256, 32, 2, 4, 4, 4, 2>(p, st);
            break;
        case 26:  // 256x192x64, 4x2 waves of 64x96, copies by waves 0-3 only
            if (S == 1) return launch_split<T, OUT, 256, 192, 64, 4, 2, 1, 4>(p, st);
            if (S == 2) return launch_split<T, OUT, 256, 192, 64, 4, 2, 2, 4>(p, st);
            break;
        case 28:  // tile 23, persistent (one workgroup per CU walks several tiles through one ring)
            if (S == 2) return launch_splitp<T, OUT, 256, 256, 64, 2, 4, 2, 4>(p, st);
            break;
        case 30:  // 192x256x64, 2x4 waves of 96x64: row-major A through registers, row-major B in place
            if constexpr (std::is_same<T, __bf16>::value) {   // the LDS-poisoning debug variant
                if (p.poison && S == 1) return launch_kn<T, OUT, 192, 256, 64, 2, 4, 1, 4, true>(p, st);
                if (p.poison && S == 2) return launch_kn<T, OUT, 192, 256, 64, 2, 4, 2, 4, true>(p, st);
            }
            if (S == 1) return launch_kn<T, OUT, 192, 256, 64, 2, 4, 1, 4>(p, st);
            if (S == 2) return launch_kn<T, OUT, 192, 256, 64, 2, 4, 2, 4>(p, st);
            break;
        case 31:  // tile 23 with 16x16x32 instructions, each slab's copies issued together right
                  // after the barrier that frees its slot (the default 256x256 tile)
            if constexpr (std::is_same<T, __bf16>::value) {   // the LDS-poisoning debug variant
                if (p.poison && S == 1) return launch_split<T, OUT, 256, 256, 64, 2, 4, 1, 4, 1, true, 16>(p, st);
                if (p.poison && S == 2) return launch_split<T, OUT, 256, 256, 64, 2, 4, 2, 4, 1, true, 16>(p, st);
            }
            if (S == 1) return launch_split<T, OUT, 256, 256, 64, 2, 4, 1, 4, 1, false, 16>(p, st);
            if (S == 2) return launch_split<T, OUT, 256, 256, 64, 2, 4, 2, 4, 1, false, 16>(p, st);
            break;
        case 32:  // tile 31's scheme on 192x256
            if (S == 1) return launch_split<T, OUT, 192, 256, 64, 2, 4, 1, 4, 1, false, 16>(p, st);
            if (S == 2) return launch_split<T, OUT, 192, 256, 64, 2, 4, 2, 4, 1, false, 16>(p, st);
            break;
        case 29:  // tile 27 (192x256) with each slab's copies spread over its 4 k-steps
            if (S == 1) return launch_split<T, OUT, 192, 256, 64, 2, 4, 1, 4, 4>(p, st);
            if (S == 2) return launch_split<T, OUT, 192, 256, 64, 2, 4, 2, 4, 4>(p, st);
            break;
#ifdef GEMM_ALL_TILES
        case 4:  // 256x256x64, 2x2 waves, copies spread over the whole slab
            if (S == 2) return launch_ring<T, OUT, 256, 256, 64, 2, 2, 2, true>(p, st);
            break;
        case 5:  // 256x256x32, 2x2 waves, copies spread
            if (S == 3) return launch_ring<T, OUT, 256, 256, 32, 2, 2, 3, true>(p, st);
            if (S == 4) return launch_ring<T, OUT, 256, 256, 32, 2, 2, 4, true>(p, st);
            break;
        case 6:  // 128x128x64, copies spread
            if (S == 2) return launch_ring<T, OUT, 128, 128, 64, 2, 2, 2, true>(p, st);
            if (S == 3) return launch_ring<T, OUT, 128, 128, 64, 2, 2, 3, true>(p, st);
            break;
        case 7:  // 256x256x64, 2x4 waves of 128x64 (two waves per SIMD), copies spread
            if (S == 2) return launch_ring<T, OUT, 256, 256, 64, 2, 4, 2, true>(p, st);
            break;
        case 8:  // 256x256x64, 4x2 waves of 64x128 (two waves per SIMD)
            if (S == 2) return launch_ring<T, OUT, 256, 256, 64, 4, 2, 2>(p, st);
            break;
        case 9:  // 256x256x32, 2x4 waves of 128x64, deeper ring, copies spread
            if (S == 3) return launch_ring<T, OUT, 256, 256, 32, 2, 4, 3, true>(p, st);
            if (S == 4) return launch_ring<T, OUT, 256, 256, 32, 2, 4, 4, true>(p, st);
            break;
        case 10:  // 256x256x64, 2x2 waves, 16x16x32 instructions
            if (S == 2) return launch_ring<T, OUT, 256, 256, 64, 2, 2, 2, false, 16>(p, st);
            break;
        case 11:  // 256x256x64, 2x2 waves, 16x16x32 instructions, copies spread
            if (S == 2) return launch_ring<T, OUT, 256, 256, 64, 2, 2, 2, true, 16>(p, st);
            break;
        case 12:  // 128x128x64, 2x2 waves, 16x16x32 instructions
            if (S == 2) return launch_ring<T, OUT, 128, 128, 64, 2, 2, 2, false, 16>(p, st);
            if (S == 3) return launch_ring<T, OUT, 128, 128, 64, 2, 2, 3, false, 16>(p, st);
            break;
        case 13:  // tile 1 with pinned issue order
            if (S == 1) return launch_ring<T, OUT, 256, 256, 64, 2, 2, 1, false, 32, true>(p, st);
            if (S == 2) return launch_ring<T, OUT, 256, 256, 64, 2, 2, 2, false, 32, true>(p, st);
            break;
        case 14:  // tile 4 (spread) with pinned issue order
            if (S == 2) return launch_ring<T, OUT, 256, 256, 64, 2, 2, 2, true, 32, true>(p, st);
            break;
        case 15:  // tile 5 (256x256x32, spread) with pinned issue order
            if (S == 3) return launch_ring<T, OUT, 256, 256, 32, 2, 2, 3, true, 32, true>(p, st);
            if (S == 4) return launch_ring<T, OUT, 256, 256, 32, 2, 2, 4, true, 32, true>(p, st);
            break;
        case 16:  // tile 9 (8 waves, 256x256x32, spread) with pinned issue order
            if (S == 3) return launch_ring<T, OUT, 256, 256, 32, 2, 4, 3, true, 32, true>(p, st);
            if (S == 4) return launch_ring<T, OUT, 256, 256, 32, 2, 4, 4, true, 32, true>(p, st);
            break;
        case 17:  // 256x128x64, 4 consumer waves (128x64) + 4 producer waves
            if (S == 1) return launch_ws<T, OUT, 256, 128, 64, 1, 4>(p, st);
            if (S == 2) return launch_ws<T, OUT, 256, 128, 64, 2, 4>(p, st);
            if (S == 3) return launch_ws<T, OUT, 256, 128, 64, 3, 4>(p, st);
            break;
        case 20:  // tile 17 (4 consumer + 4 producer waves), persistent
            if (S == 3) return launch_wsp<T, OUT, 256, 128, 64, 3, 4>(p, st);
            break;
        case 21:  // 256x256x64, 4x2 waves of 64x128, copies by waves 0-3 only
            if (S == 1) return launch_split<T, OUT, 256, 256, 64, 4, 2, 1, 4>(p, st);
            if (S == 2) return launch_split<T, OUT, 256, 256, 64, 4, 2, 2, 4>(p, st);
            break;
        case 22:  // 256x128x64, 4 consumer waves + 1 producer wave
            if (S == 3) return launch_ws<T, OUT, 256, 128, 64, 3, 1>(p, st);
            break;
        case 27:  // 192x256x64, 2x4 waves of 96x64, copies by waves 0-3 only
            if (S == 1) return launch_split<T, OUT, 192, 256, 64, 2, 4, 1, 4>(p, st);
            if (S == 2) return launch_split<T, OUT, 192, 256, 64, 2, 4, 2, 4>(p, st);
            break;
#endif
    }
    return hipErrorInvalidValue;
}

template <typename T, int OUT>
hipError_t staged_dispatch(int tile, int S, const GemmParams& p, hipStream_t st) {
    switch (tile) {
        case 1:  // 128x128x32, 2x2 waves of 64x64
            if (S == 1) return launch_staged<T, OUT, 128, 128, 32, 2, 2, 1>(p, st);
            if (S == 2) return launch_staged<T, OUT, 128, 128, 32, 2, 2, 2>(p, st);
            break;
        case 2:  // 128x128x64, 2x2 waves of 64x64 (half the barriers per FLOP)
            if (S == 1) return launch_staged<T, OUT, 128, 128, 64, 2, 2, 1>(p, st);
            if (S == 2) return launch_staged<T, OUT, 128, 128, 64, 2, 2, 2>(p, st);
            break;
    }
    return hipErrorInvalidValue;
}

}  // namespace gemm
