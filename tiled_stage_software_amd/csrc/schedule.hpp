// schedule.hpp -- the K-loop protocol of every GEMM kernel, written once.
//
// The mainloops below are templates over an `Ops` object.  On the device, Ops issues
// global->LDS copies, s_waitcnt, s_barrier, LDS->register fragment loads and the
// math; on the host (gemm_schedule in the C ABI) a recording Ops replays the very same
// control flow into an event list, which the CPU tests check for read-after-write and
// write-after-read hazards on the LDS ring.
//
// Ring protocol (direct global->LDS copies, S = nStage LDS slots):
//   * prologue: slabs 0..S-2 are issued into slots 0..S-2 (the multi-stage prologue of
//     section 5.3 of "CUTLASS-Cute 初步(6)：CUDA GEMM 计算优化、Multi-Stage 与软流水");
//   * at the first k-step of slab kt, slab kt+S-1 is issued into slot (kt+S-1) mod S,
//     the slot slab kt-1 used (the ring index advancing modulo the stage count of
//     "Matrix multiplication", and the producer index of section 5.3 running one slot
//     ahead of the consumer);
//   * at the last k-step of slab kt the wave waits until slab kt+1 has landed, leaving
//     the newer slabs in flight, then the workgroup barriers once (copy completion is
//     per thread, so a barrier is still needed before other waves read the slab, as
//     "Matrix multiplication" points out), then the first fragments of slab kt+1 are
//     read while the last k-step of slab kt is multiplied;
//   * register fragments are double-buffered across k-steps (the warp-scope double
//     buffering of "Matrix multiplication" and section 6 of the multi-stage page).
//   A copy that would be past the last slab is simply not issued: the last S-1 slabs
//   run a tail body that waits for everything still in flight, so the "stages in
//   flight" bookkeeping stays exact without dummy copies (the role of the
//   always-committed stage in the N-stage ring of "Matrix multiplication").
//   S = 1 is the single-buffer loop: load, wait, barrier, compute, barrier -- the two
//   barriers of "The bubble in the tiled loop" ("Software Pipelining and Double
//   Buffering").
//
// Staged protocol (loads through registers, S = 1 or 2): with S = 2 the global loads
// of slab kt+1 are issued into registers at the start of slab kt and written to the
// other LDS slot after slab kt's math, one barrier per slab (the listing of
// "Double buffering with shared memory" on the same page); S = 1 is the two-barrier
// loop.
#pragma once

#if defined(__HIPCC__)
#define GEMM_HD __host__ __device__ __forceinline__
#else
#define GEMM_HD inline
#endif

namespace gemm_sched {

GEMM_HD constexpr int imin(int a, int b) { return a < b ? a : b; }
GEMM_HD constexpr int imax(int a, int b) { return a > b ? a : b; }

enum { BODY_MAIN = 0, BODY_MAIN_END = 1, BODY_TAIL = 2, BODY_LAST = 3 };

// Hook right after the barrier that releases a ring slot: every wave has finished reading
// the slab in it and nothing has been issued into it yet.  Ops without a release member
// (the production kernels) do nothing there; the LDS-poisoning debug wrapper overwrites
// the slot.
template <class O>
GEMM_HD auto release_(O& o, int slot, int) -> decltype(o.release(slot), void()) { o.release(slot); }
template <class O>
GEMM_HD void release_(O&, int, long) {}

// One slab of KS k-steps.  Every branch here is on compile-time values, so the unrolled
// body is straight-line code (a run-time branch inside it lets the compiler sink the
// math below it and keep every fragment of the slab live at once).
//
// PARTS = 0: the whole copy of slab kt+S-1 is issued at the first k-step.
// PARTS = P in 1..KS: the copy is split into P parts: part 0 right after the barrier that
//   ends slab kt-1 (that barrier frees the slot), parts 1..P-1 at k-steps 0..P-2 of slab
//   kt.  With P = KS the copies trickle out at the rate the texture path drains them
//   instead of backing up the wave's issue; with P = 1 the whole slab goes out at the
//   earliest point the slot allows.  Every part is issued before the wait that counts it.
//   BODY_MAIN:     issues (its parts of) slab kt+S-1 and, with PARTS > 0, part 0 of slab
//                  kt+S after its barrier; waits for slab kt+1 leaving S-2 slabs in flight.
//   BODY_MAIN_END: the last slab that issues: no part 0 of a next slab.
//   BODY_TAIL:     nothing left to issue; waits for everything in flight.
//   BODY_LAST:     the last slab: no copy, no barrier, no read-ahead.
template <int S, int KS, int PARTS, int BODY, class Ops>
GEMM_HD void ring_slab(Ops& ops, int kt, int slot, int issue_slot, int next_slot) {
    static_assert(PARTS >= 0 && PARTS <= KS, "at most one part per k-step");
    constexpr bool ISSUING = BODY == BODY_MAIN || BODY == BODY_MAIN_END;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        int copies_here = 0;  // parts issued in this k-step (for the math's interleave)
        if (ISSUING) {
            if (PARTS == 0 && ks == 0) { ops.issue(kt + S - 1, issue_slot, 0, 1); copies_here = KS; }
            if (PARTS > 0 && ks < PARTS - 1) { ops.issue(kt + S - 1, issue_slot, ks + 1, PARTS); copies_here = 1; }
        }
        if (ks == KS - 1) {
            if (BODY != BODY_LAST) {
                ops.wait_lds();
                ops.template wait_slabs<BODY == BODY_TAIL ? 0 : S - 2>();
                ops.barrier();
                release_(ops, slot, 0);
                ops.template frag<0>(kt + 1, next_slot, 0);
                // the barrier freed this slab's slot: start the copy of slab kt+S into it
                if (PARTS > 0 && BODY == BODY_MAIN) { ops.issue(kt + S, slot, 0, PARTS); copies_here = PARTS == 1 ? KS : 1; }
            }
        } else {
            if (ks % 2 == 0) ops.template frag<1>(kt, slot, ks + 1);
            else ops.template frag<0>(kt, slot, ks + 1);
        }
        // copies_here is a compile-time constant after unrolling
        if (copies_here == KS) {
            if (ks % 2 == 0) ops.template math<0, 1, 1>(ks);
            else ops.template math<1, 1, 1>(ks);
        } else if (copies_here == 1) {
            constexpr int P = PARTS > 0 ? PARTS : 1;   // (PARTS == 0 never gets here)
            if (ks % 2 == 0) ops.template math<0, 1, P>(ks);
            else ops.template math<1, 1, P>(ks);
        } else {
            if (ks % 2 == 0) ops.template math<0, 0, 1>(ks);
            else ops.template math<1, 0, 1>(ks);
        }
    }
}

// One slab of the single-buffer loop: load, wait, barrier, compute, barrier.
template <int KS, class Ops>
GEMM_HD void single_slab_compute(Ops& ops, int kt) {
    ops.template frag<0>(kt, 0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
            if (ks % 2 == 0) ops.template frag<1>(kt, 0, ks + 1);
            else ops.template frag<0>(kt, 0, ks + 1);
        }
        if (ks % 2 == 0) ops.template math<0, 0, 1>(ks);
        else ops.template math<1, 0, 1>(ks);
    }
}

// Direct global->LDS ring.  KS = k-steps per slab (even); PARTS: see ring_slab.
// Hook after slab kt's last k-step (a persistent kernel stores a finished tile there);
// Ops without an after_slab member do nothing.
template <class O>
GEMM_HD auto after_slab_(O& o, int kt, int) -> decltype(o.after_slab(kt), void()) { o.after_slab(kt); }
template <class O>
GEMM_HD void after_slab_(O&, int, long) {}

template <int S, int KS, int PARTS, class Ops>
GEMM_HD void ring_mainloop(Ops& ops, int numK) {
    static_assert(KS % 2 == 0, "fragment double-buffering needs an even number of k-steps");
    static_assert(S >= 1, "at least one LDS slot");
    if (numK <= 0) return;
    if constexpr (S == 1) {
        for (int kt = 0; kt < numK; ++kt) {
            ops.issue(kt, 0, 0, 1);
            ops.template wait_slabs<0>();
            ops.barrier();
            single_slab_compute<KS>(ops, kt);
            ops.wait_lds();
            ops.barrier();
            release_(ops, 0, 0);
            after_slab_(ops, kt, 0);
        }
    } else {
        // prologue: slabs 0 .. S-2 (fewer if K is short); wait for slab 0
        for (int s = 0; s < S - 1; ++s)
            if (s < numK) ops.issue(s, s, 0, 1);
        if (numK >= S - 1) ops.template wait_slabs<S - 2>();
        else ops.template wait_slabs<0>();
        ops.barrier();
        ops.template frag<0>(0, 0, 0);
        // PARTS > 0: part 0 of slab S-1 goes into the still unused slot S-1
        if (PARTS > 0 && numK > S - 1) ops.issue(S - 1, S - 1, 0, PARTS);
        int kt = 0;
        int slot = 0;            // slot of slab kt
        int issue_slot = S - 1;  // slot of slab kt+S-1 (= the slot slab kt-1 used)
        const int main_end = numK - S + 1;  // slabs whose body still issues a copy
        for (; kt < main_end - 1; ++kt) {
            const int next_slot = (slot + 1 == S) ? 0 : slot + 1;
            ring_slab<S, KS, PARTS, BODY_MAIN>(ops, kt, slot, issue_slot, next_slot);
            after_slab_(ops, kt, 0);
            slot = next_slot;
            issue_slot = (issue_slot + 1 == S) ? 0 : issue_slot + 1;
        }
        if (kt < main_end) {
            const int next_slot = (slot + 1 == S) ? 0 : slot + 1;
            ring_slab<S, KS, PARTS, BODY_MAIN_END>(ops, kt, slot, issue_slot, next_slot);
            after_slab_(ops, kt, 0);
            slot = next_slot;
            ++kt;
        }
        for (; kt < numK - 1; ++kt) {
            const int next_slot = (slot + 1 == S) ? 0 : slot + 1;
            ring_slab<S, KS, PARTS, BODY_TAIL>(ops, kt, slot, 0, next_slot);
            after_slab_(ops, kt, 0);
            slot = next_slot;
        }
        ring_slab<S, KS, PARTS, BODY_LAST>(ops, kt, slot, 0, 0);
        after_slab_(ops, kt, 0);
    }
}

// One slab of the register-staged double buffer: the loads of slab kt+1 were issued
// into registers before this slab's math; after the second-to-last k-step they are
// written into the other slot, then one barrier publishes them.
template <int KS, bool LAST, class Ops>
GEMM_HD void staged_slab(Ops& ops, int kt, int slot) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (ks == KS - 1) {
            if (!LAST) {
                ops.write(kt + 1, slot ^ 1);
                ops.wait_lds();
                ops.barrier();
                ops.template frag<0>(kt + 1, slot ^ 1, 0);
            }
        } else {
            if (ks % 2 == 0) ops.template frag<1>(kt, slot, ks + 1);
            else ops.template frag<0>(kt, slot, ks + 1);
        }
        if (ks % 2 == 0) ops.template math<0, 0, 1>(ks);
        else ops.template math<1, 0, 1>(ks);
    }
}

// Register-staged loads.  S = 1 or 2.
template <int S, int KS, class Ops>
GEMM_HD void staged_mainloop(Ops& ops, int numK) {
    static_assert(KS % 2 == 0, "fragment double-buffering needs an even number of k-steps");
    static_assert(S == 1 || S == 2, "staged kernels use one or two LDS slots");
    if (numK <= 0) return;
    if constexpr (S == 1) {
        for (int kt = 0; kt < numK; ++kt) {
            ops.load(kt);
            ops.write(kt, 0);
            ops.wait_lds();
            ops.barrier();
            single_slab_compute<KS>(ops, kt);
            ops.wait_lds();
            ops.barrier();
            after_slab_(ops, kt, 0);
        }
    } else {
        ops.load(0);
        ops.write(0, 0);
        ops.wait_lds();
        ops.barrier();
        ops.template frag<0>(0, 0, 0);
        int slot = 0;
        int kt = 0;
        for (; kt < numK - 1; ++kt) {
            ops.load(kt + 1);
            staged_slab<KS, false>(ops, kt, slot);
            slot ^= 1;
        }
        staged_slab<KS, true>(ops, kt, slot);
    }
}

}  // namespace gemm_sched
