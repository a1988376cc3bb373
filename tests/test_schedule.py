"""The K-loop protocol of every kernel family, checked on the CPU (no GPU).

``gemm_schedule`` replays the very template the kernels run (schedule.hpp) with a
recording backend; this test executes the event list against a model of one
workgroup and asserts that no LDS slot is read before its slab has landed and been
published by a barrier (read-after-write), that no slot is overwritten while some wave
may still read it (write-after-read), that every slab is computed exactly once in
order, and the protocol counts the pages describe: nStage-1 slabs in the prologue,
wait-for-oldest leaving nStage-2 in flight, one barrier per slab when double buffered
and two when single buffered.
"""
import pytest

from tiled_stage_software_amd import libgemm as lg

ISSUE, WAIT, BARRIER, COMPUTE, WRITE, WAIT_LDS = 1, 2, 3, 4, 5, 6


def simulate(events, S, numK, ksteps, staged):
    slot_slab = {}          # slot -> slab whose copy / write went there last
    in_flight = []          # direct copies issued and not yet known complete (oldest first)
    complete = set()        # slabs whose copies have landed (this wave's view)
    visible = set()         # slabs published to all waves by a barrier after completion
    written_pending = set() # staged: LDS writes not yet completed (wait_lds)
    written_done = set()
    reg_loaded = set()
    slot_reads = {}         # slot -> 'read' | 'done'  (reads not yet fenced by wait_lds+barrier)
    computed = []
    barriers = 0
    waits = []
    parts_seen = {}         # slab -> [parts issued, parts]
    for (t, slab, slot, arg) in events:
        if t == ISSUE:
            if staged:
                assert slot == -1
                reg_loaded.add(slab)
                continue
            assert 0 <= slot < S
            assert slot_reads.get(slot) is None, f"WAR: copy of slab {slab} into slot {slot} while it may be read"
            part, parts = arg & 0xff, max(1, arg >> 8)
            if part == 0:
                assert slab not in parts_seen, f"slab {slab} issued twice"
                parts_seen[slab] = [0, parts]
                slot_slab[slot] = slab
                in_flight.append(slab)
            else:
                assert slot_slab.get(slot) == slab and parts_seen[slab][0] == part, "parts in order, same slot"
            parts_seen[slab][0] += 1
        elif t == WRITE:
            assert staged and slab in reg_loaded, "write before the global load"
            assert slot_reads.get(slot) is None, f"WAR: write of slab {slab} into slot {slot} while it may be read"
            slot_slab[slot] = slab
            written_pending.add(slab)
        elif t == WAIT:
            assert arg >= 0
            # the count is in whole slabs: every slab in flight must be fully issued
            assert all(parts_seen[x][0] == parts_seen[x][1] for x in in_flight), "wait with a half-issued slab"
            waits.append((len(in_flight), arg))
            while len(in_flight) > arg:
                complete.add(in_flight.pop(0))
        elif t == WAIT_LDS:
            written_done |= written_pending
            written_pending.clear()
            for s in list(slot_reads):
                slot_reads[s] = "done"
        elif t == BARRIER:
            barriers += 1
            visible |= complete
            visible |= written_done
            for s in list(slot_reads):
                if slot_reads[s] == "done":
                    del slot_reads[s]
        elif t == COMPUTE:
            assert slot_slab.get(slot) == slab, f"slot {slot} holds {slot_slab.get(slot)}, not slab {slab}"
            assert slab in visible, f"RAW: slab {slab} read before it landed and was published"
            slot_reads[slot] = "read"
            computed.append((slab, arg))
        else:
            raise AssertionError(f"unknown event {t}")
    want = [(k, s) for k in range(numK) for s in range(ksteps)]
    assert computed == want, "every k-step of every slab, once, in ascending k"
    return barriers, waits


@pytest.mark.parametrize("kernel", [lg.GEMM_KERNEL_VALU_RING, lg.GEMM_KERNEL_MFMA_RING])
@pytest.mark.parametrize("S", [1, 2, 3, 4, 5])
# code: 0 = each slab's copy issued whole at its first k-step; 1 = one part per k-step;
# c >= 2 = c - 1 parts, the first right after the barrier that frees the slot
@pytest.mark.parametrize("ksteps,spread", [(2, 0), (4, 0), (8, 0), (2, 1), (4, 1), (8, 1),
                                           (2, 2), (4, 2), (4, 3), (8, 2), (8, 3), (8, 5)])
def test_ring_protocol(kernel, S, ksteps, spread):
    for numK in list(range(0, 12)) + [33, 40]:
        ev = lg.gemm_schedule(kernel, S, numK, ksteps + 16 * spread)
        assert ev is not None
        barriers, waits = simulate(ev, S, numK, ksteps, staged=False)
        if numK == 0:
            assert ev == []
            continue
        issues = [e for e in ev if e[0] == ISSUE and (e[3] & 0xff) == 0]
        assert [e[1] for e in issues] == list(range(numK))
        assert all(e[2] == e[1] % S for e in issues), "ring slot = slab mod nStage"
        if S == 1:
            assert barriers == 2 * numK, "single buffer: two barriers per slab"
        else:
            assert barriers == numK, "ring: one barrier per slab"
            # prologue: min(S-1, numK) copies before the first wait
            first_wait = next(i for i, e in enumerate(ev) if e[0] == WAIT)
            assert sum(1 for e in ev[:first_wait] if e[0] == ISSUE and (e[3] & 0xff) == 0) == min(S - 1, numK)
            # wait for the oldest: in steady state S-2 slabs stay in flight
            if numK >= S + 1:
                assert max(a for _, a in waits) == S - 2
            # while copies are still being issued, a wait leaves exactly the newer slabs
            # in flight; only the last S-1 slabs (nothing left to issue) wait for all
            for i, (inflight, allowed) in enumerate(waits):
                assert allowed <= max(0, inflight - 1)
                if i + (S - 1) < len(waits):
                    assert allowed == max(0, inflight - 1)


@pytest.mark.parametrize("kernel", [lg.GEMM_KERNEL_VALU_STAGED, lg.GEMM_KERNEL_MFMA_STAGED])
@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("ksteps", [2, 4])
def test_staged_protocol(kernel, S, ksteps):
    for numK in list(range(0, 10)) + [33]:
        ev = lg.gemm_schedule(kernel, S, numK, ksteps)
        barriers, _ = simulate(ev, S, numK, ksteps, staged=True)
        if numK:
            assert barriers == (2 * numK if S == 1 else numK)
            loads = [e[1] for e in ev if e[0] == ISSUE]
            assert loads == list(range(numK))
        if S == 2 and numK >= 2:
            # the global load of slab k+1 is issued before slab k is computed
            first_compute = {}
            issue_pos = {}
            for i, e in enumerate(ev):
                if e[0] == ISSUE:
                    issue_pos[e[1]] = i
                if e[0] == COMPUTE and e[1] not in first_compute:
                    first_compute[e[1]] = i
            for k in range(numK - 1):
                assert issue_pos[k + 1] < first_compute[k] + 2 * ksteps


def test_bad_arguments():
    assert lg.gemm_schedule(lg.GEMM_KERNEL_MFMA_RING, 0, 4, 4) is None
    assert lg.gemm_schedule(lg.GEMM_KERNEL_MFMA_RING, 6, 4, 4) is None
    assert lg.gemm_schedule(lg.GEMM_KERNEL_MFMA_STAGED, 3, 4, 4) is None
    assert lg.gemm_schedule(lg.GEMM_KERNEL_MFMA_RING, 2, 4, 3) is None
    assert lg.gemm_schedule(lg.GEMM_KERNEL_MFMA_RING, 2, 4, 2 + 16 * 4) is None   # 3 parts of 2 k-steps
    assert lg.gemm_schedule(lg.GEMM_KERNEL_MFMA_STAGED, 2, 4, 4 + 16) is None
    assert lg.gemm_schedule(99, 2, 4, 4) is None


def _planted(events, kind):
    """Corrupt a correct schedule the way a plausible bug would."""
    ev = list(events)
    if kind == "no_barrier":
        i = [j for j, e in enumerate(ev) if e[0] == BARRIER][1]
        del ev[i]
    elif kind == "wait_too_little":
        ev = [(t, s, sl, a + 1) if t == WAIT else (t, s, sl, a) for (t, s, sl, a) in ev]
    elif kind == "wrong_slot":
        for j, e in enumerate(ev):
            if e[0] == ISSUE and e[1] == 2:
                ev[j] = (ISSUE, 2, (e[2] + 1) % 3, 0)
                break
    elif kind == "no_wait_lds":
        ev = [e for e in ev if e[0] != WAIT_LDS]
    elif kind == "late_part":
        # move the second part of slab 3's copy behind the next wait
        j = next(j for j, e in enumerate(ev) if e[0] == ISSUE and e[1] == 3 and (e[3] & 0xff) == 1)
        part = ev.pop(j)
        w = next(k for k in range(j, len(ev)) if ev[k][0] == WAIT)
        ev.insert(w + 1, part)
    return ev


@pytest.mark.parametrize("code", [1, 3])
@pytest.mark.parametrize("kind", ["no_barrier", "wait_too_little", "wrong_slot", "no_wait_lds", "late_part"])
def test_simulator_catches_planted_bugs(kind, code):
    ev = lg.gemm_schedule(lg.GEMM_KERNEL_MFMA_RING, 3, 8, 4 + 16 * code)
    simulate(ev, 3, 8, 4, staged=False)
    with pytest.raises(AssertionError):
        simulate(_planted(ev, kind), 3, 8, 4, staged=False)
