"""Oracle: two-slot schedule of the streamed stack, and a hazard checker.

Slot rule ([Jul] "Slot Tracking: i%2 + Dynamic Correction"): every block has a
hook, and the hooks form a ring (block i follows block i-1 mod n).  A step of
block h reads the slot into which the hook before it in the ring last
prefetched; while that hook has prefetched nothing yet, it reads slot h mod 2.
Each step prefetches the next block of the ring into the other slot while its
own block computes ([Jul] "How It Works"; [Aug] section 3).  For an odd
block count the plain parity h mod 2 would send the head back into the slot the
tail is reading; following the predecessor's prefetch is what keeps the two
slots alternating across the pass boundary.

Readings where the pages are silent:

* the first block goes into slot 0 before the first step ([Doc] "Pre-service
  transaction boundary": the initial prefetch completes during setup);
* the very last step of a run prefetches nothing;
* hook state does not persist from one run to the next.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class SlotEvent:
    step: int
    pass_: int
    block: int
    read_slot: int
    prefetch_block: int   # -1 on the last step
    prefetch_slot: int    # -1 on the last step


def simulate_hooks(n: int, passes: int, n_resident: int = 0):
    """The per-step slot trace produced by n circularly linked hooks over ``passes`` passes.

    With ``n_resident`` = R > 0 (the pages' resident-layer setting, [Doc]
    "Validation coverage" and the smoke-test setup that names
    dlo_resident_layers), the first R blocks of the stack stay in device memory:
    their steps read no slot (-1) and prefetch nothing.  The other n - R blocks
    carry the hooks, linked circularly among themselves, and stream through the
    two slots by the same rule; the last streamed step of the run prefetches
    nothing.
    """
    if n < 1 or passes < 1 or not 0 <= n_resident <= n:
        raise ValueError("n, passes >= 1 and 0 <= n_resident <= n required")
    m = n - n_resident
    last_prefetch = {}          # hook -> slot of its latest prefetch
    streamed_total = m * passes
    u = 0
    trace = []
    for t in range(n * passes):
        p, i = divmod(t, n)
        if i < n_resident:
            trace.append(SlotEvent(t, p, i, -1, -1, -1))
            continue
        h = i - n_resident
        read = last_prefetch.get((h - 1) % m, h % 2)
        if u + 1 < streamed_total:
            nxt, ps = n_resident + (h + 1) % m, 1 - read
            last_prefetch[h] = ps
        else:
            nxt, ps = -1, -1
        trace.append(SlotEvent(t, p, i, read, nxt, ps))
        u += 1
    return trace


def simulate_static_rule(n: int, passes: int):
    """Negative control: slots fixed at i % 2 with no correction.

    Each hook reads slot i % 2 and prefetches the next block into that block's
    own fixed slot ((i+1) mod n) % 2.  For odd n the tail (slot 0) prefetches
    the head into slot 0, the slot it is itself reading -- the collision that
    the correction exists to prevent.
    """
    total = n * passes
    trace = []
    for t in range(total):
        p, i = divmod(t, n)
        if t + 1 < total:
            nxt = (i + 1) % n
            ps = nxt % 2
        else:
            nxt, ps = -1, -1
        trace.append(SlotEvent(t, p, i, i % 2, nxt, ps))
    return trace


def trace_hazards(trace, n_slots: int = 2, first_block: int = 0, first_slot: int = 0):
    """Step-level hazards of a trace; an empty list means the trace is safe.

    * a step must read a slot that holds its block (the most recent copy into
      that slot carried this block);
    * a step must not prefetch into the slot it is reading (the copy would
      overwrite weights that are being read);
    * only ``n_slots`` slots may be used.
    """
    holds = {first_slot: first_block}
    problems = []
    for ev in trace:
        if ev.read_slot == -1 and ev.prefetch_block == -1:
            continue   # a resident block: reads no slot
        if not (0 <= ev.read_slot < n_slots):
            problems.append((ev.step, "slot out of range"))
        if holds.get(ev.read_slot) != ev.block:
            problems.append((ev.step, f"reads slot {ev.read_slot} holding block "
                                      f"{holds.get(ev.read_slot)} instead of {ev.block}"))
        if ev.prefetch_block >= 0:
            if ev.prefetch_slot == ev.read_slot:
                problems.append((ev.step, "prefetch overwrites the slot being read"))
            if not (0 <= ev.prefetch_slot < n_slots):
                problems.append((ev.step, "prefetch slot out of range"))
            holds[ev.prefetch_slot] = ev.prefetch_block
    return problems


# ---------------------------------------------------------------------------
# Happens-before checker for a program of stream operations
# ---------------------------------------------------------------------------
#
# A program is the host-order list of operations that a scheduler enqueues:
#   ("copy", stream, block, slot)            writes a slot
#   ("compute", stream, block, slot, step)   reads a slot
#   ("record", stream, event)                event := everything enqueued so far on stream
#   ("wait", stream, event)                  later work on stream waits for the event's
#                                            most recent record (as of this host point)
# Operations on one stream run in order.  The checker assigns vector clocks and
# then demands, for every slot, that each (copy, compute) pair touching it is
# ordered one way or the other, and that the last copy ordered before a compute
# carried the compute's block.


def _vector_clocks(program):
    streams = sorted({op[1] for op in program})
    sidx = {s: i for i, s in enumerate(streams)}
    clock = {s: [0] * len(streams) for s in streams}
    events = {}
    stamps = []   # per op: (stream index, position on stream, vector clock copy) or None
    for op in program:
        kind, s = op[0], op[1]
        vc = clock[s]
        if kind == "record":
            events[op[2]] = list(vc)
            stamps.append(None)
        elif kind == "wait":
            ev = events.get(op[2])
            if ev is not None:
                clock[s] = [max(a, b) for a, b in zip(vc, ev)]
            stamps.append(None)
        elif kind in ("copy", "compute"):
            vc[sidx[s]] += 1
            stamps.append((sidx[s], vc[sidx[s]], list(vc)))
        else:
            raise ValueError(f"unknown op {kind}")
    return stamps


def program_hazards(program, initial=None):
    """Ordering hazards of a stream program; an empty list means it is race-free.

    ``initial`` maps slot -> block already present before the program starts.
    """
    stamps = _vector_clocks(program)

    def hb(a, b):   # op a happens before op b
        sa, sb = stamps[a], stamps[b]
        return sa[1] <= sb[2][sa[0]] and a != b

    copies, computes = [], []
    for i, op in enumerate(program):
        if op[0] == "copy":
            copies.append(i)
        elif op[0] == "compute":
            computes.append(i)
    problems = []
    for kc in computes:
        _, _, block, slot, step = program[kc]
        if slot == -1:
            continue   # a resident block: reads no slot
        before = []
        for c in copies:
            if program[c][3] != slot:
                continue
            if hb(c, kc):
                before.append(c)
            elif not hb(kc, c):
                problems.append((step, f"copy of block {program[c][2]} into slot {slot} "
                                       f"races with the compute reading it"))
        if before:
            # the latest of the ordered copies: the one every other ordered copy precedes
            last = [c for c in before if all(c == o or hb(o, c) for o in before)]
            if len(last) != 1:
                problems.append((step, "copies into one slot are not totally ordered"))
                continue
            if program[last[0]][2] != block:
                problems.append((step, f"reads slot {slot} holding block {program[last[0]][2]}"))
        else:
            held = (initial or {}).get(slot)
            if held != block:
                problems.append((step, f"reads slot {slot} before any copy of block {block}"))
    return problems
