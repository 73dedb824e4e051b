"""Pins for oracle.schedule: hook rule, hazards, negative controls, the happens-before checker."""
import os

import pytest

from oracle import schedule as sc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_trace_n3():
    want = []
    for line in open(os.path.join(GOLDEN, "slot_trace_n3_p2.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            want.append(tuple(int(v) for v in line.split()))
    got = [(e.step, e.pass_, e.block, e.read_slot, e.prefetch_block, e.prefetch_slot)
           for e in sc.simulate_hooks(3, 2)]
    assert got == want


@pytest.mark.parametrize("passes", [1, 2, 3, 4, 5])
def test_closed_form_and_no_hazards(passes):
    for n in range(1, 301):
        tr = sc.simulate_hooks(n, passes)
        assert len(tr) == n * passes
        for e in tr:
            assert e.read_slot == e.step % 2           # slot(t) = t mod 2
            assert (e.pass_, e.block) == divmod(e.step, n)
            if e.step + 1 < n * passes:
                assert e.prefetch_block == (e.block + 1) % n
                assert e.prefetch_slot == 1 - e.read_slot
            else:
                assert (e.prefetch_block, e.prefetch_slot) == (-1, -1)
        assert sc.trace_hazards(tr) == []


def test_hand_worked_trace_n3_one_resident_layer():
    want = []
    for line in open(os.path.join(GOLDEN, "slot_trace_n3_r1_p2.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            want.append(tuple(int(v) for v in line.split()))
    got = [(e.step, e.pass_, e.block, e.read_slot, e.prefetch_block, e.prefetch_slot)
           for e in sc.simulate_hooks(3, 2, n_resident=1)]
    assert got == want


@pytest.mark.parametrize("passes", [1, 2, 3])
def test_resident_layers_reduce_to_the_plain_rule(passes):
    # the streamed steps of an n-block stack with R resident layers are exactly the
    # trace of an (n - R)-block stack, shifted by R; resident steps read nothing
    for n in range(1, 41):
        for R in range(0, n + 1):
            tr = sc.simulate_hooks(n, passes, n_resident=R)
            assert len(tr) == n * passes
            res = [e for e in tr if e.block < R]
            assert all((e.read_slot, e.prefetch_block, e.prefetch_slot) == (-1, -1, -1) for e in res)
            streamed = [e for e in tr if e.block >= R]
            if R == n:
                assert not streamed
                continue
            ref = sc.simulate_hooks(n - R, passes)
            assert len(streamed) == len(ref)
            for u, (e, r) in enumerate(zip(streamed, ref)):
                assert e.read_slot == r.read_slot == u % 2
                assert e.block == r.block + R
                assert e.prefetch_slot == r.prefetch_slot
                assert e.prefetch_block == (r.prefetch_block + R if r.prefetch_block >= 0 else -1)
            assert sc.trace_hazards(tr, first_block=R) == []


def test_resident_layer_count_is_validated():
    for bad in (-1, 4):
        with pytest.raises(ValueError):
            sc.simulate_hooks(3, 1, n_resident=bad)


def test_static_rule_fails_for_odd_counts():
    # negative control: without the correction the tail -> head prefetch of an odd stack
    # lands in the slot the tail is reading
    for n in (1, 3, 5, 127):
        probs = sc.trace_hazards(sc.simulate_static_rule(n, 2))
        assert probs, n
        assert any("overwrites" in p[1] for p in probs)
    # even counts are fine with the static rule
    for n in (2, 8, 72, 128):
        assert sc.trace_hazards(sc.simulate_static_rule(n, 3)) == []
    # a single pass of an odd stack never wraps, so it is safe too
    assert sc.trace_hazards(sc.simulate_static_rule(3, 1)) == []


def _two_slot_program(n, passes, drop_war=False, drop_raw=False, swap_slot_at=None):
    """Hand-written program for the copy/compute event scheme (used to pin the checker)."""
    prog = [("copy", "copy", 0, 0), ("record", "copy", "copied0")]
    total = n * passes
    for t in range(total):
        b, s = t % n, t % 2
        if swap_slot_at == t:
            s = 1 - s
        if t + 1 < total:
            nb, ns = (t + 1) % n, (t + 1) % 2
            if t >= 1 and not drop_war:
                prog.append(("wait", "copy", f"computed{ns}"))
            prog.append(("copy", "copy", nb, ns))
            prog.append(("record", "copy", f"copied{ns}"))
        if not drop_raw:
            prog.append(("wait", "compute", f"copied{s}"))
        prog.append(("compute", "compute", b, s, t))
        prog.append(("record", "compute", f"computed{s}"))
    return prog


def test_checker_accepts_correct_program():
    for n in (1, 2, 3, 8):
        assert sc.program_hazards(_two_slot_program(n, 3)) == []


def test_checker_rejects_missing_waits_and_wrong_slots():
    assert sc.program_hazards(_two_slot_program(3, 2, drop_war=True))
    assert sc.program_hazards(_two_slot_program(3, 2, drop_raw=True))
    assert sc.program_hazards(_two_slot_program(4, 2, swap_slot_at=5))


def test_checker_single_stream_is_always_ordered():
    prog = [("copy", "s", 0, 0), ("compute", "s", 0, 0, 0), ("copy", "s", 1, 0),
            ("compute", "s", 1, 0, 1)]
    assert sc.program_hazards(prog) == []
    prog_bad = [("copy", "s", 0, 0), ("copy", "s", 1, 0), ("compute", "s", 0, 0, 0)]
    assert sc.program_hazards(prog_bad)
