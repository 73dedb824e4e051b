"""libdlo host logic on the CPU: exports, plan, pack, schedule and fail-closed errors.

Everything here runs without a GPU: the plan, the pageable host store, the
schedule program and every validation path return before any HIP call.  The
plan, the packed bytes and the schedule are compared with the oracle's own,
independently written, implementation.
"""
import ctypes
import os
import random
import re

import numpy as np
import pytest

import synth
import layerwise_weight_streaming_amd as dlo
from oracle import plan as op
from oracle import schedule as sc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(dlo.LIB_PATH):
        from layerwise_weight_streaming_amd import _build
        _build.build()
    dlo.lib()


def _header_functions():
    src = open(os.path.join(ROOT, "include", "dlo.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dlo_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_function_is_exported_and_bound():
    names = _header_functions()
    assert len(names) >= 25
    L = ctypes.CDLL(dlo.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == dlo.EXPORTED


def test_schema_matches_input_generator():
    for d in (256, 1024, 5120):
        assert dlo.block_schema(d) == [(n, dt, int(np.prod(s))) for n, dt, s in synth.block_schema(d)]


def _dit_blocks(w, n=None):
    n = w.n_blocks if n is None else n
    return [(w.width(b), w.heads(b), [(nm, dt, int(np.prod(s))) for nm, dt, s in synth.block_schema(w.width(b))])
            for b in range(n)]


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_plan_matches_oracle_on_workloads(name):
    w = synth.WORKLOADS[name]
    blocks = _dit_blocks(w, min(w.n_blocks, 7))
    p = dlo.Plan(blocks, w.k)
    plans, slot = op.plan_stack([b[2] for b in blocks], w.k)
    assert p.slot_bytes == slot
    for b, bp in enumerate(plans):
        info = p.block_info(b)
        assert info["is_dit"]
        assert info["extent"] == bp.extent
        assert info["dtype"] == [g.dtype for g in bp.groups]
        assert info["numel"] == [g.numel for g in bp.groups]
        assert info["shard"] == [g.shard for g in bp.groups]
        assert info["region"] == [g.region for g in bp.groups]
        assert info["copy_bytes"] == sum(bp.region_bytes(g) for g in range(len(bp.groups)))
        for i in range(16):
            assert p.param_offset(b, i) == bp.param_byte_offset(i)


def _random_params(rng, n):
    out = []
    for i in range(n):
        dt = rng.choice(["bf16", "f32", "fp8"])
        numel = rng.choice([0, 1, 3, 7, 64, 255, rng.randint(0, 3000)])
        if dt == "bf16":
            a = np.frombuffer(rng.randbytes(2 * numel), dtype=np.uint16).copy()
        elif dt == "fp8":
            a = np.frombuffer(rng.randbytes(numel), dtype=np.uint8).copy()
        else:
            a = np.array([rng.uniform(-3, 3) for _ in range(numel)], dtype=np.float32)
        out.append((f"p{i}", dt, a))
    return out


def test_plan_and_pack_match_oracle_randomised():
    rng = random.Random(7)
    for trial in range(60):
        nb = rng.randint(1, 4)
        k = rng.randint(1, 8)
        params = [_random_params(rng, rng.randint(1, 5)) for _ in range(nb)]
        blocks = [(256, 4, ps) for ps in params]
        p = dlo.Plan(blocks, k)
        st = dlo.HostStore(p, pinned=False)
        assert not st.complete
        st.pack(0, blocks)
        assert st.complete
        for b, ps in enumerate(params):
            bp = op.plan_block(op.specs_of(ps), k)
            info = p.block_info(b)
            assert info["extent"] == bp.extent and info["region"] == [g.region for g in bp.groups]
            shards = op.pack_block(ps, bp)
            for g in range(len(bp.groups)):
                for r in range(k):
                    assert st.shard(b, g, r).tobytes() == shards[g][r].tobytes(), (trial, b, g, r)


def test_pack_tiny_workload_matches_oracle_bytes():
    w = synth.WORKLOADS["tiny"]
    stack = synth.make_stack(w, seed=3)
    blocks = [(w.width(b), w.heads(b), ps) for b, ps in enumerate(stack.blocks)]
    p = dlo.Plan(blocks, w.k)
    st = dlo.HostStore(p, pinned=False)
    st.pack(0, blocks[:1])
    st.pack(1, blocks[1:])
    for b, ps in enumerate(stack.blocks):
        bp = op.plan_block(op.specs_of(ps), w.k)
        sh = op.pack_block(ps, bp)
        for g in range(2):
            for r in range(w.k):
                assert st.shard(b, g, r).tobytes() == sh[g][r].tobytes()
        # reassembled region = the slot image a placement produces
        for g, (off, buf) in enumerate(op.slot_regions(bp, sh)):
            assert off == p.block_info(b)["region"][g]


@pytest.mark.parametrize("passes", [1, 2, 3, 4])
def test_schedule_program_is_race_free_and_follows_the_hook_rule(passes):
    for n in list(range(1, 25)) + [72, 127, 128]:
        blocks = [(256, 4, [("w", "bf16", 10)]) for _ in range(n)]
        prog = dlo.Plan(blocks, 2).schedule(passes)
        assert sc.program_hazards(prog) == [], (n, passes)
        computes = [o for o in prog if o[0] == "compute"]
        ref = sc.simulate_hooks(n, passes)
        assert [(o[2], o[3], o[4]) for o in computes] == [(e.block, e.read_slot, e.step) for e in ref]
        copies = [o for o in prog if o[0] == "copy"]
        want = [(0, 0)] + [(e.prefetch_block, e.prefetch_slot) for e in ref if e.prefetch_block >= 0]
        assert [(o[2], o[3]) for o in copies] == want
        # two slots only
        assert {o[3] for o in prog if o[0] in ("copy", "compute")} <= {0, 1}


@pytest.mark.parametrize("passes", [1, 2, 3])
def test_schedule_with_resident_layers_is_race_free_and_follows_the_oracle(passes):
    for n in list(range(1, 13)) + [72, 127]:
        blocks = [(256, 4, [("w", "bf16", 10)]) for _ in range(n)]
        plan = dlo.Plan(blocks, 2)
        for R in sorted({0, 1, n // 2, n - 1, n}):
            prog = plan.schedule(passes, n_resident=R)
            ref = sc.simulate_hooks(n, passes, n_resident=R)
            computes = [o for o in prog if o[0] == "compute"]
            assert [(o[2], o[3], o[4]) for o in computes] == [(e.block, e.read_slot, e.step) for e in ref]
            copies = [o for o in prog if o[0] == "copy"]
            if R == n:
                assert len(prog) == n * passes and not copies
                continue
            assert sc.program_hazards(prog) == [], (n, R, passes)
            want = [(R, 0)] + [(e.prefetch_block, e.prefetch_slot) for e in ref if e.prefetch_block >= 0]
            assert [(o[2], o[3]) for o in copies] == want
            # resident blocks are never copied and never wait
            assert all(o[2] >= R for o in copies)
            assert all(o[3] == -1 for o in computes if o[2] < R)


def test_schedule_resident_count_out_of_range():
    plan = dlo.Plan([(256, 4, [("w", "bf16", 10)]) for _ in range(3)], 2)
    for bad in (-1, 4):
        assert _status(plan.schedule, 1, bad) == "DLO_E_ARG"


def test_schedule_negative_control_detected():
    # dropping the copy stream's wait on the previous reader must be flagged by the checker
    blocks = [(256, 4, [("w", "bf16", 10)]) for _ in range(3)]
    prog = dlo.Plan(blocks, 2).schedule(2)
    broken = [o for o in prog if not (o[0] == "wait" and o[1] == "copy" and o[2].startswith("computed"))]
    assert sc.program_hazards(broken)


# ---------------------------------------------------------------------------
# fail-closed validation (no GPU needed: every check runs before any HIP call)
# ---------------------------------------------------------------------------

def _status(fn, *a, **k):
    with pytest.raises(dlo.DLOError) as ei:
        fn(*a, **k)
    return ei.value.status


def test_plan_errors():
    good = [("w", "bf16", 4)]
    assert _status(dlo.Plan, [(256, 4, good)], 0) == "DLO_E_ARG"
    assert _status(dlo.Plan, [], 2) == "DLO_E_ARG"
    assert _status(dlo.Plan, [(256, 4, [("w", 7, 4)])], 2) == "DLO_E_ARG"
    assert _status(dlo.Plan, [(256, 4, [("w", "f32", -1)])], 2) == "DLO_E_ARG"
    out = ctypes.c_void_p(123)
    assert dlo.lib().dlo_plan_blocks(None, 1, 2, ctypes.byref(out)) == -1 and out.value is None
    p = dlo.Plan([(256, 4, good)], 2)
    assert _status(p.block_info, 5) == "DLO_E_ARG"
    assert _status(p.param_offset, 0, 3) == "DLO_E_ARG"
    assert _status(p.schedule, 0) == "DLO_E_ARG"
    assert "passes" in dlo.last_error()


def test_pack_errors():
    a = np.arange(6, dtype=np.float32)
    p = dlo.Plan([(256, 4, [("a", "f32", 6)]), (256, 4, [("b", "f32", 6)])], 4)
    st = dlo.HostStore(p, pinned=False)
    assert _status(st.pack, 0, [(256, 4, [("x", "f32", a)])]) == "DLO_E_PLAN_MISMATCH"  # name
    assert _status(st.pack, 0, [(256, 4, [("a", "bf16", a.view(np.uint16)[:6])])]) == "DLO_E_PLAN_MISMATCH"
    assert _status(st.pack, 0, [(256, 4, [("a", "f32", a[:5])])]) == "DLO_E_PLAN_MISMATCH"  # numel
    assert _status(st.pack, 1, [(256, 4, [("a", "f32", a)])]) == "DLO_E_PLAN_MISMATCH"  # wrong block
    assert _status(st.pack, 2, [(256, 4, [("b", "f32", a)])]) == "DLO_E_ARG"  # range
    assert _status(st.pack, 0, [(256, 4, [("a", "f32", 6)])]) == "DLO_E_ARG"  # no source
    assert not st.complete
    st.pack(0, [(256, 4, [("a", "f32", a)])])
    assert not st.complete


def test_pinned_store_without_device_fails_closed():
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present: pinned allocation would succeed")
    except ImportError:
        pass
    p = dlo.Plan([(256, 4, [("a", "f32", 6)])], 2)
    out = ctypes.c_void_p(77)
    rc = dlo.lib().dlo_host_store_create(p.h, 0, ctypes.byref(out))
    assert rc == -3 and out.value is None
    assert "hipHostMalloc" in dlo.last_error()


def _tiny_plan_and_store(n=3, d=256, heads=4, k=2):
    blocks = [(d, heads, [(nm, dt, int(np.prod(s))) for nm, dt, s in synth.block_schema(d)])
              for _ in range(n)]
    p = dlo.Plan(blocks, k)
    st = dlo.HostStore(p, pinned=False)
    filled = [(d, heads, [(nm, dt, np.zeros(int(np.prod(s)), dtype=np.uint16 if dt == "bf16" else np.float32))
                          for nm, dt, s in synth.block_schema(d)]) for _ in range(n)]
    st.pack(0, filled)
    return p, st


def _args(p, **over):
    kw = dict(x=0x1000, x_row_stride=256, cond=0x2000, workspace=0x3000,
              workspace_bytes=p.workspace_bytes(64), compute_stream=0x10, copy_stream=0x20,
              tokens=64, passes=2, slots=(0x100000, 0x100000 + p.slot_bytes), slot_bytes=p.slot_bytes)
    kw.update(over)
    return kw


def test_forward_validation_errors():
    p, st = _tiny_plan_and_store()
    F = lambda **o: dlo.forward_stack(p, st, **_args(p, **o))
    assert _status(F, tokens=0) == "DLO_E_ARG"
    assert _status(F, passes=0) == "DLO_E_ARG"
    assert _status(F, x=0) == "DLO_E_ARG"
    assert _status(F, copy_stream=0x10) == "DLO_E_ARG"          # aliased streams
    assert _status(F, copy_stream=0) == "DLO_E_ARG"
    assert _status(F, x_row_stride=128) == "DLO_E_ARG"
    assert _status(F, x_row_stride=258) == "DLO_E_ARG"          # rows not 16-B aligned
    assert _status(F, x=0x1004) == "DLO_E_ARG"                  # x not 16-B aligned
    assert _status(F, workspace_bytes=100) == "DLO_E_WORKSPACE"
    assert _status(F, slot_bytes=p.slot_bytes - 1) == "DLO_E_SLOT_SMALL"
    assert _status(F, slots=(0x100000, 0x100000 + 256)) == "DLO_E_ARG"   # overlapping slots
    assert _status(F, slots=(0, 0x100000)) == "DLO_E_ARG"
    assert _status(F, flags=64) == "DLO_E_ARG"
    assert _status(F, flags=32) == "DLO_E_ARG"
    # DLO_ASYNC_ENQUEUE hands the run to a thread that dlo_run_enqueued joins: a handle is required
    assert _status(F, flags=dlo.ASYNC_ENQUEUE, want_run=False) == "DLO_E_ARG"
    assert _status(F, batch=-1) == "DLO_E_ARG"
    assert _status(F, batch=2, cond_stride=p.block_info(0)["d_model"] - 1) == "DLO_E_ARG"
    assert _status(F, flags=dlo.RESIDENT) == "DLO_E_ARG"        # no resident pointers
    assert _status(F, n_resident=-1) == "DLO_E_ARG"
    assert _status(F, n_resident=4) == "DLO_E_ARG"              # more than the 3 blocks
    assert _status(F, n_resident=1) == "DLO_E_ARG"              # resident layers need pointers
    assert _status(F, n_resident=2, resident_blocks=[0x200000, 0]) == "DLO_E_ARG"  # NULL entry
    # a store made by another plan is the analogue of double sharding: rejected
    p2, st2 = _tiny_plan_and_store()
    assert _status(lambda: dlo.forward_stack(p, st2, **_args(p))) == "DLO_E_PLAN_MISMATCH"
    # an incompletely packed store
    st3 = dlo.HostStore(p, pinned=False)
    assert _status(lambda: dlo.forward_stack(p, st3, **_args(p))) == "DLO_E_STATE"


def test_forward_rejects_unsupported_blocks():
    # head dim 32
    p, st = _tiny_plan_and_store(heads=8)
    assert _status(lambda: dlo.forward_stack(p, st, **_args(p))) == "DLO_E_UNSUPPORTED"
    # width not a multiple of 256
    blocks = [(320, 5, [(nm, dt, int(np.prod(s))) for nm, dt, s in synth.block_schema(320)])]
    p = dlo.Plan(blocks, 2)
    st = dlo.HostStore(p, pinned=False)
    st.pack(0, [(320, 5, [(nm, dt, np.zeros(int(np.prod(s)), dtype=np.uint16 if dt == "bf16" else np.float32))
                          for nm, dt, s in synth.block_schema(320)])])
    assert _status(lambda: dlo.forward_stack(p, st, **_args(p, x_row_stride=320))) == "DLO_E_UNSUPPORTED"
    # a block that is not the DiT schema
    p = dlo.Plan([(256, 4, [("w", "bf16", 8)])], 2)
    st = dlo.HostStore(p, pinned=False)
    st.pack(0, [(256, 4, [("w", "bf16", np.zeros(8, np.uint16))])])
    assert _status(lambda: dlo.forward_stack(p, st, **_args(p))) == "DLO_E_UNSUPPORTED"


def test_op_validation_errors():
    assert _status(dlo.op_gemm, 1, 64, 1, 64, 10, 100, 64, 1, 0, 1, 100, 0, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_gemm, 1, 64, 1, 64, 10, 256, 60, 1, 0, 1, 256, 0, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_gemm, 1, 64, 1, 64, 10, 256, 64, 1, 0, 1, 256, 2, 0) == "DLO_E_ARG"  # no gate
    # epilogue stores are 8/16-B vectors: C 16-B aligned, ldc % 4 == 0; bias and gate
    # are read as fp32 scalars, 4-B aligned (as packed in a slot)
    assert _status(dlo.op_gemm, 16, 64, 16, 64, 10, 256, 64, 16, 16, 0x1008, 256, 2, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_gemm, 16, 64, 16, 64, 10, 256, 64, 16, 16, 0x1000, 258, 2, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_gemm, 16, 64, 16, 64, 10, 256, 64, 0x1002, 16, 0x1000, 256, 0, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_gemm, 16, 64, 16, 64, 10, 256, 64, 16, 0x1006, 0x1000, 256, 2, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_attention, 16, 3 * 4 * 32, 16, 64, 10, 4, 32, 16, 128, 0) == "DLO_E_UNSUPPORTED"
    # V^T row stride below T rounded up to 64, and misaligned V^T
    assert _status(dlo.op_attention, 16, 3 * 4 * 64, 16, 56, 10, 4, 64, 16, 256, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_attention, 16, 3 * 4 * 64, 0x1008, 64, 10, 4, 64, 16, 256, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_attention, 16, 3 * 4 * 64, 0, 64, 10, 4, 64, 16, 256, 0) == "DLO_E_ARG"
    assert _status(dlo.op_v_transpose, 16, 3 * 96, 10, 96, 16, 64, 0) == "DLO_E_UNSUPPORTED"   # d % 64
    assert _status(dlo.op_v_transpose, 16, 3 * 128, 65, 128, 16, 64, 0) == "DLO_E_UNSUPPORTED"  # ldvt < 128
    assert _status(dlo.op_v_transpose, 16, 3 * 128, 10, 128, 0x1008, 64, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_v_transpose, 16, 3 * 128 - 8, 10, 128, 16, 64, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_ln_modulate, 1, 300, 4, 300, 1, 1, 1, 1, 1, 1, 0) == "DLO_E_UNSUPPORTED"
    # x rows are read as float4 (16-B aligned x, ldx % 4 == 0), out written as 4 bf16
    assert _status(dlo.op_ln_modulate, 16, 258, 4, 256, 16, 16, 16, 16, 16, 16, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_ln_modulate, 0x1004, 256, 4, 256, 16, 16, 16, 16, 16, 16, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_ln_modulate, 16, 256, 4, 256, 16, 16, 16, 16, 16, 0x1002, 0) == "DLO_E_UNSUPPORTED"
    assert _status(dlo.op_digest, 1, [3], [8], 1, 0) == "DLO_E_ARG"


# ---------------------------------------------------------------------------
# FP8 weight groups
# ---------------------------------------------------------------------------

def _bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_quantizer_matches_oracle_byte_for_byte():
    from oracle import fp8
    rng = np.random.default_rng(5)
    cases = [
        _bf16(rng.normal(0, 0.02, 5000)),
        _bf16(rng.normal(0, 0.5, 3_000_001)),                                    # threaded path
        _bf16(rng.normal(0, 1.0, 4096) * np.exp(rng.uniform(-12, 12, 4096))),   # wide dynamic range
        _bf16(np.array([0.0, -0.0, 1e-30, -3e-38, 448.0, 1.0, -1.0, 65504.0])),
        np.frombuffer(rng.bytes(2 * 3000), dtype=np.uint16).copy(),              # any bf16 bits
        np.zeros(17, np.uint16),
        np.zeros(0, np.uint16),
    ]
    for w in cases:
        finite = np.isfinite((w.astype(np.uint32) << 16).view(np.float32))
        if not finite.all():    # weights are finite; NaN/inf bit patterns go separately below
            w = w[finite]
        codes, scale = dlo.quantize_fp8(w)
        ocodes, oscale = fp8.quantize_tensor(w)
        assert scale == oscale
        assert codes.tobytes() == ocodes.tobytes()
    # NaN entries are ignored by the scale and encode as 0x7F
    w = np.concatenate([_bf16(rng.normal(0, 1, 100)), np.array([0x7FC0], np.uint16)])
    codes, scale = dlo.quantize_fp8(w)
    ocodes, oscale = fp8.quantize_tensor(w)
    assert scale == oscale and codes.tobytes() == ocodes.tobytes() and codes[-1] == 0x7F


def test_fp8_schema_matches_the_oracle_block_form():
    from oracle import fp8
    for d in (256, 1024, 5120):
        ps = synth.block_params(0, 0, 256) if d == 256 else None
        sch = dlo.block_schema(d, fp8=True)
        assert len(sch) == 21
        bf = dlo.block_schema(d)
        names = [n for n, _, _ in sch]
        for n, dt, numel in bf:
            i = names.index(n)
            assert sch[i][2] == numel and sch[i][1] == ("fp8" if dt == "bf16" else dt)
            if dt == "bf16":
                assert sch[i + 1] == (n + "_scale", "f32", 1)
        if ps is not None:
            q = fp8.quantize_block(ps)
            assert [(n, dt, int(a.size)) for n, dt, a in q] == sch


def test_fp8_block_plan_pack_and_workspace():
    from oracle import fp8
    d, k = 256, 4
    q = fp8.quantize_block(synth.block_params(1, 0, d))
    p = dlo.Plan([(d, 4, q), (d, 4, synth.block_params(1, 1, d))], k)
    info = p.block_info(0)
    assert info["fp8"] and info["is_dit"] and info["dtype"] == ["fp8", "f32"]
    assert info["numel"] == [18 * d * d, 19 * d + 7]
    assert not p.block_info(1)["fp8"] and p.block_info(1)["is_dit"]
    bp = op.plan_block(op.specs_of(q), k)
    assert info["extent"] == bp.extent and info["region"] == [g.region for g in bp.groups]
    assert info["copy_bytes"] * 2 < p.block_info(1)["copy_bytes"] * 1.01   # about half the bytes
    st = dlo.HostStore(p, pinned=False)
    st.pack(0, [(d, 4, q), (d, 4, synth.block_params(1, 1, d))])
    sh = op.pack_block(q, bp)
    for g in range(2):
        for r in range(k):
            assert st.shard(0, g, r).tobytes() == sh[g][r].tobytes()
    # the workspace grows by the widest FP8 block's four bf16 linear weights and, for the W8A8
    # form, a linear input's E4M3 codes [T, 4d] and row scales [T] (each region
    # 256-B aligned)
    p_bf = dlo.Plan([(d, 4, synth.block_params(1, 1, d))], k)
    for T in (64, 1000):
        al = lambda n: (n + 255) // 256 * 256
        assert p.workspace_bytes(T) - p_bf.workspace_bytes(T) == al(24 * d * d) + al(4 * T * d) + al(4 * T)


def test_kernel_slot_names():
    """One name per timed kernel of a block forward, in launch order, the W8A8 input
    quantisations just before the linears they feed; out of range gives NULL."""
    names = dlo.kernel_names()
    assert len(names) == dlo.KERNELS_PER_BLOCK == len(set(names))
    order = ["dequant_weights", "adaln_gemv", "ln1_modulate", "quant_h", "gemm_qk", "gemm_v_t", "attention",
             "quant_attn", "gemm_out_residual", "ln2_modulate", "quant_h2", "gemm_fc1_gelu", "quant_u",
             "gemm_fc2_residual"]
    assert names == order
    assert dlo.lib().dlo_kernel_name(dlo.KERNELS_PER_BLOCK) is None
    assert dlo.lib().dlo_kernel_name(-1) is None


# ---------------------------------------------------------------------------
# INT8 and MXFP8 weight groups
# ---------------------------------------------------------------------------

def _quant_matrices():
    rng = np.random.default_rng(11)
    a = rng.normal(0, 0.02, (64, 256))
    a[3] = 0.0                                     # zero row / zero blocks
    a[5, 7] = 3.0                                  # outlier
    a[9, 32:64] = 0.0
    b = rng.normal(0, 1.0, (48, 96)) * np.exp(rng.uniform(-14, 14, (48, 96)))   # wide dynamic range
    c = rng.normal(0, 0.5, (2048, 1024))           # the threaded path
    d = (np.frombuffer(rng.bytes(2 * 40 * 64), dtype=np.uint16).reshape(40, 64) & 0x7F7F)  # any finite bits
    e = np.zeros((3, 32))
    return [_bf16(a), _bf16(b), _bf16(c), d.astype(np.uint16), _bf16(e), np.zeros((0, 32), np.uint16)]


def test_int8_quantizer_matches_oracle_byte_for_byte():
    from oracle import quant
    for w in _quant_matrices():
        codes, scales = dlo.quantize_int8(w)
        rc, rs = quant.quantize_int8(w)
        assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32))
        assert np.array_equal(codes, rc)


def test_mxfp8_quantizer_matches_oracle_byte_for_byte():
    from oracle import quant
    for w in _quant_matrices():
        codes, scales = dlo.quantize_mxfp8(w)
        rc, rs = quant.quantize_mxfp8(w)
        assert np.array_equal(scales, rs.T)      # block-major
        assert np.array_equal(codes, rc)
    with pytest.raises(dlo.DLOError):
        dlo.quantize_mxfp8(np.zeros((2, 48), np.uint16))          # columns not a multiple of 32


@pytest.mark.parametrize("form", ["int8", "mxfp8"])
def test_quantised_schema_plan_and_pack(form):
    from oracle import quant
    d, k = 256, 4
    sch = dlo.block_schema(d, form=form)
    q = quant.quantize_block(synth.block_params(1, 0, d), form)
    assert [(n, dt, int(a.size)) for n, dt, a in q] == sch
    # libdlo's own quantizer gives the same block, byte for byte
    ql = dlo.quantize_block(synth.block_params(1, 0, d), form)
    for (n1, d1, a1), (n2, d2, a2) in zip(q, ql):
        assert (n1, d1) == (n2, d2) and np.asarray(a1).tobytes() == np.asarray(a2).tobytes()
    p = dlo.Plan([(d, 4, q), (d, 4, synth.block_params(1, 1, d))], k)
    info = p.block_info(0)
    assert info["form"] == form and p.block_info(1)["form"] == "bf16"
    want_dt = ["i8", "f32"] if form == "int8" else ["fp8", "e8m0", "f32"]
    assert info["dtype"] == want_dt
    bp = op.plan_block(op.specs_of(q), k)
    assert info["extent"] == bp.extent and info["region"] == [g.region for g in bp.groups]
    assert info["numel"] == [g.numel for g in bp.groups]
    st = dlo.HostStore(p, pinned=False)
    st.pack(0, [(d, 4, q), (d, 4, synth.block_params(1, 1, d))])
    sh = op.pack_block(q, bp)
    for g in range(len(bp.groups)):
        for r in range(k):
            assert st.shard(0, g, r).tobytes() == sh[g][r].tobytes()
    # the workspace holds all five dequantised weights (18 d^2 bf16) and the W8A8
    # input's codes [T, 4d] with its scales (INT8 fp32 [T], MXFP8 E8M0 [4d / 32, T64])
    p_bf = dlo.Plan([(d, 4, synth.block_params(1, 1, d))], k)
    al = lambda n: (n + 255) // 256 * 256
    for T in (64, 1000):
        T64 = (T + 63) // 64 * 64
        extra = al(4 * T * d) + (al(4 * d // 32 * T64) if form == "mxfp8" else al(4 * T))
        assert p.workspace_bytes(T) - p_bf.workspace_bytes(T) == al(36 * d * d) + extra
    if form == "mxfp8":
        with pytest.raises(dlo.DLOError):
            dlo.block_schema(48, form="mxfp8")


@pytest.mark.parametrize("mutate", ["per-row scale on FP8 codes", "int8 codes with E8M0 scales",
                                    "E8M0 scales per 16", "scale before weight"])
def test_forward_fails_closed_on_unvalidated_quantised_layouts(mutate):
    """Only the three quantised block forms are streamed: a quantised layout that is
    not one of them (a scale of another granularity or type, another order) plans and
    packs as plain byte groups, but the forward refuses it (DLO_E_UNSUPPORTED)."""
    from oracle import quant
    d = 256
    q = quant.quantize_block(synth.block_params(3, 0, d), "mxfp8" if mutate != "per-row scale on FP8 codes" else "int8")
    if mutate == "per-row scale on FP8 codes":      # INT8's fp32 row scales under E4M3 codes
        q = [(n, "fp8" if dt == "i8" else dt, np.asarray(a).view(np.uint8) if dt == "i8" else a) for n, dt, a in q]
    elif mutate == "int8 codes with E8M0 scales":
        q = [(n, "i8" if dt == "fp8" else dt, np.asarray(a).view(np.int8) if dt == "fp8" else a) for n, dt, a in q]
    elif mutate == "E8M0 scales per 16":
        q = [(n, dt, np.concatenate([a, a]) if dt == "e8m0" else a) for n, dt, a in q]
    else:                                            # weight_scale registered before its weight
        q = [q[1], q[0]] + q[2:]
    p = dlo.Plan([(d, 4, q)], 2)
    assert p.block_info(0)["form"] is None
    st = dlo.HostStore(p, pinned=False)
    st.pack(0, [(d, 4, q)])
    assert _status(lambda: dlo.forward_stack(p, st, **_args(p))) == "DLO_E_UNSUPPORTED"
