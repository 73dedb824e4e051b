"""End-to-end streamed stack on the GPU against the oracle.

* activations: max|gpu - ref| / max|ref| <= 2e-2 on the final x, and the same on
  the accumulated update x - x0 (a skipped block or a stale slot moves x by only
  a few percent, so the update metric is the one that catches it);
* slot trace: equal to the oracle's hook simulation, step by step;
* slot contents: per-step digests equal the oracle digest of the expected block,
  before and after the block ran (nothing overwrote a slot being read), and the
  final slot bytes equal the oracle's reassembled shards;
* streamed == resident and k-invariance: bit-exact (the method must not change
  a single bit of what the resident model computes).
"""
import numpy as np
import pytest

import synth
import layerwise_weight_streaming_amd as dlo
from oracle import forward as of
from oracle import plan as op
from oracle import schedule as sc
from tests.gpu_util import (TOL, fp8_blocks, make_runner, make_runner_params, rel_err, require_gpu,
                            say, spec_blocks)

pytestmark = pytest.mark.gpu


def _expected_regions(w, stack, k):
    regs = []
    for ps in stack.blocks:
        bp = op.plan_block(op.specs_of(ps), k)
        regs.append(op.slot_regions(bp, op.pack_block(ps, bp)))
    return regs


def _check_trace(tr, n, passes, regs=None, n_resident=0):
    ref = sc.simulate_hooks(n, passes, n_resident=n_resident)
    assert len(tr) == len(ref)
    for got, e in zip(tr, ref):
        assert (got["step"], got["pass_"], got["block"], got["read_slot"], got["prefetch_block"],
                got["prefetch_slot"]) == (e.step, e.pass_, e.block, e.read_slot, e.prefetch_block,
                                          e.prefetch_slot)
        if regs is not None:
            want = op.digest_regions(regs[e.block])
            assert got["digest_pre"] == want, f"step {e.step}: slot held other bytes before the block"
            assert got["digest_post"] == want, f"step {e.step}: slot changed while the block ran"


def _run_and_compare(name, n_blocks=None, passes=None, seed=0, tokens=None):
    torch = require_gpu()
    w = synth.WORKLOADS[name]
    if tokens is not None:
        w = w.with_(tokens=tokens)
    n = w.n_blocks if n_blocks is None else n_blocks
    P = w.passes if passes is None else passes
    say(f"stack {name} n={n} passes={P} T={w.tokens} k={w.k}")
    stack = synth.make_stack(w, seed, n)
    r = make_runner(w, stack)
    run = r.forward(P, flags=dlo.TRACE_DIGEST)
    tr = run.trace()
    x_gpu = r.x_host()
    regs = _expected_regions(w, stack, w.k)
    _check_trace(tr, n, P, regs)
    # final slot bytes: the last two steps' blocks
    total = n * P
    for t in (total - 1, total - 2):
        if t < 0:
            continue
        e = tr[t]
        slot = r.slot_host(e["read_slot"])
        for off, buf in regs[e["block"]]:
            assert slot[off:off + buf.size].tobytes() == buf.tobytes()
    say("oracle forward")
    x_ref = of.forward_stack(stack.x, stack.c, stack.blocks, [w.heads(b) for b in range(n)], P)
    e_abs = rel_err(x_gpu, x_ref)
    e_upd = rel_err(x_gpu - stack.x, x_ref - stack.x)
    say(f"rel err {e_abs:.3e}, update rel err {e_upd:.3e}")
    assert e_abs <= TOL and e_upd <= TOL
    r.close()
    return e_abs, e_upd


def test_tiny_stack_streamed():
    _run_and_compare("tiny")


def test_tiny_stack_three_passes_odd_tail():
    _run_and_compare("tiny", passes=3, seed=5)


@pytest.mark.parametrize("tokens", [1, 129])
def test_tiny_stack_ragged_token_counts(tokens):
    # one token (attention over a single key) and a count that leaves partial
    # 64-key blocks, 128-row LN/attention tiles and 256-row GEMM tiles
    _run_and_compare("tiny", passes=3, seed=8, tokens=tokens)


@pytest.mark.parametrize("n_blocks,passes", [(1, 1), (1, 3), (2, 3)])
def test_short_stacks(n_blocks, passes):
    # one block: a single step prefetches nothing; over several passes the block's
    # hook prefetches the block itself into the other slot.  Two blocks: the even
    # ring, where the plain parity and the prefetched slot agree.
    _run_and_compare("tiny", n_blocks=n_blocks, passes=passes, seed=11)


def test_8blk_stack_streamed():
    _run_and_compare("8blk")


def test_irregular_prefix_small_tokens():
    # mixed widths 2048/3072/4096 and an odd block count (tail -> head correction), 3 passes
    _run_and_compare("irregular", n_blocks=3, tokens=256, seed=2)


def test_nano_prefix_full_shape():
    # full Nano width and tokens, two blocks, one pass
    _run_and_compare("nano", n_blocks=2, passes=1, seed=4)


def _streamed_vs_resident(name, n, passes, tokens=None, ks=None):
    torch = require_gpu()
    w = synth.WORKLOADS[name]
    if tokens is not None:
        w = w.with_(tokens=tokens)
    say(f"streamed vs resident {name} n={n} passes={passes} T={w.tokens}")
    stack = synth.make_stack(w, 0, n)
    r = make_runner(w, stack)
    r.forward(passes, want_run=False)
    x_stream = r.x_host()
    r.set_inputs(stack.x, stack.c)
    r.forward(passes, resident=True, want_run=False)
    x_res = r.x_host()
    assert np.array_equal(x_stream.view(np.uint32), x_res.view(np.uint32))
    r.close()
    for k in ks or []:
        say(f"k = {k}")
        r2 = make_runner(w, stack, k=k)
        r2.forward(passes, want_run=False)
        assert np.array_equal(r2.x_host().view(np.uint32), x_stream.view(np.uint32)), k
        r2.close()
    return x_stream


def test_streamed_equals_resident_and_k_invariant_small():
    _streamed_vs_resident("tiny", 3, 3, ks=[1, 3, 4, 8])
    _streamed_vs_resident("8blk", 8, 2, ks=[1, 4])


def test_streamed_equals_resident_irregular_full_tokens():
    _streamed_vs_resident("irregular", 5, 2)


def test_streamed_equals_resident_super_prefix():
    # Super width and tokens, three blocks (odd), two passes
    _streamed_vs_resident("super", 3, 2)


def test_super_block_sampled_rows():
    """One Super-shaped block (T=28800, d=5120): sampled output rows vs the oracle."""
    torch = require_gpu()
    w = synth.WORKLOADS["super"]
    say("super one block, sampled rows")
    stack = synth.make_stack(w, 0, 1)
    r = make_runner(w, stack)
    r.forward(1, want_run=False)
    x_gpu = r.x_host()
    r.close()
    rng = np.random.default_rng(3)
    rows = np.concatenate([rng.integers(0, w.tokens, 6), [0, w.tokens - 1]])
    say("oracle rows")
    ref = of.dit_block_rows(stack.x, stack.c, of.param_dict(stack.blocks[0]), w.heads(0), rows)
    x0 = stack.x[rows]
    assert rel_err(x_gpu[rows], ref) <= TOL
    assert rel_err(x_gpu[rows] - x0, ref - x0) <= TOL


def test_repeated_calls_reuse_slots():
    """Back-to-back runs on the same slots (no host sync between them) equal two passes."""
    torch = require_gpu()
    w = synth.WORKLOADS["tiny"]
    stack = synth.make_stack(w, 9)
    r = make_runner(w, stack)
    r.forward(1, want_run=False)
    r.forward(1, want_run=False)
    x_two_calls = r.x_host()
    r.set_inputs(stack.x, stack.c)
    r.forward(2, want_run=False)
    assert np.array_equal(x_two_calls.view(np.uint32), r.x_host().view(np.uint32))
    r.close()


def test_timing_trace_is_ordered():
    torch = require_gpu()
    w = synth.WORKLOADS["8blk"]
    stack = synth.make_stack(w, 1)
    r = make_runner(w, stack)
    run = r.forward(2, flags=dlo.TRACE_TIMING)
    tr = run.trace()
    kt = run.kernel_times()
    assert kt.shape == (16, dlo.KERNELS_PER_BLOCK) and np.all(kt >= 0)
    # a bf16 block launches nothing in the dequantisation and W8A8 quantisation
    # slots: they read exactly 0; every other slot ran a kernel
    names = dlo.kernel_names()
    empty = [j for j, nm in enumerate(names) if nm == "dequant_weights" or nm.startswith("quant_")]
    assert len(empty) == 5
    assert np.all(kt[:, empty] == 0)
    assert np.all(np.delete(kt, empty, axis=1) > 0)
    for e, row in zip(tr, kt):
        assert row.sum() <= e["t_compute_end"] - e["t_compute_begin"] + 1e-3
    for e in tr:
        assert 0 <= e["t_copy_begin"] <= e["t_copy_end"] <= e["t_compute_end"]
        assert e["t_copy_end"] <= e["t_compute_begin"] + 1e-3 <= e["t_compute_end"] + 1e-3
    # a slot is refilled only after the compute that last read it has ended
    for t in range(2, len(tr)):
        assert tr[t]["t_copy_begin"] >= tr[t - 2]["t_compute_end"] - 1e-3
    r.close()


@pytest.mark.parametrize("mode,limit_blocks", [("pageable", 0), ("auto", 3)])
def test_staged_store_matches_pinned(mode, limit_blocks):
    """Blocks staged through the two pinned staging buffers give the pinned result, bit for bit."""
    torch = require_gpu()
    from layerwise_weight_streaming_amd.runner import StackRunner
    w = synth.WORKLOADS["8blk"]
    say(f"staged store {mode}")
    stack = synth.make_stack(w, 6)
    blocks = [(w.width(b), w.heads(b), ps) for b, ps in enumerate(stack.blocks)]
    specs = spec_blocks(w, w.n_blocks)
    ref = make_runner(w, stack)
    ref.forward(w.passes, want_run=False)
    x_ref = ref.x_host()
    ref.close()
    limit = 0
    if limit_blocks:
        limit = limit_blocks * (op.plan_block(op.specs_of(stack.blocks[0]), w.k).extent + 16 * 4096)
    r = StackRunner(specs, w.k, w.tokens, w.D, store_mode=mode, pinned_limit=limit)
    info = r.store.info()
    if mode == "pageable":
        assert info["pinned_blocks"] == 0 and info["staged_blocks"] == w.n_blocks
    else:
        assert info["pinned_blocks"] == limit_blocks and info["staged_blocks"] == w.n_blocks - limit_blocks
    r.pack(0, blocks)
    r.set_inputs(stack.x, stack.c)
    run = r.forward(w.passes, flags=dlo.TRACE_DIGEST)
    tr = run.trace()
    _check_trace(tr, w.n_blocks, w.passes, _expected_regions(w, stack, w.k))
    assert np.array_equal(r.x_host().view(np.uint32), x_ref.view(np.uint32))
    r.close()


@pytest.mark.parametrize("mode,limit_blocks", [("pageable", 0), ("auto", 3)])
def test_async_enqueue_staged_store(mode, limit_blocks):
    """DLO_ASYNC_ENQUEUE ([Doc] "Rank-local path without DLO AllGather": the staging slots
    as a pipeline stage of their own): the call returns before its program is enqueued
    (a synchronous call with staged blocks returns only once the last staged block is
    handed to the copy stream), another run of the plan is refused until
    dlo_run_enqueued, and the run computes the synchronous call's bits with the same
    slot trace and digests."""
    import time
    require_gpu()
    from layerwise_weight_streaming_amd.runner import StackRunner
    w = synth.WORKLOADS["8blk"]
    say(f"async enqueue, staged store {mode}")
    stack = synth.make_stack(w, 6)
    blocks = [(w.width(b), w.heads(b), ps) for b, ps in enumerate(stack.blocks)]
    limit = 0
    if limit_blocks:
        limit = limit_blocks * (op.plan_block(op.specs_of(stack.blocks[0]), w.k).extent + 16 * 4096)
    r = StackRunner(spec_blocks(w, w.n_blocks), w.k, w.tokens, w.D, store_mode=mode, pinned_limit=limit)
    r.pack(0, blocks)
    r.set_inputs(stack.x, stack.c)
    r.forward(w.passes, want_run=False)   # staging buffers allocated, code loaded
    r.synchronize()
    r.set_inputs(stack.x, stack.c)
    t0 = time.perf_counter()
    run = r.forward(w.passes, flags=dlo.TRACE_DIGEST)
    t_sync = time.perf_counter() - t0
    tr_sync = run.trace()
    x_sync = r.x_host()
    run.close()

    r.set_inputs(stack.x, stack.c)
    t0 = time.perf_counter()
    run = r.forward(w.passes, flags=dlo.TRACE_DIGEST | dlo.ASYNC_ENQUEUE)
    t_async = time.perf_counter() - t0
    with pytest.raises(dlo.DLOError) as ei:
        r.forward(1, want_run=False)
    assert ei.value.code == -7   # DLO_E_STATE: the plan is still being enqueued
    run.enqueued()
    tr = run.trace()
    say(f"the call returned after {t_async * 1e3:.2f} ms (synchronous call: {t_sync * 1e3:.2f} ms)")
    _check_trace(tr, w.n_blocks, w.passes, _expected_regions(w, stack, w.k))
    assert tr == tr_sync
    assert np.array_equal(r.x_host().view(np.uint32), x_sync.view(np.uint32))
    assert t_async < 0.5 * t_sync
    run.close()
    r.close()


@pytest.mark.parametrize("form,flags", [("bf16", 0), ("fp8", 0), ("fp8", dlo.FP8_COMPUTE)],
                         ids=["bf16", "fp8_w8a16", "fp8_w8a8"])
def test_batch_is_its_samples_one_by_one(form, flags):
    """A batch of 3 samples (own x rows, own conditioning) through one streamed run: every
    block's copy serves the three, and each sample's result is bit-identical to a run of
    that sample alone; the slot trace and digests are the single-sample ones.  fp8: the
    dequantised weights (W8A16) are made once per block step and reused by the samples."""
    require_gpu()
    w = synth.WORKLOADS["tiny"]
    B = 3
    say(f"batch {B}, {form}, flags {flags}")
    stack = synth.make_stack(w, 31)
    blocks = fp8_blocks(w, stack) if form == "fp8" else stack.blocks
    xs = [synth.activations(40 + b, w.tokens, w.D) for b in range(B)]
    cs = [synth.conditioning(40 + b, w.D) for b in range(B)]
    r1 = make_runner_params(w, blocks)
    want, tr1 = [], None
    for b in range(B):
        r1.set_inputs(xs[b], cs[b])
        run = r1.forward(w.passes, flags=flags | dlo.TRACE_DIGEST)
        tr1 = run.trace()
        want.append(r1.x_host())
        run.close()
    r1.close()
    rb = make_runner_params(w, blocks, batch=B)
    rb.set_inputs(np.concatenate(xs, axis=0), np.stack(cs, axis=0))
    run = rb.forward(w.passes, flags=flags | dlo.TRACE_DIGEST | dlo.TRACE_TIMING)
    tr = run.trace()
    kt = run.kernel_times()
    got = rb.x_host()
    run.close()
    rb.close()
    for b in range(B):
        assert np.array_equal(got[b * w.tokens:(b + 1) * w.tokens].view(np.uint32), want[b].view(np.uint32)), b
    strip = lambda t: [{k: v for k, v in e.items() if not k.startswith("t_")} for e in t]
    assert strip(tr) == strip(tr1)
    assert all(e["t_compute_end"] >= e["t_compute_begin"] >= 0 for e in tr)
    assert kt.shape == (len(tr), dlo.KERNELS_PER_BLOCK) and np.all(kt >= 0)


@pytest.mark.parametrize("n_resident", [1, 3, 7, 8])
def test_resident_layers_match_full_streaming(n_resident):
    """Blocks 0 .. R-1 resident, the rest streamed: the slot trace and digests follow
    the oracle's hook rule over the streamed blocks, and x equals the fully
    streamed result bit for bit (the streamed subset has an odd count for R = 1, 3, 7)."""
    torch = require_gpu()
    w = synth.WORKLOADS["8blk"]
    say(f"resident layers R={n_resident}")
    stack = synth.make_stack(w, 11)
    r = make_runner(w, stack)
    r.forward(w.passes, want_run=False)
    x_stream = r.x_host()
    r.set_inputs(stack.x, stack.c)
    run = r.forward(w.passes, flags=dlo.TRACE_DIGEST, n_resident=n_resident)
    tr = run.trace()
    _check_trace(tr, w.n_blocks, w.passes, _expected_regions(w, stack, w.k), n_resident=n_resident)
    assert np.array_equal(r.x_host().view(np.uint32), x_stream.view(np.uint32))
    # repeated calls with resident layers chain like passes
    r.set_inputs(stack.x, stack.c)
    r.forward(1, n_resident=n_resident, want_run=False)
    r.forward(w.passes - 1, n_resident=n_resident, want_run=False)
    assert np.array_equal(r.x_host().view(np.uint32), x_stream.view(np.uint32))
    r.close()


def _regions_of(blocks, k):
    regs = []
    for ps in blocks:
        bp = op.plan_block(op.specs_of(ps), k)
        regs.append(op.slot_regions(bp, op.pack_block(ps, bp)))
    return regs


@pytest.mark.parametrize("name,n_blocks,tokens,which", [
    ("tiny", None, None, None),                 # every block FP8, 2 passes, odd count
    ("8blk", None, None, {0, 2, 3, 5}),         # FP8 and bf16 blocks mixed in one plan
    ("irregular", 3, 256, None),                # widths 2048/3072/4096, k = 4 (uneven fp32 padding)
])
def test_fp8_weight_groups_streamed(name, n_blocks, tokens, which):
    """FP8 (E4M3 + fp32 scale) blocks: 1-byte groups sharded, streamed and placed at the
    all-gather offsets (slot bytes and digests = oracle), forward within tolerance of the
    oracle on the dequantised weights, and streamed == resident bit for bit."""
    torch = require_gpu()
    w = synth.WORKLOADS[name]
    if tokens is not None:
        w = w.with_(tokens=tokens)
    n = w.n_blocks if n_blocks is None else n_blocks
    say(f"fp8 stack {name} n={n} T={w.tokens} which={which}")
    stack = synth.make_stack(w, 21, n)
    blocks = fp8_blocks(w, stack, which)
    r = make_runner_params(w, blocks)
    for b in range(n):
        assert r.plan.block_info(b)["fp8"] == (which is None or b in which)
    r.set_inputs(stack.x, stack.c)
    run = r.forward(w.passes, flags=dlo.TRACE_DIGEST)
    tr = run.trace()
    regs = _regions_of(blocks, w.k)
    _check_trace(tr, n, w.passes, regs)
    x_gpu = r.x_host()
    say("oracle forward (dequantised weights)")
    x_ref = of.forward_stack(stack.x, stack.c, blocks, [w.heads(b) for b in range(n)], w.passes)
    e_abs, e_upd = rel_err(x_gpu, x_ref), rel_err(x_gpu - stack.x, x_ref - stack.x)
    say(f"rel err {e_abs:.3e}, update rel err {e_upd:.3e}")
    assert e_abs <= TOL and e_upd <= TOL
    r.set_inputs(stack.x, stack.c)
    r.forward(w.passes, resident=True, want_run=False)
    assert np.array_equal(r.x_host().view(np.uint32), x_gpu.view(np.uint32))
    r.close()


def test_device_weight_memory_is_two_slots_at_any_depth():
    """The device holds weights in exactly two slots of the largest block whatever
    the stack's depth: the runner's slot allocation is two slots (torch rounds an
    allocation up to 512 B), and a streamed run allocates no device memory of its
    own (measured as the device's free memory around a second, warm run)."""
    torch = require_gpu()
    w = synth.WORKLOADS["8blk"]
    slot_bytes = None
    for n in (1, 3, 8):
        say(f"device weight memory, {n} blocks")
        stack = synth.make_stack(w, 2, n)
        r = make_runner(w, stack)
        sb = r.plan.slot_bytes
        slot_bytes = sb if slot_bytes is None else slot_bytes
        assert sb == slot_bytes                      # the slot is the largest block, not the stack
        assert 0 <= r.slot_alloc_bytes - 2 * sb < 1024
        r.forward(w.passes, want_run=False)
        r.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        run = r.forward(w.passes, flags=dlo.TRACE_TIMING)
        run.trace()
        free1 = torch.cuda.mem_get_info()[0]
        assert free0 - free1 < (1 << 20), (n, free0 - free1)
        run.close()
        r.close()


def test_streamed_run_waits_for_the_previous_run():
    """A streamed run of a plan is enqueued only once the plan's previous run has
    completed (copies queued behind a run still executing ran slower): the second of
    two back-to-back calls returns only after the first run's GPU work is done."""
    import time
    require_gpu()
    w = synth.WORKLOADS["8blk"]
    stack = synth.make_stack(w, 3)
    r = make_runner(w, stack)
    r.forward(2, want_run=False)
    r.synchronize()
    t0 = time.perf_counter()
    run = r.forward(40, flags=dlo.TRACE_TIMING)   # 320 block steps, a few hundred ms of copies
    r.forward(1, want_run=False)
    t_second = time.perf_counter() - t0
    tr = run.trace()
    gpu_ms = max(e["t_compute_end"] for e in tr)
    say(f"first run {gpu_ms:.1f} ms on the GPU; the second call returned after {t_second * 1e3:.1f} ms")
    assert gpu_ms > 50
    assert t_second * 1e3 >= 0.8 * gpu_ms
    run.close()
    r.close()
