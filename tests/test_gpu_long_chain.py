"""Long chains of streamed blocks on the GPU against the oracle.

The streamed result must be the resident model's result ([Aug] "NVIDIA B300 GPU
Results", correctness paragraph), and the GPU's bf16 rounding points must not
make the error grow along the chain.  The oracle's float64 forward of a whole
Nano-shaped stack takes minutes on a CPU, so its residual rows at a few
checkpoints were written beforehand by tests/golden/make_stack_goldens.py
(which calls only the oracle and the seeded input generator) for a fixed
random sample of tokens; here the GPU runs the same seeded stacks and its rows
are compared with them:

* ``nano``: the full Nano-shaped stack (72 blocks, d = 3072, 4096 tokens,
  k = 4), checkpoints after 24 block steps (a 24-block plan, one pass), 72
  (one pass) and 144 (two chained passes in one call: the pass boundary);
* ``irregular``: 5 blocks of widths 2048, 3072, 4096, 2048, 3072 in a residual
  of width 4096 at the workload's own 8192 tokens (k = 4), checkpoints after
  1, 2 and 3 passes;
* ``super``: the first 3 Super-shaped blocks (d = 5120, 40 heads, 28 800
  tokens, k = 2), checkpoints after 1 and 2 passes.

Metrics at each checkpoint, over the sampled rows: max|gpu - ref| / max|ref|
and the same on the accumulated update x - x0, both <= 2e-2.  The per-step
slot trace of every run is checked against the oracle's hook simulation, and
for the irregular stack the per-step slot digests against the oracle's
reassembled shards as well.
"""
import os

import numpy as np
import pytest

import synth
import layerwise_weight_streaming_amd as dlo
from oracle import plan as op
from oracle import schedule as sc
from tests.gpu_util import TOL, rel_err, require_gpu, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    path = os.path.join(GOLDEN, f"stack_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} missing: run tests/golden/make_stack_goldens.py {name}")
    with np.load(path, allow_pickle=False) as z:
        return {k: z[k] for k in z.files}


def _runner(w, seed, n, digests=False):
    """A runner over the first n blocks, packed one generated block at a time, and
    (digests=True) the oracle's slot digest of each block."""
    from layerwise_weight_streaming_amd.runner import StackRunner
    specs = [(w.width(b), w.heads(b), [(nm, dt, int(np.prod(s))) for nm, dt, s in synth.block_schema(w.width(b))])
             for b in range(n)]
    r = StackRunner(specs, w.k, w.tokens, w.D)
    dig = []
    for b in range(n):
        ps = synth.block_params(seed, b, w.width(b))
        r.pack(b, [(w.width(b), w.heads(b), ps)])
        if digests:
            bp = op.plan_block(op.specs_of(ps), w.k)
            dig.append(op.digest_regions(op.slot_regions(bp, op.pack_block(ps, bp))))
    return r, dig


def _same_inputs(x0, g):
    """The seeded inputs here are the ones the goldens were written from.  The
    generator's Box-Muller runs through the C library's vector logf/cosf, whose
    last bits can differ between CPU models (measured: 2 ulp of fp32), so the
    check allows 1e-5; a wrong seed or shape is off by O(1)."""
    assert x0[g["rows"]].shape == g["x0"].shape
    assert np.max(np.abs(x0[g["rows"]].astype(np.float64) - g["x0"])) <= 1e-5


def _compare(tag, x_gpu, g, i):
    rows, x0 = g["rows"], g["x0"]
    ref = g["ref"][i]
    got = x_gpu[rows].astype(np.float64)
    e_abs, e_upd = rel_err(got, ref), rel_err(got - x0, ref - x0)
    say(f"{tag}: after {int(g['steps'][i])} block steps: rel err {e_abs:.3e}, update rel err {e_upd:.3e}")
    assert e_abs <= TOL and e_upd <= TOL, (tag, e_abs, e_upd)
    return e_abs, e_upd


def _check_trace(tr, n, passes, digests=None):
    ref = sc.simulate_hooks(n, passes)
    assert len(tr) == len(ref)
    for got, e in zip(tr, ref):
        assert (got["block"], got["read_slot"], got["prefetch_block"], got["prefetch_slot"]) == \
            (e.block, e.read_slot, e.prefetch_block, e.prefetch_slot)
        if digests:
            want = digests[e.block]
            assert got["digest_pre"] == want and got["digest_post"] == want, e.step


def test_nano_full_stack_two_passes():
    require_gpu()
    g = _golden("nano")
    seed, n, passes, T, D = (int(v) for v in g["meta"])
    w = synth.WORKLOADS["nano"]
    assert (n, passes, T, D) == (w.n_blocks, w.passes, w.tokens, w.D)
    x0 = synth.activations(seed, T, D)
    c = synth.conditioning(seed, D)
    _same_inputs(x0, g)
    errs = []
    # checkpoint 0: a 24-block plan, one pass
    n24 = int(g["steps"][0])
    say(f"nano: {n24}-block prefix, one pass")
    r, _ = _runner(w, seed, n24)
    r.set_inputs(x0, c)
    r.forward(1, want_run=False)
    errs.append(_compare("nano prefix", r.x_host(), g, 0))
    r.close()
    say("nano: full stack")
    r, _ = _runner(w, seed, n)
    r.set_inputs(x0, c)
    r.forward(1, want_run=False)
    errs.append(_compare("nano 1 pass", r.x_host(), g, 1))
    r.set_inputs(x0, c)
    run = r.forward(passes)
    _check_trace(run.trace(), n, passes)
    errs.append(_compare("nano 2 passes", r.x_host(), g, 2))
    run.close()
    r.close()
    say("nano update error along the chain (24, 72, 144 steps): " + ", ".join(f"{e[1]:.3e}" for e in errs))


def _prefix_by_passes(name):
    """The golden's first n blocks at the workload's own size, one run per pass
    count; trace and slot digests checked on every run."""
    require_gpu()
    g = _golden(name)
    seed, n, passes, T, D = (int(v) for v in g["meta"])
    w = synth.WORKLOADS[name]
    assert (T, D) == (w.tokens, w.D)
    x0 = synth.activations(seed, T, D)
    c = synth.conditioning(seed, D)
    _same_inputs(x0, g)
    r, dig = _runner(w, seed, n, digests=True)
    errs = []
    for p in range(1, passes + 1):
        say(f"{name}: {n} blocks, T={T}, {p} passes")
        r.set_inputs(x0, c)
        run = r.forward(p, flags=dlo.TRACE_DIGEST)
        _check_trace(run.trace(), n, p, dig)
        errs.append(_compare(f"{name} {p} passes", r.x_host(), g, p - 1))
        run.close()
    r.close()
    say(f"{name} update error along the chain: " + ", ".join(f"{e[1]:.3e}" for e in errs))


def test_irregular_prefix_full_tokens():
    _prefix_by_passes("irregular")


def test_super_prefix_full_size_two_passes():
    # three full Super-shaped blocks (d = 5120, 28 800 tokens, 944 MB slots): the
    # odd count takes the tail -> head correction at the pass boundary
    _prefix_by_passes("super")
