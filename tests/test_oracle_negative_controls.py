"""Negative controls: planted streaming mistakes must fail the checks the GPU tests use.

Every mistake is planted in an oracle run on the CPU: the oracle is run with the
block order a faulty streamer would produce, and the result is compared with the
correct oracle run by the same metrics the GPU stack tests apply.  A check that
let these through would not catch the failures it exists for.

* The accumulated update x - x0 is the metric that catches a skipped block or a
  stale slot (a block run with the previous block's weights): each block moves
  x by only a few percent, so the final-x metric alone is weak (its values are
  reported for contrast).
* Two swapped slots (blocks 1 and 2 run in each other's place) change the
  update by only about 1 % on the tiny stack -- small block updates nearly
  commute -- so no activation tolerance of 2e-2 can catch them.  The per-step
  slot digest does: the GPU tests compare the digest of the slot each step
  reads, before and after the block ran, with the oracle digest of the block
  the step must run.
* The slot digest catches a changed byte anywhere in a slot region, the
  zero padding of the last shard included.
"""
import numpy as np
import pytest

import synth
from oracle import forward as of
from oracle import plan as op
from tests.gpu_util import TOL, rel_err

W = synth.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def tiny():
    st = synth.make_stack(W, seed=0)
    Ps = [of.param_dict(b) for b in st.blocks]
    heads = [W.heads(b) for b in range(W.n_blocks)]
    x0 = np.asarray(st.x, dtype=np.float64)
    return st, Ps, heads, x0


def _run(Ps, heads, x0, c, order):
    """The stack with step t running block order[t] on the weights the streamer handed it."""
    y = x0
    for b in order:
        y = of.dit_block(y, c, Ps[b], heads[b])
    return y


def _correct_order():
    return [b for _ in range(W.passes) for b in range(W.n_blocks)]


@pytest.mark.parametrize("name,order", [
    ("skipped block 1 in pass 0", [0, 2, 0, 1, 2]),
    ("stale slot: step 1 reads block 0's slot again", [0, 0, 2, 0, 1, 2]),
    ("tail block read again at the pass boundary", [0, 1, 2, 2, 1, 2]),
])
def test_planted_streaming_mistake_fails_the_update_metric(tiny, name, order):
    st, Ps, heads, x0 = tiny
    c = np.asarray(st.c, dtype=np.float64)
    ref = _run(Ps, heads, x0, c, _correct_order())
    assert np.array_equal(ref, of.forward_stack(x0, c, st.blocks, heads, W.passes))
    bad = _run(Ps, heads, x0, c, order)
    upd = rel_err(bad - x0, ref - x0)
    fin = rel_err(bad, ref)
    print(f"{name}: update metric {upd:.3g}, final-x metric {fin:.3g}")
    assert upd > TOL, (name, upd)


def test_swapped_slots_slip_under_the_activation_tolerance_but_not_the_digest(tiny):
    st, Ps, heads, x0 = tiny
    c = np.asarray(st.c, dtype=np.float64)
    ref = _run(Ps, heads, x0, c, _correct_order())
    bad = _run(Ps, heads, x0, c, [0, 2, 1, 0, 1, 2])
    upd = rel_err(bad - x0, ref - x0)
    print(f"swapped slots: update metric {upd:.3g}")
    assert 0 < upd < TOL   # the activation check alone would pass this mistake
    digests = []
    for b in range(W.n_blocks):
        bp = op.plan_block(op.specs_of(st.blocks[b]), W.k)
        digests.append(op.digest_regions(op.slot_regions(bp, op.pack_block(st.blocks[b], bp))))
    assert len(set(digests)) == W.n_blocks   # step 1 reading block 2's slot is caught


def test_gpu_rounding_points_stay_well_inside_the_tolerance(tiny, monkeypatch):
    """Positive control: the GPU's bf16 rounding of the GEMM inputs h, a, u and of q, k,
    v (RNE, emulated on the oracle; the adaLN input, fp32 on the GPU, is rounded too,
    which only adds error) moves the update far less than the mistakes above."""
    st, Ps, heads, x0 = tiny
    c = np.asarray(st.c, dtype=np.float64)
    ref = _run(Ps, heads, x0, c, _correct_order())

    def bf16(a):
        return (synth.f32_to_bf16(np.asarray(a, np.float32)).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    lin, att = of.linear, of.attention
    monkeypatch.setattr(of, "linear", lambda a, w, b: lin(bf16(a), w, b))
    monkeypatch.setattr(of, "attention", lambda q, k, v, h, **kw: att(bf16(q), bf16(k), bf16(v), h, **kw))
    rounded = _run(Ps, heads, x0, c, _correct_order())
    upd = rel_err(rounded - x0, ref - x0)
    print(f"bf16 rounding points: update metric {upd:.3g}")
    assert 0 < upd < TOL / 4


def test_digest_catches_a_changed_pad_byte():
    """k = 4 leaves 2 zero fp32 elements at the end of the last fp32 shard (19 d + 2 elements)."""
    params = synth.block_params(0, 0, 256)
    bp = op.plan_block(op.specs_of(params), 4)
    f32 = next(g for g, gp in enumerate(bp.groups) if gp.dtype == "f32")
    gp = bp.groups[f32]
    assert gp.numel == 19 * 256 + 2 and bp.region_bytes(f32) - gp.numel * 4 == 8
    regs = op.slot_regions(bp, op.pack_block(params, bp))
    d0 = op.digest_regions(regs)
    off, buf = regs[f32]
    assert np.all(buf[gp.numel * 4:] == 0)
    for pos in (gp.numel * 4, buf.size - 1):
        bad = buf.copy()
        bad[pos] ^= 0x01
        regs_bad = list(regs)
        regs_bad[f32] = (off, bad)
        assert op.digest_regions(regs_bad) != d0, pos
    # a weight byte and a swap of the two groups' contents are caught as well
    off0, buf0 = regs[0]
    bad0 = buf0.copy()
    bad0[12345] ^= 0x80
    assert op.digest_regions([(off0, bad0)] + regs[1:]) != d0
