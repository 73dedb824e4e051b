"""CPU oracle for the layerwise weight-streaming DiT forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
GPU product path never touches this package, and this package never touches
the GPU path: the two share no code, only the seeded inputs made by ``synth``.

Contents, each function citing the passage it follows:

* ``oracle.plan``     -- flatten-by-dtype, ceil-div sharding with zero padding,
                         reassembly at all-gather offsets, slot sizing, slot
                         digests (the race-detector definition).
* ``oracle.schedule`` -- the two-slot hook rule (parity, corrected by the
                         ring predecessor's prefetch), a static-rule
                         negative control, and a happens-before checker for
                         programs of copy / compute / event operations.
* ``oracle.forward``  -- the DiT stack with every weight resident, in float64
                         over the same bf16 weights (exact widening).

Pages cited (by title):

* [Jul] "Distributed Layerwise Offload", vLLM-Omni project blog, 2026-07-30.
* [Aug] "Distributed Layerwise Offload: Scaling Toward 200B+ DiT Models
  Efficiently in vLLM-Omni", vLLM blog, 2026-08-17.
* [Doc] "Distributed Layerwise Offload", vLLM-Omni design documentation.

Parity status: plan, pack, reassembly, schedule and footprint are pinned by
closed forms and hand-derived fixtures; the forward is pinned by brute force,
special cases and hand-computed examples.  The pages never define the DiT
block's internals, so the block itself follows the plain adaLN-Zero reading
written out in ``oracle.forward``; that reading, not a page, is what those pins
check.
"""
from . import plan, schedule, forward  # noqa: F401
