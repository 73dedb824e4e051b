#!/usr/bin/env python3
"""Writes the oracle's long-chain reference rows used by tests/test_gpu_long_chain.py.

Test infrastructure: this script calls only the oracle (oracle.forward) and the
seeded input generator (synth); nothing from the GPU library.  It runs the
resident float64 forward of a whole stack block by block (each block's
parameters regenerated from the seed when it is needed, widened exactly from
bf16, then dropped, so a 72-block stack fits in memory), and stores, at a few
checkpoints along the chain, the residual rows of a fixed random sample of
tokens together with the input rows.

Cases (seeded, at the workloads' own shapes):

* ``nano``: the Nano-shaped stack in full -- 72 blocks, d = 3072, 24 heads,
  4096 tokens -- two chained passes (144 block steps), checkpoints after block
  steps 24, 72 and 144;
* ``irregular``: the irregular stack's first 5 blocks (widths 2048, 3072,
  4096, 2048, 3072 in a residual of width 4096) at its own 8192 tokens, three
  passes (15 steps: an odd block count crosses the pass boundary twice),
  checkpoints after steps 5, 10 and 15;
* ``super``: the Super-shaped stack's first 3 blocks (d = 5120, 40 heads,
  28 800 tokens) over two passes (6 steps: the odd count crosses the pass
  boundary at full size), checkpoints after steps 3 and 6.

Output: tests/golden/stack_<case>.npz with ``rows`` (25 token indices), ``x0``
(input rows, float64), ``steps`` (checkpoint step counts) and ``ref`` (the
oracle's float64 rows stored as float32, [len(steps), len(rows), D]: the
rounding, 2^-24 relative, is far below the 2e-2 parity bound).

Usage: python tests/golden/make_stack_goldens.py [nano] [irregular]
(about 10 min for nano, 3 min for irregular and 25 min for super on 8 cores).
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import forward as of  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))

CASES = {
    # name: (workload, seed, n_blocks, passes, tokens, checkpoint steps, sampled rows)
    "nano": ("nano", 4, 72, 2, None, (24, 72, 144), 48),
    "irregular": ("irregular", 2, 5, 3, None, (5, 10, 15), 48),
    "super": ("super", 6, 3, 2, None, (3, 6), 48),
}


def sample_rows(T: int, n: int, seed: int) -> np.ndarray:
    """Sorted distinct token indices: n draws including the first and the last
    token, thinned to every other one plus the last (n / 2 + 1 rows)."""
    rng = np.random.default_rng(1000 + seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    rows = np.sort(np.concatenate([[0, T - 1], mid])).astype(np.int64)
    return np.concatenate([rows[:-1:2], rows[-1:]])


def run_case(name: str) -> str:
    wname, seed, n, passes, tokens, steps, n_rows = CASES[name]
    w = synth.WORKLOADS[wname]
    if tokens is not None:
        w = w.with_(tokens=tokens)
    x0 = synth.activations(seed, w.tokens, w.D).astype(np.float64)
    c = synth.conditioning(seed, w.D)
    rows = sample_rows(w.tokens, n_rows, seed)
    ref = np.empty((len(steps), len(rows), w.D), dtype=np.float32)
    y = x0
    t0 = time.time()
    done = 0
    for p in range(passes):
        for b in range(n):
            P = of.param_dict(synth.block_params(seed, b, w.width(b)))
            y = of.dit_block(y, c, P, w.heads(b))
            del P
            done += 1
            if done in steps:
                ref[steps.index(done)] = y[rows]
            print(f"[golden {name}] step {done}/{n * passes} ({time.time() - t0:.0f} s)", flush=True)
    out = os.path.join(HERE, f"stack_{name}.npz")
    np.savez_compressed(out, rows=rows, x0=x0[rows], steps=np.asarray(steps, dtype=np.int64), ref=ref,
                        meta=np.asarray([seed, n, passes, w.tokens, w.D], dtype=np.int64))
    return out


def main(argv):
    names = argv[1:] or list(CASES)
    for name in names:
        print("wrote", run_case(name), flush=True)


if __name__ == "__main__":
    main(sys.argv)
