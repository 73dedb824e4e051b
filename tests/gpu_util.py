"""Shared helpers of the GPU tests (test code only)."""
import os
import sys

import numpy as np
import pytest

import synth

TOL = 2e-2   # max |gpu - ref| / max |ref| on the final activations


def require_gpu():
    try:
        import torch
    except ImportError:
        pytest.skip("torch not importable")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import layerwise_weight_streaming_amd as dlo
    dlo.lib()   # raises if the HIP library is missing: no fallback
    return torch


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def stack_blocks(w, stack):
    return [(w.width(b), w.heads(b), ps) for b, ps in enumerate(stack.blocks)]


def spec_blocks(w, n):
    return [(w.width(b), w.heads(b), [(nm, dt, int(np.prod(s))) for nm, dt, s in synth.block_schema(w.width(b))])
            for b in range(n)]


def make_runner(w, stack, k=None, pinned=True):
    from layerwise_weight_streaming_amd.runner import StackRunner
    n = len(stack.blocks)
    r = StackRunner(spec_blocks(w, n), w.k if k is None else k, w.tokens, w.D, pinned=pinned)
    r.pack(0, stack_blocks(w, stack))
    r.set_inputs(stack.x, stack.c)
    return r


def fp8_blocks(w, stack, which=None):
    """Per block, the FP8 parameter list made by libdlo's quantizer (checked equal,
    byte for byte, to the oracle's).  which: block indices to quantize (default all);
    the others keep their bf16 lists."""
    from oracle import fp8 as ofp8
    import layerwise_weight_streaming_amd as dlo
    out = []
    for b, ps in enumerate(stack.blocks):
        if which is not None and b not in which:
            out.append(ps)
            continue
        ref = ofp8.quantize_block(ps)
        got = []
        for name, dt, arr in ps:
            if dt == "bf16":
                codes, scale = dlo.quantize_fp8(arr)
                got.append((name, "fp8", codes))
                got.append((name + "_scale", "f32", np.array([scale], dtype=np.float32)))
            else:
                got.append((name, dt, arr))
        assert [(n, d) for n, d, _ in got] == [(n, d) for n, d, _ in ref]
        for (_, _, a), (_, _, b2) in zip(got, ref):
            assert a.tobytes() == b2.tobytes()
        out.append(got)
    return out


def make_runner_params(w, blocks, k=None, pinned=True, batch=1):
    """A runner over explicit per-block parameter lists (any schema form)."""
    from layerwise_weight_streaming_amd.runner import StackRunner
    specs = [(w.width(b), w.heads(b), [(nm, dt, int(a.size)) for nm, dt, a in ps]) for b, ps in enumerate(blocks)]
    r = StackRunner(specs, w.k if k is None else k, w.tokens, w.D, pinned=pinned, batch=batch)
    r.pack(0, [(w.width(b), w.heads(b), ps) for b, ps in enumerate(blocks)])
    return r
