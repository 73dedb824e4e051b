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
