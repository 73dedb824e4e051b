"""Seeded synthetic inputs for the layerwise weight-streaming DiT stack.

Only inputs are made here: workload shapes, the block's parameter list in
registration order, and seeded random values (Philox4x32-10 + Box-Muller, from
``philox_normal.c``).  Nothing in this package computes any part of the method
or of the block forward; both the CPU oracle and the GPU path consume the bytes
it produces.

Recipe (the same for every workload):

* bf16 matrices ``W ~ N(0, 0.02)`` rounded fp32 -> bf16 to nearest-even;
* fp32 biases and LayerNorm shifts ``~ N(0, 0.02)``;
* LayerNorm scales ``1 + N(0, 0.02)``;
* each LayerNorm carries a one-element fp32 ``eps`` buffer holding 1e-6;
* activations ``x ~ N(0, 1)`` fp32 ``[T, D]``; conditioning ``c ~ N(0, 1)``
  fp32 ``[D]``.

Random stream ids: 0 = parameters (counter words a = block, b = parameter
index), 1 = activations, 2 = conditioning.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_SRC_PATH = os.path.join(_HERE, "philox_normal.c")

BF16 = "bf16"
F32 = "f32"

# --------------------------------------------------------------------------
# building / loading the generator
# --------------------------------------------------------------------------


def build(force: bool = True) -> str:
    """Compile the generator with gcc (OpenMP) in-tree; returns the .so path."""
    import subprocess

    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        obj = _LIB_PATH + ".o"
        # -ffast-math only at compile time (vectorised libmvec logf/cosf); linking
        # without it keeps crtfastmath.o out, which would otherwise switch the whole
        # process to flush-to-zero when the library is loaded.
        subprocess.check_call(["gcc", "-O3", "-mavx2", "-mfma", "-ffast-math", "-fopenmp",
                               "-fPIC", "-c", _SRC_PATH, "-o", obj])
        subprocess.check_call(["gcc", "-shared", "-fopenmp", obj, "-o", tmp, "-lm"])
        os.remove(obj)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        lib.synth_philox4x32_10.argtypes = [u32p, u32p, u32p]
        lib.synth_philox4x32_10.restype = None
        for name in ("synth_normal_f32", "synth_normal_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                           ctypes.c_int64, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
            fn.restype = None
        lib.synth_f32_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_f32_to_bf16.restype = None
        _lib = lib
    return _lib


def philox4x32_10(ctr, key):
    """Raw Philox4x32-10 block: four 32-bit counter words, two key words."""
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib.synth_philox4x32_10(c, k, o)
    return [int(v) for v in o]


def normal_f32(seed, stream, a, b, shape, mean=0.0, std=1.0, out=None):
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == n
    _load().synth_normal_f32(seed, stream, a, b, n, mean, std, out.ctypes.data)
    return out


def normal_bf16(seed, stream, a, b, shape, mean=0.0, std=1.0, out=None):
    """bf16 samples as raw uint16 bit patterns."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    _load().synth_normal_bf16(seed, stream, a, b, n, mean, std, out.ctypes.data)
    return out


def f32_to_bf16(arr):
    a = np.ascontiguousarray(arr, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_f32_to_bf16(a.ctypes.data, a.size, out.ctypes.data)
    return out


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    n_blocks: int
    widths: tuple        # d of block b is widths[b % len(widths)]
    head_dim: int
    tokens: int
    k: int
    passes: int
    D: int               # residual / conditioning width
    description: str = ""

    def width(self, b: int) -> int:
        return self.widths[b % len(self.widths)]

    def heads(self, b: int) -> int:
        return self.width(b) // self.head_dim

    def block_widths(self):
        return [self.width(b) for b in range(self.n_blocks)]

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", 3, (256,), 64, 64, 2, 2, 256,
                     "3 blocks, d=256, 4 heads, 64 tokens, k=2, 2 passes"),
    "8blk": Workload("8blk", 8, (1024,), 64, 1024, 2, 4, 1024,
                     "8 blocks, d=1024, 16 heads, 1024 tokens, k=2, 4 passes"),
    "nano": Workload("nano", 72, (3072,), 128, 4096, 4, 2, 3072,
                     "Nano-shaped: 72 blocks, d=3072, 24 heads, 4096 tokens, k=4, 2 passes"),
    "super": Workload("super", 128, (5120,), 128, 28800, 2, 2, 5120,
                      "Super-shaped: 128 blocks, d=5120, 40 heads, 28800 tokens (8x45x80), k=2, 2 passes"),
    "irregular": Workload("irregular", 127, (2048, 3072, 4096), 128, 8192, 4, 3, 4096,
                          "127 blocks, d in {2048,3072,4096}, 8192 tokens, k=4, 3 passes"),
}


def block_schema(d: int):
    """Parameters of one DiT block in registration order: (name, dtype, shape)."""
    return [
        ("adaln.weight", BF16, (6 * d, d)),
        ("adaln.bias", F32, (6 * d,)),
        ("norm1.weight", F32, (d,)),
        ("norm1.bias", F32, (d,)),
        ("norm1.eps", F32, (1,)),
        ("attn.qkv.weight", BF16, (3 * d, d)),
        ("attn.qkv.bias", F32, (3 * d,)),
        ("attn.out.weight", BF16, (d, d)),
        ("attn.out.bias", F32, (d,)),
        ("norm2.weight", F32, (d,)),
        ("norm2.bias", F32, (d,)),
        ("norm2.eps", F32, (1,)),
        ("mlp.fc1.weight", BF16, (4 * d, d)),
        ("mlp.fc1.bias", F32, (4 * d,)),
        ("mlp.fc2.weight", BF16, (d, 4 * d)),
        ("mlp.fc2.bias", F32, (d,)),
    ]


WEIGHT_STD = 0.02
EPS_VALUE = 1e-6


def block_params(seed: int, b: int, d: int, out_buffers=None):
    """Seeded parameters of block ``b`` (width ``d``): list of (name, dtype, ndarray).

    bf16 tensors are uint16 arrays of bf16 bit patterns.  ``out_buffers`` (a
    dict name -> array of the right shape and dtype) lets a caller reuse memory
    across blocks.
    """
    out = []
    for p, (name, dt, shape) in enumerate(block_schema(d)):
        buf = None if out_buffers is None else out_buffers.get(name)
        if dt == BF16:
            arr = normal_bf16(seed, 0, b, p, shape, 0.0, WEIGHT_STD, out=buf)
        elif name.endswith(".eps"):
            arr = np.full(shape, EPS_VALUE, dtype=np.float32)
        elif name.startswith("norm") and name.endswith(".weight"):
            arr = normal_f32(seed, 0, b, p, shape, 1.0, WEIGHT_STD, out=buf)
        else:
            arr = normal_f32(seed, 0, b, p, shape, 0.0, WEIGHT_STD, out=buf)
        out.append((name, dt, arr))
    return out


def activations(seed: int, tokens: int, D: int):
    return normal_f32(seed, 1, 0, 0, (tokens, D))


def conditioning(seed: int, D: int):
    return normal_f32(seed, 2, 0, 0, (D,))


@dataclass
class Stack:
    workload: Workload
    seed: int
    blocks: list = field(default_factory=list)   # list of list[(name, dtype, ndarray)]
    x: np.ndarray = None
    c: np.ndarray = None


def make_stack(w: Workload, seed: int = 0, n_blocks: int | None = None) -> Stack:
    """Generate every block (or the first ``n_blocks``) plus x and c in memory."""
    n = w.n_blocks if n_blocks is None else n_blocks
    st = Stack(w, seed)
    st.blocks = [block_params(seed, b, w.width(b)) for b in range(n)]
    st.x = activations(seed, w.tokens, w.D)
    st.c = conditioning(seed, w.D)
    return st

