"""Oracle: online INT8 and MXFP8 weight forms (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
use this package; the GPU path shares no code with it.

The pages let two more online-quantised linear forms take the sharding path
besides per-tensor FP8: online INT8, an int8 weight plus an fp32 scale, and
online MXFP8, an fp8 weight plus an e8m0 block scale; all are plain 1-byte
dtypes packed in physical order like any other group ([Doc] "Request and
loading constraints", the paragraph on online FP8, INT8 and MXFP8 linears).
They fix neither the INT8 scale's granularity nor the MX block rule; the
readings here:

* INT8: symmetric, one fp32 scale per output channel (row of the [out, in]
  weight): scale_r = amax_r(|w|) / 127 in float32 (1.0 for an all-zero row,
  NaN entries ignored); code = float32(w) / scale_r (float32 division)
  rounded to the nearest integer, ties to even, clamped to [-127, 127]; the
  dequantised weight is code * scale_r.
* MXFP8: the OCP Microscaling (MX) format with E4M3 elements: blocks of 32
  consecutive elements along the input dimension share one E8M0 scale 2^X
  with X = floor(log2(amax of the block)) - 8 (8 = the largest exponent of a
  normal E4M3 value), clamped to [-127, 127]; an all-zero block takes
  X = -127; each element is the E4M3 code nearest to float32(w) / 2^X, ties to
  the even code, saturating at +-448; the E8M0 byte is X + 127 (255 is NaN).
  The dequantised weight is code_value * 2^X, exactly.  The block form keeps
  the scales block-major, [in / 32, out] (the transposed view the pages allow
  for a finalised tensor): the scales of one input block for consecutive
  output rows are adjacent, the order a block-scaled matrix product reads.
* W8A8 with MXFP8 weights: each linear's input (as stored in bf16) is
  quantised the same way, per row in blocks of 32 along the input dimension.
* W8A8 with INT8 weights: each linear's input (as stored in bf16) is
  quantised by the INT8 rule per row (symmetric, amax / 127); the product is
  the exact integer dot product of the codes times both scales.
"""
from __future__ import annotations

import numpy as np

from . import fp8

INT8_MAX = 127
MX_BLOCK = 32
E4M3_EMAX = 8          # 448 = 1.75 * 2^8


def _widen(w_bf16_bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(w_bf16_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- INT8 ----

def quantize_int8(w_bf16_bits):
    """bf16 weight [rows, cols] (bit patterns) -> (int8 codes [rows, cols], float32 scales [rows])."""
    w = _widen(w_bf16_bits)
    if w.ndim != 2:
        raise ValueError("quantize_int8 takes a matrix")
    with np.errstate(invalid="ignore"):
        amax = np.nanmax(np.abs(w), axis=1) if w.shape[1] else np.zeros(w.shape[0], np.float32)
    amax = np.where(np.isnan(amax), np.float32(0), amax).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(INT8_MAX)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        q = np.rint((w / scale[:, None]).astype(np.float32))
    q = np.where(np.isnan(q), 0, np.clip(q, -INT8_MAX, INT8_MAX))
    return q.astype(np.int8), scale


def dequantize_int8(codes, scales) -> np.ndarray:
    """int8 codes [rows, cols] and float32 scales [rows] -> float64 weights (exact)."""
    return np.asarray(codes, dtype=np.int8).astype(np.float64) * \
        np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None]


# ---------------------------------------------------------------- MXFP8 ---

def e8m0_value(code) -> np.ndarray:
    """E8M0 byte(s) -> 2^(code - 127) as float64 (NaN for 255)."""
    c = np.asarray(code, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mx_shared_exponent(amax) -> np.ndarray:
    """X = floor(log2(amax)) - 8 for amax > 0, clamped to [-127, 127]; -127 for amax == 0."""
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(a)                        # a = m 2^e, 1/2 <= m < 1  =>  floor(log2 a) = e - 1
    X = np.where(a > 0, e - 1 - E4M3_EMAX, -127)
    return np.clip(X, -127, 127).astype(np.int64)


def quantize_mxfp8(w_bf16_bits):
    """bf16 weight [rows, cols] (cols % 32 == 0) -> (E4M3 codes [rows, cols],
    E8M0 scales [rows, cols / 32])."""
    w = _widen(w_bf16_bits)
    if w.ndim != 2 or w.shape[1] % MX_BLOCK:
        raise ValueError("quantize_mxfp8 takes a matrix whose columns are a multiple of 32")
    rows, cols = w.shape
    blocks = w.reshape(rows, cols // MX_BLOCK, MX_BLOCK)
    with np.errstate(invalid="ignore"):
        amax = np.nanmax(np.abs(blocks), axis=2) if cols else np.zeros((rows, 0), np.float32)
    amax = np.where(np.isnan(amax), 0, amax)
    X = mx_shared_exponent(amax)
    scaled = (blocks.astype(np.float64) * np.ldexp(1.0, -X)[:, :, None]).astype(np.float32)  # exact
    codes = fp8.encode_e4m3(scaled).reshape(rows, cols)
    return codes, (X + 127).astype(np.uint8)


def dequantize_mxfp8(codes, scales) -> np.ndarray:
    """E4M3 codes [rows, cols] and E8M0 scales [rows, cols / 32] -> float64 weights (exact)."""
    c = np.asarray(codes, dtype=np.uint8)
    rows, cols = c.shape
    v = fp8.DECODE[c].reshape(rows, cols // MX_BLOCK, MX_BLOCK) * e8m0_value(scales)[:, :, None]
    return v.reshape(rows, cols)


# ---------------------------------------------------------------- blocks --

def quantize_block(params, form: str):
    """A bf16 DiT block's parameter list -> its INT8 ("int8") or MXFP8 ("mxfp8") form.

    Every bf16 matrix ``X.weight`` [out, in] becomes ``X.weight`` (int8 codes, or
    E4M3 codes as "fp8") followed by ``X.weight_scale`` (fp32 [out], or E8M0
    [in / 32, out] block-major as "e8m0"); fp32 parameters stay as they are, so
    each linear registers weight, weight_scale, bias.
    """
    out = []
    for name, dt, arr in params:
        if dt != "bf16":
            out.append((name, dt, arr))
            continue
        a = np.asarray(arr, dtype=np.uint16)
        if form == "int8":
            codes, scale = quantize_int8(a)
            out += [(name, "i8", codes), (name + "_scale", "f32", scale)]
        elif form == "mxfp8":
            codes, scale = quantize_mxfp8(a)
            out += [(name, "fp8", codes), (name + "_scale", "e8m0", np.ascontiguousarray(scale.T).reshape(-1))]
        else:
            raise ValueError(f"unknown form {form!r}")
    return out


def fake_quant_mx_rows(x) -> np.ndarray:
    """What a W8A8 MXFP8 linear multiplies: the input rounded to bf16 (as stored),
    quantised per row in blocks of 32 (quantize_mxfp8), dequantised exactly."""
    from .forward import round_bf16
    r = round_bf16(x).astype(np.float32)                       # exact: bf16 values
    bits = (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    codes, scales = quantize_mxfp8(bits)
    return dequantize_mxfp8(codes, scales)


def fake_quant_int8_rows(x) -> np.ndarray:
    """What a W8A8 INT8 linear multiplies: the input rounded to bf16 (as stored),
    quantised per row by the INT8 rule (quantize_int8), dequantised exactly."""
    from .forward import round_bf16
    r = round_bf16(x).astype(np.float32)                       # exact: bf16 values
    bits = (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    codes, scales = quantize_int8(bits)
    return dequantize_int8(codes, scales)
