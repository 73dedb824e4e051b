"""Oracle: FP8 E4M3 weight codes and per-tensor quantisation (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
use this package; the GPU path shares no code with it.

The pages let per-tensor online FP8 linears take the same sharding path: the
loader first finalises a 1-byte weight and an fp32 scale per tensor, and the
method then shards and reassembles those tensors by their recorded layouts like
any other dtype group ([Doc] "Request and loading constraints", the paragraph
on online FP8, INT8 and MXFP8 linears).  The pages do not fix the FP8 variant or
the scaling rule; the readings here:

* the code is OCP FP8 E4M3 ("E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa
  bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; there is
  no infinity; the largest finite magnitude is 448;
* per-tensor scale = amax(|w|) / 448 computed in float32 (1.0 for an all-zero
  tensor); the code of w is the E4M3 value nearest to float32(w) / scale,
  ties to the even code, magnitudes above 448 saturating to 448 (the
  "saturate to finite" conversion);
* the dequantised weight the block uses is code_value * scale.

Encoding here searches the table of all finite codes for the nearest value --
a different procedure from the arithmetic one in the library, checked equal
byte for byte by the tests.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code (NaN for S.1111.111), from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# all 256 codes decoded, and the finite non-negative ones sorted by value
DECODE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_POS_CODES = np.array([c for c in range(0x80) if not np.isnan(DECODE[c])], dtype=np.int64)
_POS_VALUES = DECODE[_POS_CODES]
assert np.all(np.diff(_POS_VALUES) > 0)


def encode_e4m3(x) -> np.ndarray:
    """float32 values -> E4M3 codes: nearest finite code, ties to the even code, saturating.

    NaN maps to 0x7F.  The sign is carried separately, so -0.0 gives 0x80.
    """
    x = np.asarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_x, flat_o = x.reshape(-1), out.reshape(-1)
    last = len(_POS_VALUES) - 1
    for s0 in range(0, flat_x.size, 1 << 22):
        v = flat_x[s0:s0 + (1 << 22)].astype(np.float64)
        a = np.minimum(np.abs(v), E4M3_MAX)
        j = np.searchsorted(_POS_VALUES, a)             # first table value >= a
        hi = np.minimum(j, last)
        lo = np.maximum(j - 1, 0)
        dlo, dhi = a - _POS_VALUES[lo], _POS_VALUES[hi] - a
        c_lo, c_hi = _POS_CODES[lo], _POS_CODES[hi]
        pick_hi = (dhi < dlo) | ((dhi == dlo) & (c_hi % 2 == 0))
        c = np.where(pick_hi, c_hi, c_lo)
        c = np.where(_POS_VALUES[hi] == a, c_hi, c)     # exact hit (also a = 0)
        c = c | np.where(np.signbit(v), 0x80, 0)
        c = np.where(np.isnan(v), 0x7F, c)
        flat_o[s0:s0 + c.size] = c.astype(np.uint8)
    return out


def tensor_scale(w_bf16_bits: np.ndarray) -> np.float32:
    """Per-tensor scale amax / 448 in float32 (1.0 if the tensor is all zero)."""
    w = (np.asarray(w_bf16_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    amax = np.float32(np.nanmax(np.abs(w))) if w.size else np.float32(0)   # NaN entries ignored
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E4M3_MAX))


def quantize_tensor(w_bf16_bits: np.ndarray):
    """bf16 weight (bit patterns) -> (E4M3 codes, float32 scale)."""
    scale = tensor_scale(w_bf16_bits)
    w = (np.asarray(w_bf16_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return encode_e4m3(w / scale), scale


def dequantize(codes: np.ndarray, scale) -> np.ndarray:
    """E4M3 codes and a scale -> float64 weights (code value * scale, exact)."""
    return DECODE[np.asarray(codes, dtype=np.uint8)] * np.float64(np.float32(scale))


def quantize_rows(x):
    """Per-row (per-token) dynamic E4M3 of an activation matrix [M, K].

    The reading of an online FP8 linear's input (the pages leave it open): row r
    gets scale_r = amax_r / 448 in float32 (NaN entries
    ignored, 1.0 for an all-zero row), and each element the E4M3 code nearest to
    float32(x) / scale_r, the division in float32, ties to the even code,
    saturating at +-448.  Returns (codes uint8 [M, K], scales float32 [M]).
    """
    x32 = np.asarray(x, dtype=np.float32)
    if x32.ndim != 2:
        raise ValueError("quantize_rows takes a matrix")
    if x32.shape[1] == 0:
        return np.zeros(x32.shape, dtype=np.uint8), np.ones(x32.shape[0], dtype=np.float32)
    with np.errstate(invalid="ignore"):
        amax = np.nanmax(np.abs(x32), axis=1).astype(np.float32)
    amax = np.where(np.isnan(amax), np.float32(0), amax).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        codes = encode_e4m3((x32 / scale[:, None]).astype(np.float32))
    return codes, scale


def fake_quant_rows(x):
    """What an FP8 linear multiplies: the per-row codes times their scales, in float64."""
    codes, scale = quantize_rows(x)
    return DECODE[codes] * scale.astype(np.float64)[:, None]


def quantize_block(params):
    """A bf16 DiT block's parameter list -> its per-tensor FP8 form.

    Every bf16 matrix ``X.weight`` becomes (``X.weight``, "fp8", codes) followed by
    (``X.weight_scale``, "f32", [scale]); fp32 parameters stay as they are, so
    the registration order is weight, weight_scale, bias for each linear.
    """
    out = []
    for name, dt, arr in params:
        if dt == "bf16":
            codes, scale = quantize_tensor(arr)
            out.append((name, "fp8", codes))
            out.append((name + "_scale", "f32", np.array([scale], dtype=np.float32)))
        else:
            out.append((name, dt, arr))
    return out
