"""Pins for oracle.fp8: E4M3 code values from the format definition, nearest-even
encoding with saturation, per-tensor scaling, and the FP8 block's parameter form."""
import numpy as np
import pytest

import synth
from oracle import fp8
from oracle import forward as of


def test_code_values_from_the_format_definition():
    # OCP FP8 E4M3: bias 7, subnormals m * 2^-9, S.1111.111 = NaN, max 448
    assert fp8.DECODE[0x00] == 0.0 and np.signbit(fp8.DECODE[0x80])
    assert fp8.DECODE[0x38] == 1.0
    assert fp8.DECODE[0x7E] == 448.0 and fp8.DECODE[0xFE] == -448.0
    assert fp8.DECODE[0x08] == 2.0 ** -6          # smallest normal
    assert fp8.DECODE[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert fp8.DECODE[0x01] == 2.0 ** -9          # smallest subnormal
    assert fp8.DECODE[0x3C] == 1.5 and fp8.DECODE[0x40] == 2.0
    assert np.isnan(fp8.DECODE[0x7F]) and np.isnan(fp8.DECODE[0xFF])
    assert np.sum(np.isnan(fp8.DECODE)) == 2      # no infinities, two NaN codes


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if not np.isnan(fp8.DECODE[c])], dtype=np.uint8)
    vals = fp8.DECODE[codes].astype(np.float32)
    assert np.array_equal(fp8.encode_e4m3(vals), codes)


def test_nearest_even_ties_and_saturation():
    # midpoints between neighbouring codes go to the even code
    pos = [c for c in range(0x7F)]
    for c in pos[:-1]:
        mid = np.float32((fp8.DECODE[c] + fp8.DECODE[c + 1]) / 2)
        want = c if c % 2 == 0 else c + 1
        assert fp8.encode_e4m3(mid)[()] == want, hex(c)
        assert fp8.encode_e4m3(-mid)[()] == want | 0x80
    # beyond the largest finite value: saturate, never NaN
    for v in (448.0, 460.0, 464.0, 480.0, 1e6, np.float32(3e38)):
        assert fp8.encode_e4m3(np.float32(v))[()] == 0x7E
    assert fp8.encode_e4m3(np.float32(np.nan))[()] == 0x7F


def test_encoding_is_nearest_against_brute_force():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 4000), rng.normal(0, 0.01, 2000), rng.uniform(-500, 500, 2000)])
    x = x.astype(np.float32)
    codes = fp8.encode_e4m3(x)
    finite = np.array([c for c in range(256) if not np.isnan(fp8.DECODE[c])])
    for xi, ci in zip(x, codes):
        a = min(abs(float(xi)), 448.0)
        best = np.min(np.abs(np.abs(fp8.DECODE[finite]) - a))
        assert abs(abs(fp8.DECODE[ci]) - a) == best
        assert (fp8.DECODE[ci] < 0) == (xi < 0) or fp8.DECODE[ci] == 0


def test_tensor_scale_maps_amax_to_448_and_error_bound():
    rng = np.random.default_rng(1)
    w = (rng.normal(0, 0.02, (64, 96)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    codes, scale = fp8.quantize_tensor(w)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    amax = np.max(np.abs(wf))
    assert scale == np.float32(np.float32(amax) / np.float32(448.0))
    assert np.max(np.abs(fp8.DECODE[codes])) == 448.0
    deq = fp8.dequantize(codes, scale)
    # 3 mantissa bits: relative error <= 2^-4 for normal codes; absolute error
    # <= half the subnormal step below
    err = np.abs(deq - wf)
    bound = np.maximum(np.abs(wf) * 2.0 ** -4, 2.0 ** -10 * float(scale))
    assert np.all(err <= bound * (1 + 1e-12))
    # an all-zero tensor keeps scale 1 and zero codes
    z, s = fp8.quantize_tensor(np.zeros(10, np.uint16))
    assert s == 1.0 and not z.any()


def test_fp8_block_form_and_forward_plumbing():
    d, T = 256, 16
    ps = synth.block_params(3, 0, d)
    q = fp8.quantize_block(ps)
    names = [n for n, _, _ in q]
    # registration order: weight, weight_scale, bias for each linear
    for lin in ("adaln", "attn.qkv", "attn.out", "mlp.fc1", "mlp.fc2"):
        i = names.index(lin + ".weight")
        assert names[i + 1] == lin + ".weight_scale" and names[i + 2] == lin + ".bias"
    assert len(q) == len(ps) + 5
    # the FP8 block's forward is the bf16 block's forward with the dequantised weights
    P = of.param_dict(q)
    P_ref = of.param_dict(ps)
    for n, dt, a in q:
        if dt == "fp8":
            scale = dict((m, b) for m, _, b in q)[n + "_scale"][0]
            P_ref[n] = fp8.dequantize(a, scale)
            assert np.array_equal(P[n], P_ref[n])
    x = np.random.default_rng(2).normal(size=(T, d))
    c = np.random.default_rng(3).normal(size=d)
    assert np.array_equal(of.dit_block(x, c, P, 4), of.dit_block(x, c, P_ref, 4))
    # and it differs from the bf16 block by the quantisation only (a few percent of the update)
    y_bf16, y_fp8 = of.dit_block(x, c, of.param_dict(ps), 4), of.dit_block(x, c, P, 4)
    upd = np.max(np.abs(y_bf16 - x))
    assert 0 < np.max(np.abs(y_fp8 - y_bf16)) < 0.2 * upd


# ---------------------------------------------------------------------------
# per-token activation quantization (the W8A8 reading of an FP8 block's linears)
# ---------------------------------------------------------------------------

def _nearest_code_brute(v):
    """Index of the finite E4M3 value nearest to v; ties to the even code (v finite)."""
    best = None
    for c in range(256):
        val = fp8.DECODE[c]
        if np.isnan(val) or (val == 0 and c == 0x80):
            continue
        dist = abs(val - v)
        if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (dist, c)
    return best[1]


def test_quantize_rows_against_brute_force_and_per_row_amax():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((6, 40)) * np.array([1e-3, 0.1, 1, 7, 300, 2e4])[:, None]).astype(np.float32)
    codes, scale = fp8.quantize_rows(x)
    for r in range(6):
        amax = np.float32(np.max(np.abs(x[r])))
        assert scale[r] == np.float32(amax / np.float32(448.0))
        for j in range(40):
            y = np.float32(x[r, j] / scale[r])
            c = int(codes[r, j])
            v = abs(float(y))
            want = _nearest_code_brute(min(v, 448.0)) | (0x80 if y < 0 else 0)
            assert c == want, (r, j, y, c, want)
        # the largest magnitude maps to +-448 (code 0x7E / 0xFE)
        jmax = int(np.argmax(np.abs(x[r])))
        assert codes[r, jmax] & 0x7F == 0x7E


def test_quantize_rows_zero_rows_scaling_and_error_bound():
    x = np.zeros((3, 8), np.float32)
    x[1] = [1, -2, 3, -4, 5, -6, 7, -8]
    x[2] = x[1] * 64          # a power of two scales the scale, not the codes
    codes, scale = fp8.quantize_rows(x)
    assert scale[0] == 1.0 and np.all(codes[0] == 0)
    assert scale[2] == scale[1] * 64 and np.array_equal(codes[1], codes[2])
    # relative error of a normal-range element at most half a 3-bit mantissa step, 2^-4
    rng = np.random.default_rng(12)
    y = rng.standard_normal((50, 64)).astype(np.float32)
    deq = fp8.fake_quant_rows(y)
    big = np.abs(y) >= (np.max(np.abs(y), axis=1, keepdims=True) / 448.0) * 2.0 ** -6
    assert np.all(np.abs(deq - y)[big] <= 2.0 ** -4 * np.abs(y)[big] * (1 + 1e-6))


def test_w8a8_block_is_close_to_the_bf16_block_and_keeps_the_identity():
    d, H, T = 64, 2, 12
    blk = fp8.quantize_block(synth.block_params(3, 0, d))
    P = of.param_dict(blk)
    rng = np.random.default_rng(13)
    x, c = rng.standard_normal((T, d)), rng.standard_normal(d)
    y = of.dit_block(x, c, P, H)
    yq = of.dit_block(x, c, P, H, act_fp8=True)
    upd, updq = y - x, yq - x
    err = np.max(np.abs(updq - upd)) / np.max(np.abs(upd))
    assert 0 < err < 0.1        # FP8 inputs move the update by a few percent, not more
    # adaLN-zero: gates 0 => output == input, quantized or not
    P0 = dict(P)
    P0["adaln.weight"] = np.zeros_like(P["adaln.weight"])
    P0["adaln.bias"] = np.zeros_like(P["adaln.bias"])
    assert np.array_equal(of.dit_block(x, c, P0, H, act_fp8=True), x)


def test_round_bf16_is_the_nearest_even_bf16_value():
    """Against the input generator's float32 -> bf16 rounding (a bit-level routine, not
    the oracle's frexp form) on float32 inputs, and by the definition on float64 ones:
    the result is a bf16 value, no bf16 value lies closer, and exact midpoints go to
    the even significand."""
    rng = np.random.default_rng(5)
    x32 = (rng.standard_normal(20000) * np.exp2(rng.uniform(-40, 40, 20000))).astype(np.float32)
    want = (synth.f32_to_bf16(x32).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(of.round_bf16(x32.astype(np.float64)), want)
    x = rng.standard_normal(20000) * np.exp2(rng.uniform(-20, 20, 20000))
    r = of.round_bf16(x)
    r32 = r.astype(np.float32)
    assert np.array_equal(r32.astype(np.float64), r)                 # a float32 ...
    assert np.all(r32.view(np.uint32) & 0xFFFF == 0)                  # ... with 8 significant bits
    up = (r32.view(np.uint32) + np.where(r >= 0, 0x10000, -0x10000).astype(np.uint32)).view(np.float32)
    dn = (r32.view(np.uint32) - np.where(r >= 0, 0x10000, -0x10000).astype(np.uint32)).view(np.float32)
    for nb in (up, dn):                                                # neighbours are no closer
        assert np.all(np.abs(x - r) <= np.abs(x - nb.astype(np.float64)))
    # midpoints between consecutive bf16 values 1 + j/128 and 1 + (j+1)/128
    j = np.arange(128)
    mid = 1.0 + (j + 0.5) / 128.0
    got = of.round_bf16(np.concatenate([mid, -mid * 2.0 ** -30]))
    even = 1.0 + np.where(j % 2 == 0, j, j + 1) / 128.0
    assert np.array_equal(got, np.concatenate([even, -even * 2.0 ** -30]))
    assert of.round_bf16(0.0) == 0.0 and of.round_bf16(2.0 ** -140) == 0.0
    assert of.round_bf16(3 * 2.0 ** -134) == 2.0 ** -132             # subnormal tie to even
