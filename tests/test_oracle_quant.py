"""Pins of the INT8 and MXFP8 weight forms of the oracle (oracle/quant.py).

Each check uses a procedure other than the oracle's: exhaustive search over all
candidate codes, the shared exponent found by doubling, exact power-of-two
arithmetic, and block-by-block independence.
"""
import numpy as np
import pytest

import synth
from oracle import forward as of
from oracle import fp8, quant


def _bf16(x):
    return synth.f32_to_bf16(np.asarray(x, np.float32))


def _f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_int8_codes_are_the_nearest_integers_by_exhaustive_search():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 40)) * np.exp2(rng.uniform(-6, 6, (6, 1)))
    x[2, 5] = 40.0                          # an outlier
    x[3] = 0.0                              # a zero row
    w = _bf16(x)
    codes, scale = quant.quantize_int8(w)
    assert codes.dtype == np.int8 and scale.dtype == np.float32
    cand = np.arange(-127, 128, dtype=np.float64)
    for r in range(w.shape[0]):
        y = (_f32(w[r]) / scale[r]).astype(np.float64)      # the float32 quotient
        for j, v in enumerate(y):
            dist = np.abs(cand - v)
            best = cand[dist == dist.min()]
            want = best[0] if best.size == 1 else best[best % 2 == 0][0]   # ties to even
            assert codes[r, j] == want, (r, j, v, codes[r, j], want)
    # the row's largest magnitude maps to +-127; a zero row has scale 1 and zero codes
    for r in (0, 1, 2, 4, 5):
        assert np.max(np.abs(codes[r].astype(int))) == 127
    assert scale[3] == 1.0 and np.all(codes[3] == 0)
    # scale = amax / 127 in float32
    amax = np.max(np.abs(_f32(w)), axis=1)
    assert np.array_equal(scale[amax > 0], (amax / np.float32(127))[amax > 0])


def test_int8_error_bound_and_power_of_two_rows():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    w = _bf16(x)
    codes, scale = quant.quantize_int8(w)
    deq = quant.dequantize_int8(codes, scale)
    # half a step, plus the float32 rounding of the quotient (at most 127 * 2^-24 of a step)
    assert np.all(np.abs(deq - _f32(w)) <= scale[:, None] * (0.5 + 127 * 2.0 ** -24) * (1 + 1e-12))
    # multiplying a row by 2^k scales its scale by 2^k and keeps its codes
    w2 = _bf16(_f32(w) * np.float32(2.0 ** 5))
    c2, s2 = quant.quantize_int8(w2)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scale * np.float32(32))


def _shared_exp_by_doubling(a):
    """Largest integer e with 2^e <= a (a > 0), by repeated doubling and halving."""
    e, p = 0, 1.0
    while p > a:
        p /= 2
        e -= 1
    while p * 2 <= a:
        p *= 2
        e += 1
    return e


def test_mx_shared_exponent_and_codes():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 128)) * np.exp2(rng.uniform(-10, 10, (4, 128)))
    x[1, 32:64] = 0.0                        # an all-zero block
    x[2, 64:96] = 2.0 ** -3                  # a constant power of two
    x[3, 96:128] = rng.uniform(-1, 1, 32)
    x[3, 100] = -1.96                        # scaled by 2^8 to 502: saturates to -448
    w = _bf16(x)
    codes, scales = quant.quantize_mxfp8(w)
    assert codes.shape == w.shape and scales.shape == (4, 4) and scales.dtype == np.uint8
    wf = _f32(w).astype(np.float64)
    for r in range(4):
        for b in range(4):
            blk = wf[r, 32 * b:32 * b + 32]
            amax = np.max(np.abs(blk))
            if amax == 0:
                assert scales[r, b] == 0 and np.all(codes[r, 32 * b:32 * b + 32] == 0)
                continue
            X = _shared_exp_by_doubling(amax) - 8
            assert scales[r, b] == X + 127
            y = blk / 2.0 ** X
            assert 256 <= np.max(np.abs(y)) < 512          # the block's amax lands in [2^8, 2^9)
            for j, v in enumerate(y):
                d = np.abs(fp8.DECODE[:0x7F] - min(abs(v), 448.0))   # finite non-negative codes
                d[np.isnan(d)] = np.inf
                best = np.flatnonzero(d == d.min())
                want = best[0] if best.size == 1 else best[best % 2 == 0][0]
                want |= 0x80 if v < 0 else 0
                assert codes[r, 32 * b + j] == want, (r, b, j, v)
    # the constant block: 2^-3 = 2^8 * 2^X with X = -11, code 0x78 (2^8)
    assert scales[2, 2] == 127 - 11 and np.all(codes[2, 64:96] == 0x78)
    assert scales[3, 3] == 127 - 8 and codes[3, 100] == 0xFE


def test_mx_dequantisation_is_exact_and_blocks_are_independent():
    rng = np.random.default_rng(4)
    w = _bf16(rng.standard_normal((3, 96)))
    codes, scales = quant.quantize_mxfp8(w)
    deq = quant.dequantize_mxfp8(codes, scales)
    want = fp8.DECODE[codes] * np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
    assert np.array_equal(deq, want)
    # relative error of a normal-range element within half a 3-bit mantissa step; the
    # scaled block maximum lies in [256, 512), so elements above 448 saturate to 448
    # (relative error below 1/8)
    unit = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    y = np.abs(_f32(w)) / unit
    err = np.abs(deq - _f32(w))
    normal = (y >= 2.0 ** -6) & (y <= 448)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(_f32(w))[normal] * (1 + 1e-9))
    sat = y > 464
    assert np.all(np.abs(deq[sat]) == 448 * unit[sat]) and np.all(err[sat] < np.abs(_f32(w))[sat] / 8)
    # changing one block leaves the others' codes and scales alone
    w2 = w.copy()
    w2[1, 32:64] = _bf16(_f32(w[1, 32:64]) * np.float32(1000.0))
    c2, s2 = quant.quantize_mxfp8(w2)
    mask = np.ones((3, 3), bool)
    mask[1, 1] = False
    assert np.array_equal(s2[mask], scales[mask]) and s2[1, 1] != scales[1, 1]
    keep = np.repeat(mask, 32, axis=1)
    assert np.array_equal(c2[keep], codes[keep])
    assert np.isnan(quant.e8m0_value(255)) and quant.e8m0_value(127) == 1.0


@pytest.mark.parametrize("form", ["int8", "mxfp8"])
def test_quantised_block_form_is_the_bf16_block_with_dequantised_weights(form):
    """The block form registers weight, weight_scale, bias per linear, and its forward is
    the bf16 forward run on the dequantised weights (bit for bit)."""
    d, H, T = 64, 2, 12
    params = synth.block_params(5, 0, d)
    q = quant.quantize_block(params, form)
    names = [n for n, _, _ in q]
    assert names[:3] == ["adaln.weight", "adaln.weight_scale", "adaln.bias"]
    assert len(q) == 21
    P = of.param_dict(q)
    deq = {}
    for name, dt, arr in q:
        if dt in ("i8", "fp8"):
            sc = dict((n, a) for n, _, a in q)[name + "_scale"]
            deq[name] = (quant.dequantize_int8(arr, sc) if form == "int8"
                         else quant.dequantize_mxfp8(arr, sc.reshape(-1, arr.shape[0]).T))
            assert np.array_equal(P[name], deq[name])
    rng = np.random.default_rng(6)
    x, c = rng.standard_normal((T, d)), rng.standard_normal(d)
    Pb = of.param_dict(params)
    Pb.update(deq)
    assert np.array_equal(of.dit_block(x, c, P, H), of.dit_block(x, c, Pb, H))
    # the quantised block stays close to the bf16 one
    y, yb = of.dit_block(x, c, P, H), of.dit_block(x, c, of.param_dict(params), H)
    assert np.max(np.abs((y - x) - (yb - x))) < 0.1 * np.max(np.abs(yb - x))


def test_mx_block_form_keeps_scales_block_major():
    """X.weight_scale of the MXFP8 form lists, for each 32-wide input block, the scales
    of all output rows: element (b, r) sits at b * out + r."""
    d = 64
    params = synth.block_params(7, 0, d)
    q = dict((n, (dt, a)) for n, dt, a in quant.quantize_block(params, "mxfp8"))
    w = dict((n, a) for n, _, a in params)["mlp.fc2.weight"]          # [d, 4d]
    _, rs = quant.quantize_mxfp8(w)                                   # [d, 4d / 32]
    dt, sc = q["mlp.fc2.weight_scale"]
    assert dt == "e8m0" and sc.size == d * 4 * d // 32
    for b in range(4 * d // 32):
        for r in range(d):
            assert sc[b * d + r] == rs[r, b]


def test_mx_activation_fake_quant():
    """W8A8 MXFP8 input: round to bf16, quantise per row in blocks of 32, dequantise;
    against the block rule written out for one row."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 64)) * np.exp2(rng.uniform(-8, 8, (3, 64)))
    y = quant.fake_quant_mx_rows(x)
    for r in range(3):
        for b in range(2):
            blk = of.round_bf16(x[r, 32 * b:32 * b + 32])
            X = _shared_exp_by_doubling(np.max(np.abs(blk))) - 8
            for j in range(32):
                v = blk[j] / 2.0 ** X
                d_ = np.abs(fp8.DECODE[:0x7F] - min(abs(v), 448.0))
                d_[np.isnan(d_)] = np.inf
                best = np.flatnonzero(d_ == d_.min())
                code = best[0] if best.size == 1 else best[best % 2 == 0][0]
                want = fp8.DECODE[code] * 2.0 ** X * (-1 if v < 0 else 1)
                assert y[r, 32 * b + j] == want
    # an MXFP8 block in the W8A8 form stays close to its W8A16 form
    d, H, T = 64, 2, 12
    P = of.param_dict(quant.quantize_block(synth.block_params(8, 0, d), "mxfp8"))
    xx, c = rng.standard_normal((T, d)), rng.standard_normal(d)
    y16, y8 = of.dit_block(xx, c, P, H), of.dit_block(xx, c, P, H, act_mx=True)
    err = np.max(np.abs((y8 - xx) - (y16 - xx))) / np.max(np.abs(y16 - xx))
    assert 0 < err < 0.1


def test_int8_activation_fake_quant():
    """W8A8 INT8 input: round to bf16, quantise per row by the INT8 rule, dequantise;
    against the rule written out (nearest integer by search, amax / 127 in float32)."""
    rng = np.random.default_rng(10)
    x = rng.standard_normal((4, 48)) * np.exp2(rng.uniform(-6, 6, (4, 1)))
    x[2] = 0.0
    y = quant.fake_quant_int8_rows(x)
    cand = np.arange(-127, 128, dtype=np.float64)
    for r in range(4):
        xb = of.round_bf16(x[r]).astype(np.float32)
        amax = np.float32(np.max(np.abs(xb)))
        s = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(127))
        for j in range(48):
            v = float(np.float32(xb[j] / s))
            d_ = np.abs(cand - v)
            best = cand[d_ == d_.min()]
            q = best[0] if best.size == 1 else best[best % 2 == 0][0]
            assert y[r, j] == q * float(s)
    assert np.all(y[2] == 0)
    # an INT8 block in the W8A8 form stays close to its W8A16 form
    d, H, T = 64, 2, 12
    P = of.param_dict(quant.quantize_block(synth.block_params(9, 0, d), "int8"))
    xx, c = rng.standard_normal((T, d)), rng.standard_normal(d)
    y16, y8 = of.dit_block(xx, c, P, H), of.dit_block(xx, c, P, H, act_int8=True)
    err = np.max(np.abs((y8 - xx) - (y16 - xx))) / np.max(np.abs(y16 - xx))
    assert 0 < err < 0.1
