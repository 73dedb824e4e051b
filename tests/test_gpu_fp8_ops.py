"""GPU parity of the FP8 compute ops (W8A8) against the oracle, through the C-ABI.

* Per-row E4M3 quantization: codes and scales bit-exact with
  ``oracle.fp8.quantize_rows`` (both sides divide in IEEE float32 and round to
  the nearest even code, so the decision is taken in the same precision).
* FP8 GEMM: every product of two E4M3 codes is exact, but the FP8 matrix
  instruction does not add them as IEEE float32 does: small products beside a
  large one lose low bits (1 + 3 * 2^-15 comes back as 1).  Measured over full-
  range and normal-shaped codes, the worst element error is 2^-12 of
  sum_k |a_k b_k| (at K = 64; less for longer K), so the fp32-output check
  allows 2^-10 of that sum; the bf16-output checks use the bf16 GEMM tests'
  bound, whose output rounding term is far larger.
"""
import numpy as np
import pytest

import synth
import layerwise_weight_streaming_amd as dlo
from oracle import forward as of
from oracle import fp8
from tests.gpu_util import bf16_to_f64, rel_err, require_gpu, say

pytestmark = pytest.mark.gpu


def _close_bf16(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -9 * np.max(np.abs(ref))
    bad = np.abs(got - ref) > bound
    return int(bad.sum()), float(np.max(np.abs(got - ref) / np.maximum(bound, 1e-30)))


def _dev(torch, arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def _bf16_rand(seed, shape, std=1.0):
    return synth.normal_bf16(seed, 11, 0, 0, shape, 0.0, std)


def _as_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _quant_inputs(M, K, seed):
    """bf16 rows of mixed scale: plain normals, a zero row, a row with one outlier,
    rows spanning 2^-20 .. 2^8 (subnormal codes), a row of exact E4M3 ties and NaNs."""
    x = _bf16_rand(seed, (M, K))
    f = _as_f32(x).copy()
    rng = np.random.default_rng(seed)
    if M > 1:
        f[1] = 0.0
    if M > 2:
        f[2, rng.integers(0, K)] = 3.0e4
    if M > 3:
        f[3] *= np.exp2(rng.uniform(-20, 8, K)).astype(np.float32)
    if M > 4:
        # amax 448 -> scale 1: the row holds halfway points between neighbouring codes
        mid = (fp8.DECODE[0x30:0x37] + fp8.DECODE[0x31:0x38]) / 2
        f[4] = np.resize(np.concatenate([mid, -mid, [448.0]]), K)
        f[4, -1] = 448.0
    if M > 5:
        f[5, ::7] = np.nan
    return synth.f32_to_bf16(f)


@pytest.mark.parametrize("M,K,ldx_extra,ldq_extra", [(7, 64, 0, 0), (300, 5120, 8, 16), (33, 20480, 0, 8),
                                                      (1, 8, 0, 0), (129, 1032, 24, 0)])
def test_quantize_rows_bit_exact(M, K, ldx_extra, ldq_extra):
    torch = require_gpu()
    say("quantize rows", M, K, ldx_extra, ldq_extra)
    x = _quant_inputs(M, K, M * 13 + K)
    ldx, ldq = K + ldx_extra, K + ldq_extra
    xp = np.full((M, ldx), 0x7F7F, np.uint16)   # huge padding: read, it would change the scale
    xp[:, :K] = x
    dx = _dev(torch, xp.view(np.int16))
    dq = torch.full((M, ldq), 0xA5, dtype=torch.uint8, device="cuda")
    ds = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
    dlo.op_quantize_rows_fp8(dx.data_ptr(), ldx, M, K, dq.data_ptr(), ldq, ds.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    q, s = dq.cpu().numpy(), ds.cpu().numpy()
    codes, scales = fp8.quantize_rows(_as_f32(x))
    assert np.array_equal(s.view(np.uint32), scales.view(np.uint32))
    bad = np.argwhere(q[:, :K] != codes)
    assert bad.size == 0, (len(bad), bad[:5], q[tuple(bad[0])], codes[tuple(bad[0])])
    assert np.all(q[:, K:] == 0xA5)


def test_quantize_rows_rejects_unsupported_shapes():
    torch = require_gpu()
    x = torch.zeros((4, 64), dtype=torch.int16, device="cuda")
    q = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
    s = torch.zeros(4, dtype=torch.float32, device="cuda")
    for M, K, ldx, ldq in [(4, 60, 64, 64), (4, 64, 60, 64), (4, 64, 64, 56), (0, 64, 64, 64)]:
        with pytest.raises(dlo.DLOError):
            dlo.op_quantize_rows_fp8(x.data_ptr(), ldx, M, K, q.data_ptr(), ldq, s.data_ptr(), 0)


def _fp8_operands(M, N, K, seed):
    """A: per-row quantized bf16 activations; B: a per-tensor quantized bf16 weight."""
    a_codes, a_scale = fp8.quantize_rows(_as_f32(_bf16_rand(seed, (M, K))))
    b_codes, b_scale = fp8.quantize_tensor(_bf16_rand(seed + 1, (N, K), 0.05))
    return a_codes, a_scale, b_codes, np.float32(b_scale)


def _ref(a_codes, a_scale, b_codes, b_scale, bias):
    return of.linear(fp8.dequantize(a_codes, 1.0) * a_scale.astype(np.float64)[:, None],
                     fp8.dequantize(b_codes, b_scale), bias.astype(np.float64))


def _abs_products(a_codes, a_scale, b_codes, b_scale):
    """sum_k |a_mk b_nk| of the scaled operands, the scale of the FP8 instruction's addition error."""
    return (np.abs(fp8.dequantize(a_codes, 1.0)) * a_scale.astype(np.float64)[:, None]) @ \
        np.abs(fp8.dequantize(b_codes, b_scale)).T


def _run_gemm_fp8(torch, a_codes, a_scale, b_codes, b_scale, bias, gate, C, ldc, epi, M, N, K):
    dA, dsa, dB = _dev(torch, a_codes), _dev(torch, a_scale), _dev(torch, b_codes)
    dsb = torch.tensor([b_scale], dtype=torch.float32, device="cuda")
    db = _dev(torch, bias)
    dg = _dev(torch, gate) if gate is not None else None
    dlo.op_gemm_fp8(dA.data_ptr(), K, dsa.data_ptr(), dB.data_ptr(), K, dsb.data_ptr(), M, N, K,
                    db.data_ptr(), dg.data_ptr() if dg is not None else 0, C.data_ptr(), ldc, epi,
                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K", [(300, 512, 128), (64, 768, 256), (1000, 256, 320), (1, 256, 64),
                                   (129, 512, 64)])
@pytest.mark.parametrize("epi", [dlo.EPI_BIAS, dlo.EPI_BIAS_GELU, dlo.EPI_GATED_RESIDUAL, dlo.EPI_BIAS_T])
def test_gemm_fp8_small(M, N, K, epi):
    torch = require_gpu()
    say("gemm fp8", M, N, K, "epi", epi)
    a_codes, a_scale, b_codes, b_scale = _fp8_operands(M, N, K, M * 7 + N + K)
    bias = synth.normal_f32(3, 11, 1, 0, (N,), 0.0, 0.1)
    gate = synth.normal_f32(4, 11, 2, 0, (N,), 0.0, 1.0)
    ref = _ref(a_codes, a_scale, b_codes, b_scale, bias)
    if epi == dlo.EPI_GATED_RESIDUAL:
        X0 = synth.normal_f32(5, 11, 3, 0, (M, N))
        dX = _dev(torch, X0)
        _run_gemm_fp8(torch, a_codes, a_scale, b_codes, b_scale, bias, gate, dX, N, epi, M, N, K)
        got = dX.cpu().numpy().astype(np.float64)
        want = X0.astype(np.float64) + gate.astype(np.float64) * ref
        mag = _abs_products(a_codes, a_scale, b_codes, b_scale)
        bound = 2.0 ** -10 * np.abs(gate.astype(np.float64)) * mag + 2.0 ** -22 * (np.abs(want) + np.abs(X0))
        bad = np.abs(got - want) > bound
        assert not bad.any(), (int(bad.sum()), float(np.max(np.abs(got - want) / bound)))
        assert rel_err(got - X0, want - X0) < 1e-4
    elif epi == dlo.EPI_BIAS_T:
        M64 = (M + 63) // 64 * 64
        ldc = M64 + 8
        dCt = torch.full((N, ldc), 0x7FC0, dtype=torch.int16, device="cuda")
        _run_gemm_fp8(torch, a_codes, a_scale, b_codes, b_scale, bias, None, dCt, ldc, epi, M, N, K)
        dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        _run_gemm_fp8(torch, a_codes, a_scale, b_codes, b_scale, bias, None, dC, N, dlo.EPI_BIAS, M, N, K)
        ct = dCt.cpu().numpy().view(np.uint16)
        nbad, worst = _close_bf16(bf16_to_f64(ct[:, :M].T), ref)
        assert nbad == 0, (nbad, worst)
        assert np.all(ct[:, M:M64] == 0)
        assert np.all(ct[:, M64:] == 0x7FC0)
        assert np.array_equal(ct[:, :M].T, dC.cpu().numpy().view(np.uint16))
    else:
        dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        _run_gemm_fp8(torch, a_codes, a_scale, b_codes, b_scale, bias, None, dC, N, epi, M, N, K)
        got = bf16_to_f64(dC.cpu().numpy().view(np.uint16))
        want = of.gelu_erf(ref) if epi == dlo.EPI_BIAS_GELU else ref
        nbad, worst = _close_bf16(got, want)
        assert nbad == 0, (nbad, worst)


def _uniform_codes(seed, shape):
    """E4M3 codes spread over the whole table (the low byte of bf16 normals), NaN codes
    replaced by their neighbour 0x7E / 0xFE."""
    c = (synth.normal_bf16(seed, 12, 0, 0, shape, 0.0, 1.0) & 0xFF).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] ^= 0x01
    return c


def test_gemm_fp8_full_size_sampled():
    """FFN-up product of the Super workload in FP8 (M=28800, N=20480, K=5120), codes
    over the whole E4M3 range, sampled rows and columns."""
    torch = require_gpu()
    M, N, K = 28800, 20480, 5120
    say("gemm fp8 full size", M, N, K)
    A = _uniform_codes(21, (M, K))
    B = _uniform_codes(22, (N, K))
    a_scale = np.exp2(synth.normal_f32(23, 11, 1, 0, (M,), -8.0, 2.0)).astype(np.float32)
    b_scale = np.float32(3.0e-4)
    bias = synth.normal_f32(24, 11, 1, 0, (N,), 0.0, 0.02)
    dC = torch.empty((M, N), dtype=torch.int16, device="cuda")
    _run_gemm_fp8(torch, A, a_scale, B, b_scale, bias, None, dC, N, dlo.EPI_BIAS, M, N, K)
    rng = np.random.default_rng(1)
    rows = np.concatenate([rng.integers(0, M, 48), [0, M - 1, 28671, 28672]])
    cols = np.concatenate([rng.integers(0, N, 48), [0, N - 1, 255, 256]])
    C = dC[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16)[:, cols]
    ref = _ref(A[rows], a_scale[rows], B[cols], b_scale, bias[cols])
    nbad, worst = _close_bf16(bf16_to_f64(C), ref)
    assert nbad == 0, (nbad, worst)


@pytest.mark.parametrize("d", [256, 1024, 5120])
def test_adaln_fp8(d):
    """The adaLN GEMV on E4M3 codes: weights enter as code value * scale, exactly as
    the oracle dequantises them; fp32 accumulation over d terms."""
    torch = require_gpu()
    say("adaln fp8", d)
    codes, scale = fp8.quantize_tensor(_bf16_rand(40 + d, (6 * d, d), 0.02))
    b = synth.normal_f32(41, 11, 0, 0, (6 * d,), 0.0, 0.02)
    c = synth.normal_f32(42, 11, 0, 0, (d,))
    dW, db, dc = _dev(torch, codes), _dev(torch, b), _dev(torch, c)
    ds = torch.tensor([scale], dtype=torch.float32, device="cuda")
    out = torch.zeros(6 * d, dtype=torch.float32, device="cuda")
    ws = torch.empty(4 * d, dtype=torch.uint8, device="cuda")
    dlo.op_adaln_fp8(dW.data_ptr(), ds.data_ptr(), db.data_ptr(), dc.data_ptr(), 6 * d, d, out.data_ptr(),
                     ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = of.linear(of.silu(c.astype(np.float64))[None, :], fp8.dequantize(codes, scale), b.astype(np.float64))[0]
    assert rel_err(out.cpu().numpy(), ref) < 1e-5
    with pytest.raises(dlo.DLOError):
        dlo.op_adaln_fp8(dW.data_ptr(), ds.data_ptr(), db.data_ptr(), dc.data_ptr(), 6 * d, d - 8,
                         out.data_ptr(), ws.data_ptr(), ws.numel(), 0)


def test_gemm_fp8_rejects_unsupported_shapes():
    torch = require_gpu()
    a = torch.zeros((64, 128), dtype=torch.uint8, device="cuda")
    b = torch.zeros((256, 128), dtype=torch.uint8, device="cuda")
    s = torch.ones(64, dtype=torch.float32, device="cuda")
    bias = torch.zeros(256, dtype=torch.float32, device="cuda")
    c = torch.zeros((64, 256), dtype=torch.int16, device="cuda")
    for M, N, K, lda, epi in [(64, 256, 96, 128, 0), (64, 200, 128, 128, 0), (64, 256, 128, 120, 0),
                              (64, 256, 128, 128, 4), (64, 256, 128, 128, dlo.EPI_GATED_RESIDUAL)]:
        with pytest.raises(dlo.DLOError):
            dlo.op_gemm_fp8(a.data_ptr(), lda, s.data_ptr(), b.data_ptr(), 128, s.data_ptr(), M, N, K,
                            bias.data_ptr(), 0, c.data_ptr(), 256, epi, 0)


# ---------------------------------------------------------------------------
# MXFP8 (W8A8 with E8M0 block scales applied by the matrix instruction)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,ldx_extra,lds_extra", [(7, 64, 0, 1), (300, 5120, 8, 20), (33, 20480, 0, 3),
                                                     (1, 32, 0, 0), (129, 1056, 24, 63)])
def test_quantize_rows_mxfp8_bit_exact(M, K, ldx_extra, lds_extra):
    torch = require_gpu()
    from oracle import quant
    say("quantize rows mxfp8", M, K, ldx_extra, lds_extra)
    x = _quant_inputs(M, K, M * 17 + K)
    ldx, lds = K + ldx_extra, M + lds_extra
    xp = np.full((M, ldx), 0x7F7F, np.uint16)
    xp[:, :K] = x
    dx = _dev(torch, xp.view(np.int16))
    dq = torch.full((M, K), 0xA5, dtype=torch.uint8, device="cuda")
    ds = torch.full((K // 32, lds), 0xEE, dtype=torch.uint8, device="cuda")
    dlo.op_quantize_rows_mxfp8(dx.data_ptr(), ldx, M, K, dq.data_ptr(), K, ds.data_ptr(), lds,
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    q, s = dq.cpu().numpy(), ds.cpu().numpy()
    codes, scales = quant.quantize_mxfp8(x)
    assert np.array_equal(s[:, :M], scales.T)
    assert np.all(s[:, M:] == 127)
    bad = np.argwhere(q != codes)
    assert bad.size == 0, (len(bad), bad[:5])


def _mx_operand(seed, rows, K, std, lds):
    """bf16 normals quantised by the oracle: codes [rows, K], scales block-major [K / 32, lds]
    (padding rows 127, as the quantizer op leaves them)."""
    from oracle import quant
    codes, sc = quant.quantize_mxfp8(_bf16_rand(seed, (rows, K), std))
    blk = np.full((K // 32, lds), 127, np.uint8)
    blk[:, :rows] = sc.T
    return codes, blk


def _mx_ref(a_codes, a_blk, b_codes, b_blk, bias):
    from oracle import quant
    M, N = a_codes.shape[0], b_codes.shape[0]
    a = quant.dequantize_mxfp8(a_codes, a_blk[:, :M].T)
    b = quant.dequantize_mxfp8(b_codes, b_blk[:, :N].T)
    return of.linear(a, b, bias.astype(np.float64)), np.abs(a) @ np.abs(b).T


@pytest.mark.parametrize("M,N,K,b_pad", [(300, 512, 128, 0), (64, 768, 256, 256), (1000, 256, 320, 0),
                                         (1, 256, 64, 4), (129, 512, 64, 0)])
@pytest.mark.parametrize("epi", [dlo.EPI_BIAS, dlo.EPI_BIAS_GELU, dlo.EPI_GATED_RESIDUAL, dlo.EPI_BIAS_T])
def test_gemm_mxfp8_small(M, N, K, b_pad, epi):
    """b_pad > 0: B's scales sit at a column offset inside a wider block-major array
    (lds_b = N + 2 b_pad, base + b_pad), as a slice of the fused qkv weight does."""
    torch = require_gpu()
    say("gemm mxfp8", M, N, K, "epi", epi, "b_pad", b_pad)
    lds_a = (M + 3) // 4 * 4
    a_codes, a_blk = _mx_operand(M * 7 + N + K, M, K, 1.0, lds_a)
    b_codes, b_blk = _mx_operand(M * 7 + N + K + 1, N, K, 0.05, N)
    lds_b = N + 2 * b_pad
    b_wide = np.full((K // 32, lds_b), 0xFF, np.uint8)      # NaN scales outside the slice
    b_wide[:, b_pad:b_pad + N] = b_blk
    bias = synth.normal_f32(3, 11, 1, 0, (N,), 0.0, 0.1)
    gate = synth.normal_f32(4, 11, 2, 0, (N,), 0.0, 1.0)
    ref, mag = _mx_ref(a_codes, a_blk, b_codes, b_blk, bias)
    dA, dsa, dB, dsb = _dev(torch, a_codes), _dev(torch, a_blk), _dev(torch, b_codes), _dev(torch, b_wide)
    db, dg = _dev(torch, bias), _dev(torch, gate)
    s = torch.cuda.current_stream().cuda_stream

    def run(C, ldc, e, g=0):
        dlo.op_gemm_mxfp8(dA.data_ptr(), K, dsa.data_ptr(), lds_a, dB.data_ptr(), K, dsb.data_ptr() + b_pad, lds_b,
                          M, N, K, db.data_ptr(), g, C.data_ptr(), ldc, e, s)
        torch.cuda.synchronize()

    if epi == dlo.EPI_GATED_RESIDUAL:
        X0 = synth.normal_f32(5, 11, 3, 0, (M, N))
        dX = _dev(torch, X0)
        run(dX, N, epi, dg.data_ptr())
        got = dX.cpu().numpy().astype(np.float64)
        want = X0.astype(np.float64) + gate.astype(np.float64) * ref
        bound = 2.0 ** -10 * np.abs(gate.astype(np.float64)) * mag + 2.0 ** -22 * (np.abs(want) + np.abs(X0))
        bad = np.abs(got - want) > bound
        assert not bad.any(), (int(bad.sum()), float(np.max(np.abs(got - want) / bound)))
    elif epi == dlo.EPI_BIAS_T:
        M64 = (M + 63) // 64 * 64
        ldc = M64 + 8
        dCt = torch.full((N, ldc), 0x7FC0, dtype=torch.int16, device="cuda")
        run(dCt, ldc, epi)
        dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        run(dC, N, dlo.EPI_BIAS)
        ct = dCt.cpu().numpy().view(np.uint16)
        nbad, worst = _close_bf16(bf16_to_f64(ct[:, :M].T), ref)
        assert nbad == 0, (nbad, worst)
        assert np.all(ct[:, M:M64] == 0) and np.all(ct[:, M64:] == 0x7FC0)
        assert np.array_equal(ct[:, :M].T, dC.cpu().numpy().view(np.uint16))
    else:
        dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        run(dC, N, epi)
        got = bf16_to_f64(dC.cpu().numpy().view(np.uint16))
        want = of.gelu_erf(ref) if epi == dlo.EPI_BIAS_GELU else ref
        nbad, worst = _close_bf16(got, want)
        assert nbad == 0, (nbad, worst)


def test_gemm_mxfp8_full_size_sampled():
    """FFN-up product of the Super workload in MXFP8 (M=28800, N=20480, K=5120): codes over
    the whole E4M3 range and block scales from 2^-17 to 2^3, sampled rows and columns."""
    torch = require_gpu()
    from oracle import quant
    M, N, K = 28800, 20480, 5120
    say("gemm mxfp8 full size", M, N, K)
    A = _uniform_codes(31, (M, K))
    B = _uniform_codes(32, (N, K))
    rng = np.random.default_rng(33)
    sa = rng.integers(110, 131, (K // 32, M)).astype(np.uint8)
    sb = rng.integers(110, 131, (K // 32, N)).astype(np.uint8)
    bias = synth.normal_f32(34, 11, 1, 0, (N,), 0.0, 0.02)
    dA, dsa, dB, dsb, db = _dev(torch, A), _dev(torch, sa), _dev(torch, B), _dev(torch, sb), _dev(torch, bias)
    dC = torch.empty((M, N), dtype=torch.int16, device="cuda")
    dlo.op_gemm_mxfp8(dA.data_ptr(), K, dsa.data_ptr(), M, dB.data_ptr(), K, dsb.data_ptr(), N, M, N, K,
                      db.data_ptr(), 0, dC.data_ptr(), N, dlo.EPI_BIAS, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rows = np.concatenate([rng.integers(0, M, 48), [0, M - 1, 28671, 28672]])
    cols = np.concatenate([rng.integers(0, N, 48), [0, N - 1, 255, 256]])
    C = dC[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16)[:, cols]
    a = quant.dequantize_mxfp8(A[rows], sa[:, rows].T)
    b = quant.dequantize_mxfp8(B[cols], sb[:, cols].T)
    ref = of.linear(a, b, bias[cols].astype(np.float64))
    nbad, worst = _close_bf16(bf16_to_f64(C), ref)
    assert nbad == 0, (nbad, worst)


def test_mxfp8_ops_reject_unsupported_shapes():
    torch = require_gpu()
    a = torch.zeros((64, 128), dtype=torch.uint8, device="cuda")
    b = torch.zeros((256, 128), dtype=torch.uint8, device="cuda")
    s = torch.ones(4096, dtype=torch.uint8, device="cuda")
    bias = torch.zeros(256, dtype=torch.float32, device="cuda")
    c = torch.zeros((64, 256), dtype=torch.int16, device="cuda")
    for M, N, K, lds_a, lds_b in [(64, 256, 96, 64, 256), (64, 256, 128, 62, 256), (64, 256, 128, 66, 256),
                                  (64, 256, 128, 64, 254), (64, 200, 128, 64, 200)]:
        with pytest.raises(dlo.DLOError):
            dlo.op_gemm_mxfp8(a.data_ptr(), 128, s.data_ptr(), lds_a, b.data_ptr(), 128, s.data_ptr(), lds_b, M, N, K,
                              bias.data_ptr(), 0, c.data_ptr(), 256, 0, 0)
    x = torch.zeros((4, 64), dtype=torch.int16, device="cuda")
    for M, K, lds in [(4, 48, 4), (4, 64, 3)]:
        with pytest.raises(dlo.DLOError):
            dlo.op_quantize_rows_mxfp8(x.data_ptr(), 64, M, K, a.data_ptr(), 64, s.data_ptr(), lds, 0)
