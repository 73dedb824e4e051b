"""GPU parity of the W8A8 INT8 ops through the C-ABI: the per-row int8
quantisation of a linear's input (bit-exact against the oracle's INT8 rule) and
the int8 product (exact integer sums, checked against float64 integer
arithmetic), [Doc] "Request and loading constraints" (online INT8 linears)."""
import numpy as np
import pytest

import synth
import layerwise_weight_streaming_amd as dlo
from oracle import forward as of
from oracle import quant
from tests.gpu_util import bf16_to_f64, rel_err, require_gpu, say

pytestmark = pytest.mark.gpu


def _close_bf16(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -9 * np.max(np.abs(ref))
    bad = np.abs(got - ref) > bound
    return int(bad.sum()), float(np.max(np.abs(got - ref) / np.maximum(bound, 1e-30)))


def _dev(torch, arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def _as_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _quant_inputs(M, K, seed):
    """bf16 rows: plain normals, a zero row, a row with one outlier, a row spanning
    2^-20 .. 2^8, a row of exact ties (amax 127 -> scale 1, entries k + 1/2) and NaNs."""
    f = _as_f32(synth.normal_bf16(seed, 13, 0, 0, (M, K), 0.0, 1.0)).copy()
    rng = np.random.default_rng(seed)
    if M > 1:
        f[1] = 0.0
    if M > 2:
        f[2, rng.integers(0, K)] = 3.0e4
    if M > 3:
        f[3] *= np.exp2(rng.uniform(-20, 8, K)).astype(np.float32)
    if M > 4:
        ties = np.arange(-126, 126, dtype=np.float32) + 0.5
        f[4] = np.resize(ties, K)
        f[4, -1] = 127.0
    if M > 5:
        f[5, ::7] = np.nan
    return synth.f32_to_bf16(f)


@pytest.mark.parametrize("M,K,ldx_extra,ldq_extra", [(7, 64, 0, 0), (300, 5120, 8, 16), (33, 20480, 0, 8),
                                                      (1, 8, 0, 0), (129, 1032, 24, 0)])
def test_quantize_rows_int8_bit_exact(M, K, ldx_extra, ldq_extra):
    torch = require_gpu()
    say("quantize rows int8", M, K, ldx_extra, ldq_extra)
    x = _quant_inputs(M, K, M * 17 + K)
    ldx, ldq = K + ldx_extra, K + ldq_extra
    xp = np.full((M, ldx), 0x7F7F, np.uint16)   # huge padding: read, it would change the scale
    xp[:, :K] = x
    dx = _dev(torch, xp.view(np.int16))
    dq = torch.full((M, ldq), 0x55, dtype=torch.int8, device="cuda")
    ds = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
    dlo.op_quantize_rows_int8(dx.data_ptr(), ldx, M, K, dq.data_ptr(), ldq, ds.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    q, s = dq.cpu().numpy(), ds.cpu().numpy()
    codes, scales = quant.quantize_int8(x)
    assert np.array_equal(s.view(np.uint32), scales.view(np.uint32))
    bad = np.argwhere(q[:, :K] != codes)
    assert bad.size == 0, (len(bad), bad[:5], q[tuple(bad[0])], codes[tuple(bad[0])])
    assert np.all(q[:, K:] == 0x55)
    if M > 4:   # amax 127 (scale 1): the ties k + 1/2 went to the even neighbour
        n = min(K - 1, 252)
        assert s[4] == 1.0
        assert np.array_equal(q[4, :n], (2 * np.round((np.arange(-126, 126) + 0.5) / 2)).astype(np.int8)[:n])


def _operands(M, N, K, seed):
    """A: per-row int8 activations; B: a per-output-row int8 weight (both the oracle's rule)."""
    a_codes, a_scale = quant.quantize_int8(synth.normal_bf16(seed, 13, 1, 0, (M, K), 0.0, 1.0))
    b_codes, b_scale = quant.quantize_int8(synth.normal_bf16(seed + 1, 13, 2, 0, (N, K), 0.0, 0.05))
    return a_codes, a_scale, b_codes, b_scale


def _ref(a_codes, a_scale, b_codes, b_scale, bias):
    """Exact integer sums (float64 holds them exactly) times both scales, plus bias."""
    acc = a_codes.astype(np.float64) @ b_codes.astype(np.float64).T
    return acc * a_scale.astype(np.float64)[:, None] * b_scale.astype(np.float64)[None, :] + \
        bias.astype(np.float64)


def _run(torch, a_codes, a_scale, b_codes, b_scale, bias, gate, C, ldc, epi, M, N, K, b_off=0):
    dA, dsa, dB = _dev(torch, a_codes), _dev(torch, a_scale), _dev(torch, b_codes)
    # b_scale at a 4-B (not 16-B) offset, as in a packed block
    dsb = _dev(torch, np.concatenate([np.zeros(b_off, np.float32), b_scale]))
    db = _dev(torch, bias)
    dg = _dev(torch, gate) if gate is not None else None
    dlo.op_gemm_int8(dA.data_ptr(), K, dsa.data_ptr(), dB.data_ptr(), K, dsb.data_ptr() + 4 * b_off, M, N, K,
                     db.data_ptr(), dg.data_ptr() if dg is not None else 0, C.data_ptr(), ldc, epi,
                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K", [(300, 512, 128), (64, 768, 256), (1000, 256, 320), (1, 256, 64),
                                   (129, 512, 64)])
@pytest.mark.parametrize("epi", [dlo.EPI_BIAS, dlo.EPI_BIAS_GELU, dlo.EPI_GATED_RESIDUAL, dlo.EPI_BIAS_T])
def test_gemm_int8_small(M, N, K, epi):
    torch = require_gpu()
    say("gemm int8", M, N, K, "epi", epi)
    a_codes, a_scale, b_codes, b_scale = _operands(M, N, K, M * 7 + N + K)
    bias = synth.normal_f32(3, 13, 1, 0, (N,), 0.0, 0.1)
    gate = synth.normal_f32(4, 13, 2, 0, (N,), 0.0, 1.0)
    ref = _ref(a_codes, a_scale, b_codes, b_scale, bias)
    if epi == dlo.EPI_GATED_RESIDUAL:
        X0 = synth.normal_f32(5, 13, 3, 0, (M, N))
        dX = _dev(torch, X0)
        _run(torch, a_codes, a_scale, b_codes, b_scale, bias, gate, dX, N, epi, M, N, K, b_off=1)
        got = dX.cpu().numpy().astype(np.float64)
        want = X0.astype(np.float64) + gate.astype(np.float64) * ref
        # exact sums; only fp32 roundings of the scaling, bias, gate and residual remain
        mag = np.abs(ref - bias) + np.abs(bias)
        bound = 2.0 ** -21 * np.abs(gate.astype(np.float64)) * mag + 2.0 ** -22 * (np.abs(want) + np.abs(X0))
        bad = np.abs(got - want) > bound
        assert not bad.any(), (int(bad.sum()), float(np.max(np.abs(got - want) / bound)))
        assert rel_err(got - X0, want - X0) < 1e-5
    elif epi == dlo.EPI_BIAS_T:
        M64 = (M + 63) // 64 * 64
        ldc = M64 + 8
        dCt = torch.full((N, ldc), 0x7FC0, dtype=torch.int16, device="cuda")
        _run(torch, a_codes, a_scale, b_codes, b_scale, bias, None, dCt, ldc, epi, M, N, K, b_off=3)
        dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        _run(torch, a_codes, a_scale, b_codes, b_scale, bias, None, dC, N, dlo.EPI_BIAS, M, N, K)
        ct = dCt.cpu().numpy().view(np.uint16)
        nbad, worst = _close_bf16(bf16_to_f64(ct[:, :M].T), ref)
        assert nbad == 0, (nbad, worst)
        assert np.all(ct[:, M:M64] == 0)
        assert np.all(ct[:, M64:] == 0x7FC0)
        assert np.array_equal(ct[:, :M].T, dC.cpu().numpy().view(np.uint16))
    else:
        dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        _run(torch, a_codes, a_scale, b_codes, b_scale, bias, None, dC, N, epi, M, N, K, b_off=2)
        got = bf16_to_f64(dC.cpu().numpy().view(np.uint16))
        want = of.gelu_erf(ref) if epi == dlo.EPI_BIAS_GELU else ref
        nbad, worst = _close_bf16(got, want)
        assert nbad == 0, (nbad, worst)


def test_gemm_int8_full_size_sampled():
    """FFN-up product of the Super workload in INT8 (M=28800, N=20480, K=5120), codes
    uniform over [-127, 127] (sums up to K 127^2 = 8.3e7, exact in int32), sampled rows
    and columns."""
    torch = require_gpu()
    M, N, K = 28800, 20480, 5120
    say("gemm int8 full size", M, N, K)
    A = ((synth.normal_bf16(31, 13, 0, 0, (M, K), 0.0, 1.0) & 0xFF).astype(np.int64) % 255 - 127).astype(np.int8)
    B = ((synth.normal_bf16(32, 13, 0, 0, (N, K), 0.0, 1.0) & 0xFF).astype(np.int64) % 255 - 127).astype(np.int8)
    a_scale = np.exp2(synth.normal_f32(33, 13, 1, 0, (M,), -8.0, 2.0)).astype(np.float32)
    b_scale = np.exp2(synth.normal_f32(34, 13, 1, 0, (N,), -12.0, 1.0)).astype(np.float32)
    bias = synth.normal_f32(35, 13, 1, 0, (N,), 0.0, 0.02)
    dC = torch.empty((M, N), dtype=torch.int16, device="cuda")
    _run(torch, A, a_scale, B, b_scale, bias, None, dC, N, dlo.EPI_BIAS, M, N, K)
    rng = np.random.default_rng(1)
    rows = np.concatenate([rng.integers(0, M, 48), [0, M - 1, 28671, 28672]])
    cols = np.concatenate([rng.integers(0, N, 48), [0, N - 1, 255, 256]])
    C = dC[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16)[:, cols]
    ref = _ref(A[rows], a_scale[rows], B[cols], b_scale[cols], bias[cols])
    nbad, worst = _close_bf16(bf16_to_f64(C), ref)
    assert nbad == 0, (nbad, worst)


def test_int8_ops_reject_unsupported_shapes():
    torch = require_gpu()
    x = torch.zeros((4, 64), dtype=torch.int16, device="cuda")
    q = torch.zeros((4, 64), dtype=torch.int8, device="cuda")
    s = torch.zeros(4, dtype=torch.float32, device="cuda")
    for M, K, ldx, ldq in [(4, 60, 64, 64), (4, 64, 60, 64), (4, 64, 64, 56), (0, 64, 64, 64)]:
        with pytest.raises(dlo.DLOError):
            dlo.op_quantize_rows_int8(x.data_ptr(), ldx, M, K, q.data_ptr(), ldq, s.data_ptr(), 0)
    A = torch.zeros((256, 128), dtype=torch.int8, device="cuda")
    sc = torch.ones(256, dtype=torch.float32, device="cuda")
    C = torch.zeros((256, 256), dtype=torch.float32, device="cuda")
    for N, K, epi in [(200, 128, 0), (256, 96, 0), (256, 128, 7)]:
        with pytest.raises(dlo.DLOError):
            dlo.op_gemm_int8(A.data_ptr(), 128, sc.data_ptr(), A.data_ptr(), 128, sc.data_ptr(), 64, N, K,
                             sc.data_ptr(), 0, C.data_ptr(), 256, epi, 0)
