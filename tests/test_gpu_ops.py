"""Per-kernel parity on the GPU, through the C ABI, against the float64 oracle.

Small shapes that span several tiles plus a ragged tail are compared element by
element; the Super-shaped sizes are compared on sampled outputs that the oracle
computes one at a time.  Inputs are seeded (synth); expected values come from
oracle.forward only.
"""
import numpy as np
import pytest

import synth
import layerwise_weight_streaming_amd as dlo
from oracle import forward as of
from oracle import plan as op
from tests.gpu_util import bf16_to_f64, rel_err, require_gpu, say

pytestmark = pytest.mark.gpu

# bf16 outputs carry a relative rounding error of at most 2^-9; fp32 accumulation
# over K <= 20480 products of bf16 operands adds far less.  Element bound:
# |gpu - ref| <= 2^-8 |ref| + 2^-9 max|ref|.
def _close_bf16(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -9 * np.max(np.abs(ref))
    bad = np.abs(got - ref) > bound
    return int(bad.sum()), float(np.max(np.abs(got - ref) / np.maximum(bound, 1e-30)))


def _dev(torch, arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def _bf16_rand(seed, shape, std=1.0):
    return synth.normal_bf16(seed, 9, 0, 0, shape, 0.0, std)


@pytest.mark.parametrize("M,N,K", [(300, 512, 128), (64, 768, 256), (1000, 256, 320), (1, 256, 64)])
@pytest.mark.parametrize("epi", [dlo.EPI_BIAS, dlo.EPI_BIAS_GELU, dlo.EPI_GATED_RESIDUAL])
def test_gemm_small(M, N, K, epi):
    torch = require_gpu()
    say("gemm", M, N, K, "epi", epi)
    A = _bf16_rand(M * 7 + 1, (M, K))
    B = _bf16_rand(N * 5 + 2, (N, K), 0.05)
    bias = synth.normal_f32(3, 9, 1, 0, (N,), 0.0, 0.1)
    gate = synth.normal_f32(4, 9, 2, 0, (N,), 0.0, 1.0)
    X0 = synth.normal_f32(5, 9, 3, 0, (M, N))
    ref = of.linear(bf16_to_f64(A), bf16_to_f64(B), bias.astype(np.float64))
    dA, dB, db, dg = _dev(torch, A), _dev(torch, B), _dev(torch, bias), _dev(torch, gate)
    s = torch.cuda.current_stream().cuda_stream
    if epi == dlo.EPI_GATED_RESIDUAL:
        dX = _dev(torch, X0)
        dlo.op_gemm(dA.data_ptr(), K, dB.data_ptr(), K, M, N, K, db.data_ptr(), dg.data_ptr(),
                    dX.data_ptr(), N, epi, s)
        torch.cuda.synchronize()
        got = dX.cpu().numpy().astype(np.float64)
        want = X0.astype(np.float64) + gate.astype(np.float64) * ref
        assert rel_err(got - X0, want - X0) < 1e-5
    else:
        dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        dlo.op_gemm(dA.data_ptr(), K, dB.data_ptr(), K, M, N, K, db.data_ptr(), 0,
                    dC.data_ptr(), N, epi, s)
        torch.cuda.synchronize()
        got = bf16_to_f64(dC.cpu().numpy().view(np.uint16))
        want = of.gelu_erf(ref) if epi == dlo.EPI_BIAS_GELU else ref
        nbad, worst = _close_bf16(got, want)
        assert nbad == 0, (nbad, worst)


@pytest.mark.parametrize("offset_floats", [1, 2, 3])
@pytest.mark.parametrize("epi", [dlo.EPI_BIAS, dlo.EPI_BIAS_GELU, dlo.EPI_GATED_RESIDUAL, dlo.EPI_BIAS_T])
def test_gemm_bias_and_gate_at_slot_offsets(offset_floats, epi):
    """bias and gate 4-B aligned only (4, 8 and 12 bytes past a 16-B boundary), the
    way the fp32 parameters of a block sit back to back in a slot: the same result
    as with 16-B aligned copies of the same values, bit for bit, and the oracle's."""
    torch = require_gpu()
    M, N, K = 300, 512, 128
    say("gemm bias/gate offset", offset_floats, "epi", epi)
    A = _bf16_rand(41, (M, K))
    B = _bf16_rand(42, (N, K), 0.05)
    bias = synth.normal_f32(43, 9, 1, 0, (N,), 0.0, 0.1)
    gate = synth.normal_f32(44, 9, 2, 0, (N,), 0.0, 1.0)
    X0 = synth.normal_f32(45, 9, 3, 0, (M, N))
    # one fp32 buffer holding bias then gate, each starting offset_floats past 16 B
    packed = np.zeros(2 * N + 16, np.float32)
    packed[offset_floats:offset_floats + N] = bias
    packed[N + 4 + offset_floats:2 * N + 4 + offset_floats] = gate
    dP = _dev(torch, packed)
    p_bias = dP.data_ptr() + 4 * offset_floats
    p_gate = dP.data_ptr() + 4 * (N + 4 + offset_floats)
    assert p_bias % 16 != 0 and p_gate % 16 != 0
    da_bias, da_gate = _dev(torch, bias), _dev(torch, gate)
    dA, dB = _dev(torch, A), _dev(torch, B)
    s = torch.cuda.current_stream().cuda_stream
    ref = of.linear(bf16_to_f64(A), bf16_to_f64(B), bias.astype(np.float64))
    outs = []
    for pb, pg in ((p_bias, p_gate), (da_bias.data_ptr(), da_gate.data_ptr())):
        if epi == dlo.EPI_GATED_RESIDUAL:
            dX = _dev(torch, X0)
            dlo.op_gemm(dA.data_ptr(), K, dB.data_ptr(), K, M, N, K, pb, pg, dX.data_ptr(), N, epi, s)
            torch.cuda.synchronize()
            outs.append(dX.cpu().numpy())
        else:
            ldc = (M + 63) // 64 * 64 if epi == dlo.EPI_BIAS_T else N
            rows = N if epi == dlo.EPI_BIAS_T else M
            dC = torch.zeros((rows, ldc), dtype=torch.int16, device="cuda")
            dlo.op_gemm(dA.data_ptr(), K, dB.data_ptr(), K, M, N, K, pb, 0, dC.data_ptr(), ldc, epi, s)
            torch.cuda.synchronize()
            outs.append(dC.cpu().numpy().view(np.uint16))
    assert np.array_equal(outs[0].view(np.uint32 if outs[0].dtype == np.float32 else np.uint16),
                          outs[1].view(np.uint32 if outs[1].dtype == np.float32 else np.uint16))
    if epi == dlo.EPI_GATED_RESIDUAL:
        got = outs[0].astype(np.float64)
        assert rel_err(got - X0, gate.astype(np.float64) * ref) < 1e-5
    else:
        got = bf16_to_f64(outs[0][:, :M].T if epi == dlo.EPI_BIAS_T else outs[0])
        want = of.gelu_erf(ref) if epi == dlo.EPI_BIAS_GELU else ref
        nbad, worst = _close_bf16(got, want)
        assert nbad == 0, (nbad, worst)


def test_gemm_full_size_sampled():
    """QKV-shaped product of the Super workload (M=28800, N=15360, K=5120), sampled."""
    torch = require_gpu()
    M, N, K = 28800, 15360, 5120
    say("gemm full size", M, N, K)
    A = _bf16_rand(11, (M, K))
    B = _bf16_rand(12, (N, K), 0.02)
    bias = synth.normal_f32(13, 9, 1, 0, (N,), 0.0, 0.02)
    dA, dB, db = _dev(torch, A), _dev(torch, B), _dev(torch, bias)
    dC = torch.empty((M, N), dtype=torch.int16, device="cuda")
    dlo.op_gemm(dA.data_ptr(), K, dB.data_ptr(), K, M, N, K, db.data_ptr(), 0, dC.data_ptr(), N,
                dlo.EPI_BIAS, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.concatenate([rng.integers(0, M, 48), [0, M - 1, 28671, 28672]])
    cols = np.concatenate([rng.integers(0, N, 48), [0, N - 1, 255, 256]])
    C = dC[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16)[:, cols]
    ref = of.linear(bf16_to_f64(A[rows]), bf16_to_f64(B[cols]), bias[cols].astype(np.float64))
    nbad, worst = _close_bf16(bf16_to_f64(C), ref)
    assert nbad == 0, (nbad, worst)


@pytest.mark.parametrize("M,N,K,extra", [(300, 512, 128, 0), (64, 768, 256, 8), (1000, 256, 320, 64),
                                         (1, 256, 64, 0), (513, 256, 64, 0)])
def test_gemm_transposed_store(M, N, K, extra):
    """Epilogue 3: C[n, m] = (A B^T + bias)[m, n]; zeros for M <= m < M64, nothing written beyond."""
    torch = require_gpu()
    say("gemm transposed", M, N, K, extra)
    A = _bf16_rand(M * 3 + 7, (M, K))
    B = _bf16_rand(N * 11 + 5, (N, K), 0.05)
    bias = synth.normal_f32(6, 9, 1, 0, (N,), 0.0, 0.1)
    ref = of.linear(bf16_to_f64(A), bf16_to_f64(B), bias.astype(np.float64))
    M64 = (M + 63) // 64 * 64
    ldc = M64 + extra
    dA, dB, db = _dev(torch, A), _dev(torch, B), _dev(torch, bias)
    s = torch.cuda.current_stream().cuda_stream
    dCt = torch.full((N, ldc), 0x7FC0, dtype=torch.int16, device="cuda")
    dlo.op_gemm(dA.data_ptr(), K, dB.data_ptr(), K, M, N, K, db.data_ptr(), 0, dCt.data_ptr(), ldc,
                dlo.EPI_BIAS_T, s)
    dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    dlo.op_gemm(dA.data_ptr(), K, dB.data_ptr(), K, M, N, K, db.data_ptr(), 0, dC.data_ptr(), N,
                dlo.EPI_BIAS, s)
    torch.cuda.synchronize()
    ct = dCt.cpu().numpy().view(np.uint16)
    nbad, worst = _close_bf16(bf16_to_f64(ct[:, :M].T), ref)
    assert nbad == 0, (nbad, worst)
    assert np.all(ct[:, M:M64] == 0)
    assert np.all(ct[:, M64:] == 0x7FC0)
    # the same products as the row-major store, element for element
    assert np.array_equal(ct[:, :M].T, dC.cpu().numpy().view(np.uint16))


def _attention_case(torch, T, H, dh, seed):
    d = H * dh
    qkv = _bf16_rand(seed, (T, 3 * d), 1.0)
    dq = _dev(torch, qkv)
    ldvt = dlo.v_t_stride(T)
    # V^T starts as NaN everywhere: the attention must only see what the transpose wrote
    dvt = torch.full((d, ldvt), 0x7FC0, dtype=torch.int16, device="cuda")
    dout = torch.zeros((T, d), dtype=torch.int16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    dlo.op_v_transpose(dq.data_ptr(), 3 * d, T, d, dvt.data_ptr(), ldvt, s)
    dlo.op_attention(dq.data_ptr(), 3 * d, dvt.data_ptr(), ldvt, T, H, dh, dout.data_ptr(), d, s)
    torch.cuda.synchronize()
    return qkv, bf16_to_f64(dout.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("T,d,extra", [(1, 64, 0), (64, 256, 8), (300, 1024, 64), (777, 192, 0)])
def test_v_transpose_bit_exact(T, d, extra):
    """V^T holds the v columns of qkv transposed, zeros up to T rounded to 64, nothing beyond."""
    torch = require_gpu()
    say("v_transpose", T, d, extra)
    qkv = _bf16_rand(T + d, (T, 3 * d), 1.0)
    ldvt = dlo.v_t_stride(T) + extra
    dvt = torch.full((d, ldvt), 0x7FC0, dtype=torch.int16, device="cuda")
    dlo.op_v_transpose(_dev(torch, qkv).data_ptr(), 3 * d, T, d, dvt.data_ptr(), ldvt,
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    vt = dvt.cpu().numpy().view(np.uint16)
    T64 = dlo.v_t_stride(T)
    assert np.array_equal(vt[:, :T], qkv[:, 2 * d:].T)
    assert np.all(vt[:, T:T64] == 0)
    assert np.all(vt[:, T64:] == 0x7FC0)


@pytest.mark.parametrize("T,H,dh", [(1, 1, 64), (64, 4, 64), (300, 2, 128), (1000, 3, 64), (777, 2, 128)])
def test_attention_small(T, H, dh):
    torch = require_gpu()
    say("attention", T, H, dh)
    qkv, got = _attention_case(torch, T, H, dh, T + H + dh)
    d = H * dh
    q = bf16_to_f64(qkv[:, :d])
    k = bf16_to_f64(qkv[:, d:2 * d])
    v = bf16_to_f64(qkv[:, 2 * d:])
    ref = of.attention(q, k, v, H)
    # P is rounded to bf16 before P V and the output to bf16: 2^-7 of max|ref| is generous
    assert rel_err(got, ref) < 2.0 ** -7, rel_err(got, ref)


# score offsets (log2 units) of successive 32-key halves: the running max must be
# raised in a first half, in a second half only, several times in a row, and in
# the partial last block; dips in between take the common path
_RAISE_OFFSETS = [0, 5, 70, 65, 140, 130, 120, 200, 150, 100, 210, 205, 90, 80, 280, 350,
                  100, 0, 10, 290, 300, 430]


@pytest.mark.parametrize("dh", [128, 64])
def test_attention_running_max_raises(dh):
    """Keys whose scores jump by more than 64 log2 units above every earlier block's
    (through one shared q/k coordinate per head), so the rescale-and-redo path runs."""
    torch = require_gpu()
    T, H = 64 * 11 - 20, 2
    d = H * dh
    say("attention raises", T, H, dh)
    c = np.log2(np.e) / np.sqrt(dh)
    q = bf16_to_f64(_bf16_rand(1, (T, d), 1.0))
    k = bf16_to_f64(_bf16_rand(2, (T, d), 1.0))
    v = bf16_to_f64(_bf16_rand(3, (T, d), 1.0))
    alpha = np.array([np.round(o / (8 * c)) for o in _RAISE_OFFSETS])   # rounded to bf16 below, for both sides
    for h in range(H):
        q[:, h * dh] = 8.0
        k[:, h * dh] = alpha[np.arange(T) // 32]
    qkv = synth.f32_to_bf16(np.concatenate([q, k, v], axis=1).astype(np.float32))
    dq = _dev(torch, qkv)
    ldvt = dlo.v_t_stride(T)
    dvt = torch.full((d, ldvt), 0x7FC0, dtype=torch.int16, device="cuda")
    dout = torch.zeros((T, d), dtype=torch.int16, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    dlo.op_v_transpose(dq.data_ptr(), 3 * d, T, d, dvt.data_ptr(), ldvt, st)
    dlo.op_attention(dq.data_ptr(), 3 * d, dvt.data_ptr(), ldvt, T, H, dh, dout.data_ptr(), d, st)
    torch.cuda.synchronize()
    got = bf16_to_f64(dout.cpu().numpy().view(np.uint16))
    ref = of.attention(bf16_to_f64(qkv[:, :d]), bf16_to_f64(qkv[:, d:2 * d]), bf16_to_f64(qkv[:, 2 * d:]), H)
    assert np.all(np.isfinite(got))
    assert rel_err(got, ref) < 2.0 ** -7, rel_err(got, ref)


def test_attention_full_size_sampled():
    """Super-shaped attention: T=28800, 40 heads of 128, sampled query rows and heads."""
    torch = require_gpu()
    T, H, dh = 28800, 40, 128
    say("attention full size", T, H, dh)
    qkv, got = _attention_case(torch, T, H, dh, 77)
    d = H * dh
    rng = np.random.default_rng(1)
    rows = np.concatenate([rng.integers(0, T, 12), [0, T - 1, 28672, 28671]])
    for h in (0, 17, 39):
        cols = slice(h * dh, (h + 1) * dh)
        q = bf16_to_f64(qkv[rows, h * dh:(h + 1) * dh])
        k = bf16_to_f64(qkv[:, d + h * dh:d + (h + 1) * dh])
        v = bf16_to_f64(qkv[:, 2 * d + h * dh:2 * d + (h + 1) * dh])
        ref = of.attention(q, k, v, 1)
        assert rel_err(got[rows][:, cols], ref) < 2.0 ** -7


# (T, d, ldx, goff): the 16-B path (d % 1024 == 0, ldx % 4 == 0) with gamma and beta
# at 4-B offsets as in a slot's fp32 region (goff = 1), the per-element path for
# other widths and for ldx % 4 != 0
@pytest.mark.parametrize("T,d,ldx,goff", [(1, 256, 256, 0), (33, 1024, 1024, 0), (17, 5120, 5120, 1),
                                          (9, 2048, 4096, 0), (5, 3072, 3076, 1), (7, 1024, 1032, 0),
                                          (3, 768, 768, 1),
                                          # more rows than workgroups: each takes several rows
                                          (2000, 3072, 3072, 0), (1537, 5120, 5124, 1), (1030, 8192, 8192, 0),
                                          (800, 2304, 2304, 1)])
def test_ln_modulate(T, d, ldx, goff):
    torch = require_gpu()
    say("ln_modulate", T, d, ldx, goff)
    x = synth.normal_f32(20, 9, 0, 0, (T, ldx), 0.5, 2.0)
    gamma = synth.normal_f32(21, 9, 0, 0, (d,), 1.0, 0.1)
    beta = synth.normal_f32(22, 9, 0, 0, (d,), 0.0, 0.1)
    shift = synth.normal_f32(23, 9, 0, 0, (d,), 0.0, 0.1)
    scale = synth.normal_f32(24, 9, 0, 0, (d,), 0.0, 0.1)
    eps = np.array([1e-6], np.float32)
    dx, de, dsh, dsc = (_dev(torch, a) for a in (x, eps, shift, scale))
    dgb = _dev(torch, np.concatenate([np.zeros(goff, np.float32), gamma, beta]))
    dout = torch.zeros((T, d), dtype=torch.int16, device="cuda")
    dlo.op_ln_modulate(dx.data_ptr(), ldx, T, d, dgb.data_ptr() + 4 * goff, dgb.data_ptr() + 4 * (goff + d),
                       de.data_ptr(), dsh.data_ptr(), dsc.data_ptr(), dout.data_ptr(),
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = bf16_to_f64(dout.cpu().numpy().view(np.uint16))
    ref = of.layer_norm(x[:, :d].astype(np.float64), gamma, beta, 1e-6) * (1 + scale.astype(np.float64)) + shift
    nbad, worst = _close_bf16(got, ref)
    assert nbad == 0, (nbad, worst)


@pytest.mark.parametrize("rows,d", [(6 * 256, 256), (6 * 1024, 1024), (6 * 2048, 2048), (6 * 5120, 5120),
                                    (6 * 8192, 8192),
                                    # the row-looping form (d % 512 == 0, d >= 2048): fewer rows than
                                    # waves, and several rows per wave
                                    (37, 4096), (13001, 2048)])
def test_adaln(rows, d):
    torch = require_gpu()
    say("adaln", rows, d)
    W = _bf16_rand(30 + d, (rows, d), 0.02)
    b = synth.normal_f32(31, 9, 0, 0, (rows,), 0.0, 0.02)
    c = synth.normal_f32(32, 9, 0, 0, (d,))
    dW, db, dc = _dev(torch, W), _dev(torch, b), _dev(torch, c)
    out = torch.zeros(rows, dtype=torch.float32, device="cuda")
    ws = torch.empty(4 * d, dtype=torch.uint8, device="cuda")
    dlo.op_adaln(dW.data_ptr(), db.data_ptr(), dc.data_ptr(), rows, d, out.data_ptr(),
                 ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = of.linear(of.silu(c.astype(np.float64))[None, :], bf16_to_f64(W), b.astype(np.float64))[0]
    assert rel_err(out.cpu().numpy(), ref) < 1e-5


def test_digest_matches_oracle_definition():
    torch = require_gpu()
    say("digest")
    rng = np.random.default_rng(5)
    buf = rng.integers(0, 256, size=1 << 20, dtype=np.uint8)
    dbuf = _dev(torch, buf)
    out = torch.zeros(1, dtype=torch.int64, device="cuda")
    for offs, lens in [([0], [1 << 20]), ([256, 4096], [1001, 5000]), ([0, 1 << 19], [7, 3])]:
        dlo.op_digest(dbuf.data_ptr(), offs, lens, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        got = int(out.cpu().numpy().view(np.uint64)[0])
        want = op.digest_regions([(o, buf[o:o + n]) for o, n in zip(offs, lens)])
        assert got == want


def _bf16_rne(x32):
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("scale", [1.0, 0.0371, 3.5e-5])
def test_dequant_fp8_every_code(scale):
    """All 256 E4M3 codes: the kernel's bf16(value * scale) equals the oracle's code
    value times the scale in float32, rounded to nearest even; NaN codes give NaN."""
    torch = require_gpu()
    from oracle import fp8
    codes = np.tile(np.arange(256, dtype=np.uint8), 24)              # 6144 codes
    dc = torch.from_numpy(codes).cuda()
    ds = torch.tensor([scale], dtype=torch.float32, device="cuda")
    out = torch.empty(codes.size, dtype=torch.int16, device="cuda")
    dlo.op_dequant_fp8(dc.data_ptr(), codes.size, ds.data_ptr(), out.data_ptr(), 0)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    vals = fp8.DECODE[codes]
    nan = np.isnan(vals)
    want = _bf16_rne(vals[~nan].astype(np.float32) * np.float32(scale))
    assert np.array_equal(got[~nan], want)
    gotf = (got[nan].astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(gotf))


def test_dequant_fp8_rejects_misaligned_sizes():
    torch = require_gpu()
    c = torch.zeros(64, dtype=torch.uint8, device="cuda")
    s_ = torch.ones(1, device="cuda")
    o = torch.empty(64, dtype=torch.int16, device="cuda")
    with pytest.raises(dlo.DLOError):
        dlo.op_dequant_fp8(c.data_ptr(), 63, s_.data_ptr(), o.data_ptr(), 0)
