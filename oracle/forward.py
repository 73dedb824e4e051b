"""Oracle: the DiT stack forward with every weight resident, in float64.

The weight-streaming method must reproduce exactly what a fully resident model
computes: the pages verify it by byte-identical outputs across execution
strategies ([Aug] "NVIDIA B300 GPU Results", correctness paragraph).  So the
oracle is the plain resident forward.  It reads the same bf16 weights, widened
exactly to float64, and computes every activation in float64 with no rounding
to bf16 anywhere -- except where an activation decides an integer: the W8A8
form of an FP8 block quantizes each linear's input to E4M3 codes, and takes
that decision on the input as the model stores it, bf16 (round_bf16).

The pages never spell out the block (the model code is used unchanged, [Jul]
"Module Architecture").  The block below is the plainest adaLN-Zero DiT block
that matches the stated workloads (adaLN 6-way modulation from a conditioning
vector, LayerNorm, fused QKV, attention, output projection, 4d GELU MLP,
residual).  Readings where the pages leave a step open:

* mod = SiLU(c[:d]) @ W_ada^T + b_ada, split into six d-wide chunks in the
  order shift1, scale1, gate1, shift2, scale2, gate2;
* modulation h = LN(x) * (1 + scale) + shift; LN uses the biased variance over
  the d features and the block's own eps buffer;
* fused QKV weight [3d, d] holds q, k, v row blocks; head j owns the
  contiguous columns [j*dh, (j+1)*dh) of each;
* attention is non-causal, unmasked, scaled by 1/sqrt(dh), softmax over all
  tokens (max-subtracted);
* GELU is the exact erf form;
* residual updates are gated: x += gate * branch;
* a block of width d reads and updates x[:, :d] (residual width D >= d) and
  uses c[:d];
* passes chain: x <- stack(x).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf


def round_bf16(x) -> np.ndarray:
    """float64 -> the nearest bfloat16 value (8 significant bits, ties to the even
    significand), as float64.  Exponents below bfloat16's smallest normal keep its
    subnormal spacing 2^-133; the values here never reach its overflow range."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = m 2^e with 1/2 <= |m| < 1
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def param_dict(params):
    """[(name, dtype, array)] -> {name: float64 array} (bf16 widened).

    A quantised block carries each linear as ``X.weight`` (codes) plus
    ``X.weight_scale``; ``X.weight`` is then the dequantised weight and the
    scale entry is dropped: E4M3 codes with one fp32 scale (per-tensor FP8,
    oracle.fp8), int8 codes with one fp32 scale per output row, or E4M3 codes
    with E8M0 scales per 32-element block (oracle.quant).
    """
    from . import fp8, quant

    out, codes = {}, {}
    raw = {name: (dt, arr) for name, dt, arr in params}
    for name, dt, arr in params:
        if name.endswith("_scale") and name[:-len("_scale")] in raw and \
                raw[name[:-len("_scale")]][0] in ("fp8", "i8"):
            continue
        if dt in ("fp8", "i8"):
            codes[name] = (dt, arr)
        elif dt == "bf16":
            out[name] = widen_bf16(arr)
        else:
            out[name] = np.asarray(arr, dtype=np.float64)
    for name, (dt, c) in codes.items():
        sdt, sc = raw[name + "_scale"]
        if dt == "fp8" and sdt == "f32":
            out[name] = fp8.dequantize(c, np.float32(np.asarray(sc).reshape(-1)[0]))
        elif dt == "i8" and sdt == "f32":
            scl = np.asarray(sc, np.float32).reshape(-1)
            out[name] = quant.dequantize_int8(np.asarray(c, np.int8).reshape(scl.size, -1), scl)
        elif dt == "fp8" and sdt == "e8m0":   # scales block-major [in / 32, out]
            c2 = np.asarray(c, np.uint8)
            out[name] = quant.dequantize_mxfp8(c2, np.asarray(sc, np.uint8).reshape(-1, c2.shape[0]).T)
        else:
            raise ValueError(f"{name}: no dequantisation for {dt} codes with {sdt} scales")
    return out


def silu(z):
    return z / (1.0 + np.exp(-z))


def layer_norm(v, gamma, beta, eps):
    mean = v.mean(axis=-1, keepdims=True)
    dev = v - mean
    var = (dev * dev).mean(axis=-1, keepdims=True)
    return dev / np.sqrt(var + eps) * gamma + beta


def gelu_erf(z):
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def linear(a, w, b):
    """a @ w^T + b with w stored [out, in]."""
    return a @ w.T + b


def attention(q, k, v, n_heads, chunk=1024, progress=None):
    """Per head: softmax(q_j k_j^T / sqrt(dh)) v_j over all keys; heads concatenated.

    q: [Tq, d], k and v: [Tk, d]; computed in query chunks of at most ``chunk``
    rows (a memory bound only: each query row is independent).  progress, if
    given, is called with a short message after each head (no effect on the
    result).
    """
    tq, d = q.shape
    dh = d // n_heads
    scale = 1.0 / math.sqrt(dh)
    out = np.empty((tq, d), dtype=np.float64)
    for j in range(n_heads):
        cols = slice(j * dh, (j + 1) * dh)
        kj, vj = k[:, cols], v[:, cols]
        for r0 in range(0, tq, chunk):
            s = (q[r0:r0 + chunk, cols] @ kj.T) * scale
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[r0:r0 + chunk, cols] = p @ vj
        if progress is not None:
            progress(f"attention head {j + 1}/{n_heads}")
    return out


def modulation(c, P, d):
    mod = linear(silu(np.asarray(c[:d], dtype=np.float64))[None, :], P["adaln.weight"],
                 P["adaln.bias"])[0]
    return [mod[i * d:(i + 1) * d] for i in range(6)]


def dit_block(x, c, P, n_heads, act_fp8=False, act_mx=False, act_int8=False, progress=None):
    """One block on residual x [T, D] (float64, updated copy returned).

    act_fp8: the four block linears take their input through per-token E4M3
    quantization (oracle.fp8.quantize_rows), the W8A8 form of an FP8 block's
    online FP8 linears; the adaLN linear keeps its float input.  The quantizer
    reads the input as the model stores it, rounded to bf16 (round_bf16): the
    pages fix no precision for this decision, so it is taken in the storage
    precision of the activations it quantizes.  act_mx: the same with MXFP8
    inputs (oracle.quant.fake_quant_mx_rows: per row, blocks of 32 along the
    input dimension), the W8A8 form of an MXFP8 block's linears.  act_int8:
    the same with per-row int8 inputs (oracle.quant.fake_quant_int8_rows), the
    W8A8 form of an INT8 block's linears.  progress, if given, is called with a
    short message after each stage (no effect on the result).
    """
    from . import fp8, quant

    if act_int8:
        lin_in = quant.fake_quant_int8_rows
    elif act_mx:
        lin_in = quant.fake_quant_mx_rows
    elif act_fp8:
        lin_in = lambda t: fp8.fake_quant_rows(round_bf16(t))
    else:
        lin_in = lambda t: t
    d = P["norm1.weight"].shape[0]
    x = np.array(x, dtype=np.float64, copy=True)
    shift1, scale1, gate1, shift2, scale2, gate2 = modulation(c, P, d)
    xb = x[:, :d]
    h = layer_norm(xb, P["norm1.weight"], P["norm1.bias"], P["norm1.eps"][0]) * (1.0 + scale1) + shift1
    say = progress if progress is not None else (lambda msg: None)
    qkv = linear(lin_in(h), P["attn.qkv.weight"], P["attn.qkv.bias"])
    say("qkv")
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    a = attention(q, k, v, n_heads, progress=progress)
    xb += gate1 * linear(lin_in(a), P["attn.out.weight"], P["attn.out.bias"])
    say("out")
    h2 = layer_norm(xb, P["norm2.weight"], P["norm2.bias"], P["norm2.eps"][0]) * (1.0 + scale2) + shift2
    u = gelu_erf(linear(lin_in(h2), P["mlp.fc1.weight"], P["mlp.fc1.bias"]))
    say("fc1")
    xb += gate2 * linear(lin_in(u), P["mlp.fc2.weight"], P["mlp.fc2.bias"])
    say("fc2")
    return x


def dit_block_rows(x, c, P, n_heads, rows):
    """Output rows ``rows`` of one block, computed one query row at a time.

    Keys and values need every token, so LN1 and the k/v projections run over
    all T rows; everything else runs only for the requested rows.  Used to
    check sampled outputs at sizes where the full block is too slow on a CPU.
    """
    d = P["norm1.weight"].shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    x = np.asarray(x, dtype=np.float64)
    shift1, scale1, gate1, shift2, scale2, gate2 = modulation(c, P, d)
    xb = x[:, :d]
    h = layer_norm(xb, P["norm1.weight"], P["norm1.bias"], P["norm1.eps"][0]) * (1.0 + scale1) + shift1
    W, bqkv = P["attn.qkv.weight"], P["attn.qkv.bias"]
    k = linear(h, W[d:2 * d], bqkv[d:2 * d])
    v = linear(h, W[2 * d:], bqkv[2 * d:])
    q = linear(h[rows], W[:d], bqkv[:d])
    a = attention(q, k, v, n_heads)
    y = np.array(x[rows], dtype=np.float64, copy=True)
    yb = y[:, :d]
    yb += gate1 * linear(a, P["attn.out.weight"], P["attn.out.bias"])
    h2 = layer_norm(yb, P["norm2.weight"], P["norm2.bias"], P["norm2.eps"][0]) * (1.0 + scale2) + shift2
    u = gelu_erf(linear(h2, P["mlp.fc1.weight"], P["mlp.fc1.bias"]))
    yb += gate2 * linear(u, P["mlp.fc2.weight"], P["mlp.fc2.bias"])
    return y


def forward_stack(x, c, blocks, heads, passes, act_fp8=False):
    """``passes`` chained passes over the blocks.

    blocks: list of [(name, dtype, array)] per block; heads: heads per block.
    act_fp8: blocks with per-tensor FP8, MXFP8 or INT8 weights run their
    linears in the W8A8 form (see dit_block: per-row E4M3, MXFP8 or int8
    inputs); bf16 blocks are unaffected.
    """
    Ps = [param_dict(b) for b in blocks]
    mx_block = [any(dt == "e8m0" for _, dt, _ in b) for b in blocks]
    i8_block = [any(dt == "i8" for _, dt, _ in b) for b in blocks]
    fp8_block = [any(dt == "fp8" for _, dt, _ in b) and not mx for b, mx in zip(blocks, mx_block)]
    y = np.asarray(x, dtype=np.float64)
    for _ in range(passes):
        for P, H, f8, mx, i8 in zip(Ps, heads, fp8_block, mx_block, i8_block):
            y = dit_block(y, c, P, H, act_fp8=act_fp8 and f8, act_mx=act_fp8 and mx, act_int8=act_fp8 and i8)
    return y
