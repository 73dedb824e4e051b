"""A CPU model of the GPU's W8A8 block forward (test infrastructure).

The oracle computes a W8A8 block in float64 from exactly widened weights; the
GPU computes it in fp32 arithmetic with bf16 storage between kernels, and every
E4M3 / int8 decision it takes is taken on those bf16 values.  This model takes
the oracle's steps, with the oracle's own primitives and quantizers
(oracle.forward, oracle.fp8, oracle.quant), at the GPU's storage and
arithmetic precisions:

* adaLN: fp32 GEMV of SiLU(c) (fp32) on W_ada as the GPU reads it (FP8 block:
  code value x scale; INT8 block: the bf16 dequantised copy; MXFP8: exact);
* LayerNorm + modulate in fp32, stored bf16 (h, h2);
* each linear's input quantised from its bf16 values, the product in fp32
  with the fp32 bias, q,k and v stored bf16;
* attention on bf16 q, k, v: q times log2(e) / sqrt(dh) rounded to bf16,
  fp32 scores, P = exp2(score - row max) rounded to bf16, row sums of that
  bf16 P in fp32, O = P V / sum in fp32, stored bf16;
* the out and fc2 products scaled by their gates and added to the fp32
  residual; GELU in fp32 on the fc1 product, stored bf16 (u).

With ``exact=True`` every rounding point is switched off and the arithmetic is
float64: the model must then be the oracle's W8A8 block (a test checks it), so
its composition is the oracle's.  Its distance to the oracle with the rounding
points on predicts the GPU's distance, on the CPU, before the GPU runs; with a
second fp32 summation order (``order=1``: every product's K dimension summed in
four chunks) its distance to itself estimates how far two correct fp32
implementations drift apart through the chaotic bf16 / E4M3 decisions, which
bounds the GPU's distance to the model.
"""
from __future__ import annotations

import numpy as np

from oracle import forward as of
from oracle import fp8, quant


class _Prec:
    def __init__(self, exact: bool, order: int, noise: float = 0.0, seed: int = 0):
        self.exact, self.order, self.noise = exact, order, noise
        self.F = np.float64 if exact else np.float32
        self.rng = np.random.default_rng(seed)

    def bf16(self, a):
        a = np.asarray(a, dtype=np.float64)
        return a if self.exact else of.round_bf16(a)

    def f(self, a):
        return np.asarray(a, dtype=self.F)

    def mm(self, a, b):
        """a @ b in the working precision; order 1 sums K in four chunks."""
        a, b = self.f(a), self.f(b)
        if self.order == 0 or a.shape[1] < 4:
            return a @ b
        ks = np.array_split(np.arange(a.shape[1]), 4)
        out = a[:, ks[0]] @ b[ks[0]]
        for k in ks[1:]:
            out = out + a[:, k] @ b[k]
        return out

    def mm8(self, a, b):
        """A W8A8 linear's product: mm, plus (noise > 0) an error of up to
        noise * sum_k |a_k b_k| per output, uniform in sign and size."""
        out = self.mm(a, b)
        if self.noise > 0:
            mag = np.abs(self.f(a)) @ np.abs(self.f(b))
            out = out + (self.noise * mag * self.rng.uniform(-1.0, 1.0, out.shape)).astype(self.F)
        return out


def _layer_norm(p: _Prec, v, gamma, beta, eps):
    v = p.f(v)
    mean = v.mean(axis=-1, keepdims=True, dtype=p.F)
    dev = v - mean
    var = (dev * dev).mean(axis=-1, keepdims=True, dtype=p.F)
    return dev * (p.F(1.0) / np.sqrt(var + p.F(eps))) * p.f(gamma) + p.f(beta)


def _attention(p: _Prec, q, k, v, n_heads):
    tq, d = q.shape
    dh = d // n_heads
    cst = p.F(np.log2(np.e) / np.sqrt(dh))
    out = np.empty((tq, d), dtype=p.F)
    for j in range(n_heads):
        cs = slice(j * dh, (j + 1) * dh)
        qs = p.bf16(p.f(q[:, cs]) * cst)
        s = p.mm(qs, p.f(k[:, cs]).T)
        pr = p.bf16(np.exp2(s - s.max(axis=1, keepdims=True)))
        l = p.f(pr).sum(axis=1, keepdims=True, dtype=p.F)
        out[:, cs] = p.mm(pr, v[:, cs]) / l
    return p.bf16(out)


def _gelu(p: _Prec, z):
    from scipy.special import erf
    z = p.f(z)
    return p.f(0.5 * z * (1.0 + erf(z / np.sqrt(2.0)).astype(p.F)))


def block(x, c, params, n_heads, form, exact=False, order=0, noise=0.0, seed=0):
    """One W8A8 block (form 'fp8', 'mxfp8' or 'int8') on residual x [T, D]."""
    p = _Prec(exact, order, noise, seed)
    P = of.param_dict(params)
    d = P["norm1.weight"].shape[0]
    if form == "fp8":   # the oracle's FP8 input rounding, on values the model may already hold in bf16
        lin_in = lambda t: fp8.fake_quant_rows(of.round_bf16(t))
    elif form == "mxfp8":
        lin_in = lambda t: quant.fake_quant_mx_rows(p.bf16(t))
    else:
        lin_in = lambda t: quant.fake_quant_int8_rows(p.bf16(t))

    def lin(a, name):
        return p.mm8(a, p.f(P[name + ".weight"]).T) + p.f(P[name + ".bias"])

    w_ada = P["adaln.weight"]
    if form == "int8" and not exact:   # the GPU multiplies the bf16 dequantised copy
        w_ada = p.bf16(w_ada)
    cc = p.f(np.asarray(c[:d], dtype=np.float64))
    s = cc / (p.F(1.0) + np.exp(-cc))
    mod = p.mm(s[None, :], p.f(w_ada).T)[0] + p.f(P["adaln.bias"])
    shift1, scale1, gate1, shift2, scale2, gate2 = (mod[i * d:(i + 1) * d] for i in range(6))

    y = p.f(np.array(x, dtype=np.float64, copy=True))
    yb = y[:, :d]
    h = p.bf16(_layer_norm(p, yb, P["norm1.weight"], P["norm1.bias"], P["norm1.eps"][0]) * (1 + scale1) + shift1)
    hq = lin_in(h)
    W, bq = P["attn.qkv.weight"], P["attn.qkv.bias"]
    qk = p.bf16(p.mm8(hq, p.f(W[:2 * d]).T) + p.f(bq[:2 * d]))
    v = p.bf16(p.mm8(hq, p.f(W[2 * d:]).T) + p.f(bq[2 * d:]))
    a = _attention(p, qk[:, :d], qk[:, d:], v, n_heads)
    yb += gate1 * lin(lin_in(a), "attn.out")
    h2 = p.bf16(_layer_norm(p, yb, P["norm2.weight"], P["norm2.bias"], P["norm2.eps"][0]) * (1 + scale2) + shift2)
    u = p.bf16(_gelu(p, lin(lin_in(h2), "mlp.fc1")))
    yb += gate2 * lin(lin_in(u), "mlp.fc2")
    return np.asarray(y, dtype=np.float64)


def stack(x, c, blocks, heads, passes, form, exact=False, order=0, noise=0.0, seed=0):
    """``passes`` chained passes of W8A8 blocks of one form."""
    y = np.asarray(x, dtype=np.float64)
    step = 0
    for _ in range(passes):
        for ps, H in zip(blocks, heads):
            y = block(y, c, ps, H, form, exact, order, noise, seed + step)
            step += 1
    return y
