"""Pins for oracle.forward: brute force, special cases and hand-worked blocks.

Every expected number here is either brute force (explicit loops), a closed
form worked by hand for a constructed input, a standard-normal / logistic table
value, or an invariant (permutation equivariance, chaining, untouched columns).
"""
import math

import numpy as np
import pytest

import synth
from oracle import forward as of

# standard normal CDF and logistic values from tables
PHI_1 = 0.8413447460685429      # Phi(1)
PHI_2 = 0.9772498680518208      # Phi(2)
SIGMOID_1 = 0.7310585786300049  # 1 / (1 + e^-1)
SIGMOID_2 = 0.8807970779778823  # 1 / (1 + e^-2)
TANH_2 = 0.9640275800758169


def _bf16_bits(values):
    return synth.f32_to_bf16(np.asarray(values, dtype=np.float32))


def _block(d, *, W_ada=None, b_ada=None, Wqkv=None, bqkv=None, Wout=None, bout=None,
           W1=None, b1=None, W2=None, b2=None, g1=None, be1=None, eps1=0.0, g2=None, be2=None,
           eps2=0.0):
    z = lambda *s: np.zeros(s, dtype=np.float32)
    o = lambda *s: np.ones(s, dtype=np.float32)
    return [
        ("adaln.weight", "bf16", _bf16_bits(z(6 * d, d) if W_ada is None else W_ada)),
        ("adaln.bias", "f32", z(6 * d) if b_ada is None else np.asarray(b_ada, np.float32)),
        ("norm1.weight", "f32", o(d) if g1 is None else np.asarray(g1, np.float32)),
        ("norm1.bias", "f32", z(d) if be1 is None else np.asarray(be1, np.float32)),
        ("norm1.eps", "f32", np.array([eps1], np.float32)),
        ("attn.qkv.weight", "bf16", _bf16_bits(z(3 * d, d) if Wqkv is None else Wqkv)),
        ("attn.qkv.bias", "f32", z(3 * d) if bqkv is None else np.asarray(bqkv, np.float32)),
        ("attn.out.weight", "bf16", _bf16_bits(z(d, d) if Wout is None else Wout)),
        ("attn.out.bias", "f32", z(d) if bout is None else np.asarray(bout, np.float32)),
        ("norm2.weight", "f32", o(d) if g2 is None else np.asarray(g2, np.float32)),
        ("norm2.bias", "f32", z(d) if be2 is None else np.asarray(be2, np.float32)),
        ("norm2.eps", "f32", np.array([eps2], np.float32)),
        ("mlp.fc1.weight", "bf16", _bf16_bits(z(4 * d, d) if W1 is None else W1)),
        ("mlp.fc1.bias", "f32", z(4 * d) if b1 is None else np.asarray(b1, np.float32)),
        ("mlp.fc2.weight", "bf16", _bf16_bits(z(d, 4 * d) if W2 is None else W2)),
        ("mlp.fc2.bias", "f32", z(d) if b2 is None else np.asarray(b2, np.float32)),
    ]


def _chunks(d, **vals):
    """adaLN bias with the named chunks set (order shift1, scale1, gate1, shift2, scale2, gate2)."""
    order = ["shift1", "scale1", "gate1", "shift2", "scale2", "gate2"]
    b = np.zeros(6 * d, dtype=np.float32)
    for k, v in vals.items():
        i = order.index(k)
        b[i * d:(i + 1) * d] = v
    return b


def _run(block, x, c, heads=1):
    return of.dit_block(np.asarray(x, np.float64), np.asarray(c, np.float64),
                        of.param_dict(block), heads)


# --- P1: brute-force attention -------------------------------------------------------------

def _attention_loops(q, k, v, H):
    T, d = q.shape
    dh = d // H
    out = np.zeros((T, d))
    for h in range(H):
        for i in range(T):
            scores = []
            for j in range(k.shape[0]):
                s = 0.0
                for e in range(dh):
                    s += q[i, h * dh + e] * k[j, h * dh + e]
                scores.append(s / math.sqrt(dh))
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            tot = sum(w)
            for e in range(dh):
                out[i, h * dh + e] = sum(w[j] * v[j, h * dh + e] for j in range(len(w))) / tot
    return out


@pytest.mark.parametrize("T,Tk,H,dh", [(1, 1, 1, 4), (5, 7, 2, 4), (16, 16, 2, 8), (3, 16, 1, 8)])
def test_attention_brute_force(T, Tk, H, dh):
    rng = np.random.default_rng(T * 100 + Tk)
    q = rng.normal(size=(T, H * dh)) * 2
    k = rng.normal(size=(Tk, H * dh)) * 2
    v = rng.normal(size=(Tk, H * dh))
    got = of.attention(q, k, v, H, chunk=2)
    want = _attention_loops(q, k, v, H)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_attention_single_key_returns_value():
    rng = np.random.default_rng(3)
    q, k, v = rng.normal(size=(4, 8)), rng.normal(size=(1, 8)), rng.normal(size=(1, 8))
    assert np.array_equal(of.attention(q, k, v, 2), np.repeat(v, 4, axis=0))


# --- P8: linear against an explicit sum ----------------------------------------------------

def test_linear_brute_force():
    rng = np.random.default_rng(5)
    a, w, b = rng.normal(size=(3, 5)), rng.normal(size=(4, 5)), rng.normal(size=4)
    got = of.linear(a, w, b)
    for i in range(3):
        for j in range(4):
            assert abs(got[i, j] - (sum(a[i, e] * w[j, e] for e in range(5)) + b[j])) < 1e-12


# --- P7 / P9: LayerNorm statistics, GELU and SiLU table values -------------------------------

def test_layer_norm_statistics_and_eps():
    rng = np.random.default_rng(9)
    v = rng.normal(size=(6, 64)) * 3 + 1
    y = of.layer_norm(v, np.ones(64), np.zeros(64), 1e-6)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose(y.var(axis=1), 1, atol=1e-5)
    # eps enters under the square root: row [0, 0, 0, 2e-3] has mean 5e-4 and
    # biased variance 7.5e-7, so the first output is -5e-4 / sqrt(7.5e-7 + 1e-6)
    y = of.layer_norm(np.array([[0.0, 0.0, 0.0, 2e-3]]), np.ones(4), np.zeros(4), 1e-6)
    assert abs(y[0, 0] - (-5e-4 / math.sqrt(1.75e-6))) < 1e-15
    # a constant row maps to the shift
    y = of.layer_norm(np.full((1, 4), 5.0), np.full(4, 2.0), np.arange(4.0), 1e-6)
    assert np.array_equal(y[0], np.arange(4.0))


def test_gelu_and_silu_table_values():
    z = np.array([0.0, 1.0, -1.0, 2.0, -2.0, 8.0, -8.0])
    g = of.gelu_erf(z)
    assert g[0] == 0.0
    assert abs(g[1] - PHI_1) < 1e-15 and abs(g[2] + (1 - PHI_1)) < 1e-15
    assert abs(g[3] - 2 * PHI_2) < 1e-15 and abs(g[4] + 2 * (1 - PHI_2)) < 1e-15
    assert abs(g[5] - 8.0) < 1e-13 and abs(g[6]) < 1e-13
    s = of.silu(np.array([1.0, -1.0, 2.0, 0.0]))
    assert abs(s[0] - SIGMOID_1) < 1e-15 and abs(s[1] + (1 - SIGMOID_1)) < 1e-15
    assert abs(s[2] - 2 * SIGMOID_2) < 1e-15 and s[3] == 0.0


# --- hand-worked blocks (d = 4, one head) ---------------------------------------------------

I4 = np.eye(4, dtype=np.float32)
Z4 = np.zeros((4, 4), dtype=np.float32)
V_ONLY = np.vstack([Z4, Z4, I4])          # qkv weight with k = q = 0, v = h
X_LN11 = [1.0, 1.0, 3.0, 3.0]             # LN -> [-1, -1, 1, 1] (eps = 0)


def test_block_attention_branch_single_token():
    # gate1 = 1, every other chunk 0; T = 1 so attention returns v = h = LN(x); out = I
    blk = _block(4, b_ada=_chunks(4, gate1=1.0), Wqkv=V_ONLY, Wout=I4)
    y = _run(blk, [[1.0, 2.0, 3.0, 4.0]], np.zeros(4))
    r5 = math.sqrt(5.0)   # LN([1,2,3,4]) = [-3, -1, 1, 3] / sqrt(5)
    assert np.allclose(y[0], [1 - 3 / r5, 2 - 1 / r5, 3 + 1 / r5, 4 + 3 / r5], rtol=0, atol=1e-14)


def test_block_modulation_scale_and_shift():
    # scale1 = 1 doubles the normalised row, shift1 = 0.5 adds one half
    blk = _block(4, b_ada=_chunks(4, gate1=1.0, scale1=1.0, shift1=0.5), Wqkv=V_ONLY, Wout=I4)
    y = _run(blk, [[1.0, 2.0, 3.0, 4.0]], np.zeros(4))
    r5 = math.sqrt(5.0)
    want = [1.5 - 6 / r5, 2.5 - 2 / r5, 3.5 + 2 / r5, 4.5 + 6 / r5]
    assert np.allclose(y[0], want, rtol=0, atol=1e-14)


def test_block_silu_of_conditioning_feeds_shift():
    # the first d rows of W_ada (the shift1 chunk) are the identity: shift1 = silu(c)
    W_ada = np.zeros((24, 4), dtype=np.float32)
    W_ada[:4] = I4
    blk = _block(4, W_ada=W_ada, b_ada=_chunks(4, gate1=1.0), Wqkv=V_ONLY, Wout=I4)
    y = _run(blk, [X_LN11], [1.0, -1.0, 0.0, 2.0])
    want = [1 - 1 + SIGMOID_1, 1 - 1 - (1 - SIGMOID_1), 3 + 1 + 0.0, 3 + 1 + 2 * SIGMOID_2]
    assert np.allclose(y[0], want, rtol=0, atol=1e-7)  # W_ada = 1 is exact in bf16; c is float64


def test_block_mlp_branch_gate2_and_scale2():
    # gate2 = 1 only: x + GELU(LN2(x) * (1 + scale2)); fc1 = [I;0;0;0], fc2 = [I 0 0 0]
    W1 = np.vstack([I4, Z4, Z4, Z4])
    W2 = np.hstack([I4, Z4, Z4, Z4])
    blk = _block(4, b_ada=_chunks(4, gate2=1.0), W1=W1, W2=W2)
    y = _run(blk, [X_LN11], np.zeros(4))
    assert np.allclose(y[0], [1 - (1 - PHI_1), 1 - (1 - PHI_1), 3 + PHI_1, 3 + PHI_1], atol=1e-14)
    blk = _block(4, b_ada=_chunks(4, gate2=1.0, scale2=1.0), W1=W1, W2=W2)
    y = _run(blk, [X_LN11], np.zeros(4))
    g2, gm2 = 2 * PHI_2, -2 * (1 - PHI_2)
    assert np.allclose(y[0], [1 + gm2, 1 + gm2, 3 + g2, 3 + g2], atol=1e-14)


def test_block_two_token_softmax_scale():
    # q = k = v = h; rows h1 = [-1,-1,1,1], h2 = -h1; dh = 4 so scores are +-4/2 = +-2 and
    # each output row is (sigma(4) - sigma(-4)) h_i = tanh(2) h_i
    blk = _block(4, b_ada=_chunks(4, gate1=1.0), Wqkv=np.vstack([I4, I4, I4]), Wout=I4)
    y = _run(blk, [X_LN11, [3.0, 3.0, 1.0, 1.0]], np.zeros(4))
    h1 = np.array([-1.0, -1.0, 1.0, 1.0])
    assert np.allclose(y[0], np.array(X_LN11) + TANH_2 * h1, atol=1e-14)
    assert np.allclose(y[1], np.array([3.0, 3.0, 1.0, 1.0]) - TANH_2 * h1, atol=1e-14)


def test_block_biases_reach_output():
    # out bias passes through gate1; fc2 bias passes through gate2
    blk = _block(4, b_ada=_chunks(4, gate1=0.5, gate2=0.25), bout=[1, 2, 3, 4], b2=[4, 0, 0, 8])
    y = _run(blk, [X_LN11], np.zeros(4))
    assert np.allclose(y[0], np.array(X_LN11) + 0.5 * np.array([1, 2, 3, 4]) + 0.25 * np.array([4, 0, 0, 8]),
                       atol=1e-14)


# --- P5 / P10 / stack invariants on random blocks ----------------------------------------------

def _random_block(seed, d):
    return synth.block_params(seed, 0, d)


def test_adaln_zero_is_identity():
    blk = _random_block(11, 32)
    blk[0] = ("adaln.weight", "bf16", np.zeros((6 * 32, 32), np.uint16))
    blk[1] = ("adaln.bias", "f32", np.zeros(6 * 32, np.float32))
    rng = np.random.default_rng(0)
    x = rng.normal(size=(8, 32))
    assert np.array_equal(of.dit_block(x, rng.normal(size=32), of.param_dict(blk), 2), x)


def test_token_permutation_equivariance():
    blk = of.param_dict(_random_block(12, 32))
    rng = np.random.default_rng(1)
    x, c = rng.normal(size=(9, 32)), rng.normal(size=32)
    perm = rng.permutation(9)
    y = of.dit_block(x, c, blk, 4)
    yp = of.dit_block(x[perm], c, blk, 4)
    assert np.allclose(yp, y[perm], atol=1e-12)


def test_narrow_block_leaves_wide_residual_columns():
    blk = of.param_dict(_random_block(13, 16))
    rng = np.random.default_rng(2)
    x, c = rng.normal(size=(5, 24)), rng.normal(size=24)
    y = of.dit_block(x, c, blk, 2)
    assert np.array_equal(y[:, 16:], x[:, 16:])
    assert not np.allclose(y[:, :16], x[:, :16])
    c2 = c.copy(); c2[16:] = 99.0   # only c[:d] is read
    assert np.array_equal(of.dit_block(x, c2, blk, 2), y)


def test_passes_chain():
    blocks = [_random_block(20 + b, 16) for b in range(3)]
    rng = np.random.default_rng(4)
    x, c = rng.normal(size=(6, 16)), rng.normal(size=16)
    once = of.forward_stack(x, c, blocks, [2, 2, 2], 1)
    twice = of.forward_stack(x, c, blocks, [2, 2, 2], 2)
    assert np.allclose(of.forward_stack(once, c, blocks, [2, 2, 2], 1), twice, atol=1e-12)


def test_rows_variant_matches_full_block():
    blk = of.param_dict(_random_block(30, 32))
    rng = np.random.default_rng(6)
    x, c = rng.normal(size=(20, 40)), rng.normal(size=40)
    full = of.dit_block(x, c, blk, 4)
    rows = [0, 7, 19, 3]
    assert np.allclose(of.dit_block_rows(x, c, blk, 4, rows), full[rows], atol=1e-12)


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xC020, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    w = of.widen_bf16(bits)
    assert w[0] == 1.0 and w[1] == -2.5 and w[2] == 2.0 ** -133 and w[4] == 0.0
    assert w[3] == (2 - 2 ** -7) * 2.0 ** 127
