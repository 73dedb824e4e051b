"""GPU parity of the INT8 and MXFP8 weight forms: the dequantisation kernels bit for
bit, and INT8 / MXFP8 stacks streamed through the two slots against the oracle."""
import numpy as np
import pytest

import synth
import layerwise_weight_streaming_amd as dlo
from oracle import forward as of
from oracle import fp8
from oracle import plan as op
from oracle import quant
from oracle import schedule as sc
from tests.gpu_util import TOL, make_runner_params, rel_err, require_gpu, say

pytestmark = pytest.mark.gpu


def _bf16_rne(x32):
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_dequant_int8_every_code():
    """Every int8 code against per-row scales over twelve binades: the kernel's
    bf16(code * scale) equals the float32 product rounded to nearest even."""
    torch = require_gpu()
    rows, cols = 96, 512
    rng = np.random.default_rng(7)
    codes = np.tile(np.arange(-128, 128, dtype=np.int8), rows * cols // 256).reshape(rows, cols)
    rng.shuffle(codes, axis=1)
    scales = (np.exp2(rng.uniform(-20, 10, rows)) * rng.uniform(1, 2, rows)).astype(np.float32)
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    out = torch.empty((rows, cols), dtype=torch.int16, device="cuda")
    dlo.op_dequant_int8(dc.data_ptr(), rows, cols, ds.data_ptr(), out.data_ptr(), 0)
    torch.cuda.synchronize()
    want = _bf16_rne(codes.astype(np.float32) * scales[:, None])
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)


def test_dequant_mxfp8_every_code():
    """Every E4M3 code against E8M0 scales from 2^-107 to 2^103 (block-major
    [cols / 32, rows]): the product is exact in bf16 (the code's 4 significant bits
    fit), NaN codes and the NaN scale give NaN."""
    torch = require_gpu()
    rows, cols = 64, 256
    n = rows * cols
    rng = np.random.default_rng(8)
    codes = np.tile(np.arange(256, dtype=np.uint8), n // 256)
    rng.shuffle(codes)
    scales = rng.integers(20, 231, (cols // 32, rows)).astype(np.uint8)
    scales[1, 5] = 255
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    dlo.op_dequant_mxfp8(dc.data_ptr(), rows, cols, ds.data_ptr(), out.data_ptr(), 0)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    vals = (fp8.DECODE[codes].reshape(rows, cols) *
            np.repeat(quant.e8m0_value(scales).T, 32, axis=1)).reshape(-1)
    nan = np.isnan(vals)
    assert np.array_equal(got[~nan], _bf16_rne(vals[~nan].astype(np.float32)))
    assert np.array_equal(vals[~nan], ((got[~nan].astype(np.uint32) << 16).view(np.float32)).astype(np.float64))
    assert np.all(np.isnan((got[nan].astype(np.uint32) << 16).view(np.float32)))


def test_dequant_rejects_unsupported_shapes():
    torch = require_gpu()
    c = torch.zeros(64, dtype=torch.uint8, device="cuda")
    s_ = torch.ones(4, device="cuda")
    o = torch.empty(64, dtype=torch.int16, device="cuda")
    with pytest.raises(dlo.DLOError):
        dlo.op_dequant_int8(c.data_ptr(), 2, 24, s_.data_ptr(), o.data_ptr(), 0)
    with pytest.raises(dlo.DLOError):
        dlo.op_dequant_mxfp8(c.data_ptr(), 1, 48, s_.data_ptr(), o.data_ptr(), 0)


def _check_trace(tr, n, passes, regs):
    ref = sc.simulate_hooks(n, passes)
    assert len(tr) == len(ref)
    for got, e in zip(tr, ref):
        assert (got["step"], got["block"], got["read_slot"], got["prefetch_block"]) == \
            (e.step, e.block, e.read_slot, e.prefetch_block)
        want = op.digest_regions(regs[e.block])
        assert got["digest_pre"] == want and got["digest_post"] == want, e.step


@pytest.mark.parametrize("form", ["int8", "mxfp8"])
@pytest.mark.parametrize("name,n_blocks,tokens,which", [
    ("tiny", None, None, None),                 # every block quantised, 2 passes, odd count
    ("8blk", None, None, {0, 2, 3, 5}),         # quantised and bf16 blocks mixed
    ("irregular", 3, 256, None),                # widths 2048/3072/4096, k = 4 (three groups for MXFP8)
])
def test_quantised_weight_groups_streamed(form, name, n_blocks, tokens, which):
    """INT8 (int8 + fp32 row scales) and MXFP8 (E4M3 + E8M0 block scales) blocks: their
    1-byte groups sharded, streamed and placed at the all-gather offsets (slot digests =
    oracle), the forward within tolerance of the oracle on the dequantised weights, and
    streamed == resident bit for bit."""
    require_gpu()
    w = synth.WORKLOADS[name]
    if tokens is not None:
        w = w.with_(tokens=tokens)
    n = w.n_blocks if n_blocks is None else n_blocks
    say(f"{form} stack {name} n={n} T={w.tokens} which={which}")
    stack = synth.make_stack(w, 31, n)
    blocks = [quant.quantize_block(ps, form) if which is None or b in which else ps
              for b, ps in enumerate(stack.blocks)]
    r = make_runner_params(w, blocks)
    for b in range(n):
        assert r.plan.block_info(b)["form"] == (form if which is None or b in which else "bf16")
    r.set_inputs(stack.x, stack.c)
    run = r.forward(w.passes, flags=dlo.TRACE_DIGEST)
    tr = run.trace()
    regs = []
    for ps in blocks:
        bp = op.plan_block(op.specs_of(ps), w.k)
        regs.append(op.slot_regions(bp, op.pack_block(ps, bp)))
    _check_trace(tr, n, w.passes, regs)
    x_gpu = r.x_host()
    r.set_inputs(stack.x, stack.c)
    r.forward(w.passes, resident=True, want_run=False)
    assert np.array_equal(r.x_host().view(np.uint32), x_gpu.view(np.uint32))
    r.close()
    say("oracle forward (dequantised weights)")
    x_ref = of.forward_stack(stack.x, stack.c, blocks, [w.heads(b) for b in range(n)], w.passes)
    e_abs, e_upd = rel_err(x_gpu, x_ref), rel_err(x_gpu - stack.x, x_ref - stack.x)
    say(f"rel err {e_abs:.3e}, update rel err {e_upd:.3e}")
    assert e_abs <= TOL and e_upd <= TOL


@pytest.mark.parametrize("form", ["int8", "mxfp8"])
def test_quantised_weights_ragged_tokens(form):
    """A token count off the 64-row grid (T = 77) with INT8 / MXFP8 weights: within the
    stack tolerance of the oracle on the dequantised weights, streamed == resident."""
    require_gpu()
    w = synth.WORKLOADS["tiny"].with_(tokens=77)
    stack = synth.make_stack(w, 35)
    blocks = [quant.quantize_block(ps, form) for ps in stack.blocks]
    r = make_runner_params(w, blocks)
    r.set_inputs(stack.x, stack.c)
    r.forward(w.passes, want_run=False)
    x_gpu = r.x_host()
    r.set_inputs(stack.x, stack.c)
    r.forward(w.passes, resident=True, want_run=False)
    assert np.array_equal(r.x_host().view(np.uint32), x_gpu.view(np.uint32))
    r.close()
    x_ref = of.forward_stack(stack.x, stack.c, blocks, [w.heads(b) for b in range(w.n_blocks)], w.passes)
    assert rel_err(x_gpu - stack.x, x_ref - stack.x) <= TOL and rel_err(x_gpu, x_ref) <= TOL
