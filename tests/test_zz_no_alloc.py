"""The allocation-free adaLN entry point against the one with a workspace.

dlo_op_adaln_noalloc stages SiLU(c) in the library's static device array
instead of a caller workspace; it must give dlo_op_adaln's result bit for bit,
also on a second call in a row with a smaller input (the array keeps the first
call's contents, which the second call must not read), and match the oracle
within the adaLN test's bound.  Sizes beyond the array are rejected.
"""
import numpy as np
import pytest

import synth
import layerwise_weight_streaming_amd as dlo
from oracle import forward as of
from tests.gpu_util import bf16_to_f64, rel_err, require_gpu, say

pytestmark = pytest.mark.gpu


def _case(torch, d, rows, seed):
    W = synth.normal_bf16(seed, 9, 0, 0, (rows, d), 0.0, 0.02)
    b = synth.normal_f32(seed + 1, 9, 0, 0, (rows,), 0.0, 0.02)
    c = synth.normal_f32(seed + 2, 9, 0, 0, (d,))
    dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (W, b, c)]
    return W, b, c, dev


def test_adaln_noalloc_matches_workspace_entry_point():
    torch = require_gpu()
    s = torch.cuda.current_stream().cuda_stream
    # the largest width first, then a smaller one: the second call runs on an
    # array still holding the first call's values
    for d, rows, seed in [(dlo.NOALLOC_MAX_D, 6 * 1024, 70), (1024, 6 * 1024, 71), (256, 6 * 256, 72)]:
        say("adaln noalloc", d, rows)
        W, b, c, (dW, db, dc) = _case(torch, d, rows, seed)
        want = torch.zeros(rows, dtype=torch.float32, device="cuda")
        ws = torch.empty(4 * d, dtype=torch.uint8, device="cuda")
        dlo.op_adaln(dW.data_ptr(), db.data_ptr(), dc.data_ptr(), rows, d, want.data_ptr(), ws.data_ptr(),
                     ws.numel(), s)
        got = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        dlo.op_adaln_noalloc(dW.data_ptr(), db.data_ptr(), dc.data_ptr(), rows, d, got.data_ptr(), s)
        torch.cuda.synchronize()
        g, w = got.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(g.view(np.uint32), w.view(np.uint32))
        ref = of.linear(of.silu(c.astype(np.float64))[None, :], bf16_to_f64(W), b.astype(np.float64))[0]
        assert rel_err(g, ref) < 1e-5


def test_adaln_noalloc_rejects_widths_beyond_its_scratch():
    torch = require_gpu()
    d = dlo.NOALLOC_MAX_D + 8
    dW = torch.zeros((8, d), dtype=torch.int16, device="cuda")
    db = torch.zeros(8, dtype=torch.float32, device="cuda")
    dc = torch.zeros(d, dtype=torch.float32, device="cuda")
    out = torch.zeros(8, dtype=torch.float32, device="cuda")
    with pytest.raises(dlo.DLOError) as e:
        dlo.op_adaln_noalloc(dW.data_ptr(), db.data_ptr(), dc.data_ptr(), 8, d, out.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert e.value.status == "DLO_E_UNSUPPORTED"
