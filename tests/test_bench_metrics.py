"""Host-side measurement logic of bench.py (no GPU): interval algebra, the
overlap / link / MFMA figures of a trace, algorithmic work, counted traffic."""
import numpy as np
import pytest

import bench


def _measure(iv, grid):
    """Length of a union of intervals by brute force on a fine grid."""
    inside = np.zeros(grid.size - 1, dtype=bool)
    mid = 0.5 * (grid[1:] + grid[:-1])
    for a, b in iv:
        inside |= (mid >= a) & (mid < b)
    return inside.sum() * (grid[1] - grid[0]), inside


def test_union_and_intersection_match_brute_force():
    rng = np.random.default_rng(3)
    grid = np.linspace(0.0, 100.0, 200001)
    for _ in range(20):
        a = [tuple(sorted(rng.uniform(0, 100, 2))) for _ in range(rng.integers(1, 12))]
        b = [tuple(sorted(rng.uniform(0, 100, 2))) for _ in range(rng.integers(1, 12))]
        ua, ub = bench.union(a), bench.union(b)
        la, ia = _measure(a, grid)
        lb, ib = _measure(b, grid)
        assert abs(bench.length(ua) - la) < 1e-2
        assert abs(bench.length(ub) - lb) < 1e-2
        both = (ia & ib).sum() * (grid[1] - grid[0])
        assert abs(bench.intersect(ua, ub) - both) < 2e-2
        # a union is sorted and disjoint
        assert all(x[1] < y[0] for x, y in zip(ua, ua[1:]))


def test_clip_and_empty_intervals():
    assert bench.union([(3, 3), (5, 4)]) == []
    assert bench.clip([[0, 10], [20, 30]], 5, 25) == [[5, 10], [20, 25]]
    assert bench.clip([[0, 1]], 2, 3) == []


def _trace(n, copy_ms, compute_ms, pipelined):
    """n streamed steps, one block each; copy t+1 right after copy t when pipelined,
    else after compute t."""
    tr, t_copy = [], 0.0
    t_comp_end = 0.0
    for t in range(n):
        cb = t_copy if pipelined else max(t_copy, t_comp_end)
        ce = cb + copy_ms
        sb = max(ce, t_comp_end)
        se = sb + compute_ms
        tr.append({"step": t, "block": t, "read_slot": t % 2, "t_copy_begin": cb, "t_copy_end": ce,
                   "t_compute_begin": sb, "t_compute_end": se})
        t_copy, t_comp_end = ce, se
    return tr


def test_overlap_of_a_perfect_pipeline_is_one():
    n = 12
    tr = _trace(n, copy_ms=10.0, compute_ms=4.0, pipelined=True)
    m = bench.overlap_metrics(tr, copy_bytes=[10 ** 9] * n, flops=[2.5e12] * n)
    assert m["overlap_eff"] == pytest.approx(1.0)
    assert m["bound"] == "h2d"
    # window: copy(1) start .. compute(n-2) end; copies back to back in between
    assert m["window_ms"] == pytest.approx(tr[n - 2]["t_compute_end"] - tr[1]["t_copy_begin"])
    # 1 GB per 10 ms of copying = 100 GB/s while busy
    assert m["h2d_busy_GBps"] == pytest.approx(100.0, rel=0.05)


def test_overlap_of_a_serial_schedule_is_zero():
    n = 10
    tr = _trace(n, copy_ms=6.0, compute_ms=9.0, pipelined=False)
    m = bench.overlap_metrics(tr, copy_bytes=[10 ** 9] * n, flops=[2.5e12] * n)
    assert m["overlap_eff"] == pytest.approx(0.0, abs=1e-9)
    assert m["bound"] == "compute"
    # compute busy 9 of every 15 ms
    assert m["wall_eff"] == pytest.approx(9.0 / 15.0, rel=0.1)
    # 2.5 TFLOP per 9 ms busy = 277.8 TFLOP/s = 0.111 of 2.5 PFLOP/s
    assert m["mfma_util_busy"] == pytest.approx(2.5e12 / 9e-3 / 2.5e15, rel=1e-6)


def test_block_flops_and_kernel_work():
    # 24 T d^2 (linears) + 4 T^2 d (attention) + 12 d^2 (adaLN GEMV), Super shape
    assert bench.block_flops(5120, 28800) == pytest.approx(3.511e13, rel=1e-3)
    total = sum(bench.kernel_work(k, 5120, 28800)[0] for k in
                ("gemm_qk", "gemm_v_t", "attention", "gemm_out_residual", "gemm_fc1_gelu", "gemm_fc2_residual"))
    assert total * 1e12 == pytest.approx(24 * 28800 * 5120 ** 2 + 4 * 28800 ** 2 * 5120, rel=1e-12)
    assert bench.kernel_work("attention", 5120, 28800)[2] == "mfma"
    assert bench.kernel_work("ln1_modulate", 5120, 28800)[2] == "hbm"
    assert bench.kernel_work("dequant_weights", 5120, 28800, form="bf16")[0] == 0
    assert bench.kernel_work("dequant_weights", 5120, 28800, form="int8")[0] == pytest.approx((54 * 5120 ** 2 + 60 * 5120) / 1e9)


def test_counted_traffic_is_null_once_the_kernel_changed(monkeypatch):
    recorded = {}
    for ln in open(bench.TRAFFIC_FILE):
        t = ln.split()
        if len(t) == 4 and t[0] == "kernel_source":
            recorded[t[2]] = t[3]
    # the source hash the counters were taken on: the figure is reported
    monkeypatch.setattr(bench, "kernel_source_sha", lambda f: recorded[f])
    v = bench.counted_traffic("attention", "super")
    assert v is not None and v > 1e9
    # any other source: null
    monkeypatch.setattr(bench, "kernel_source_sha", lambda f: "0" * 64)
    assert bench.counted_traffic("attention", "super") is None
    # counted on the Super shape only
    monkeypatch.setattr(bench, "kernel_source_sha", lambda f: recorded[f])
    assert bench.counted_traffic("attention", "nano") is None


def test_kernel_work_of_the_quantised_forms():
    """Algorithmic bytes per slot for each weight form and compute mode (Super shape)."""
    d, T = 5120, 28800
    kw = lambda n, f, w8=False: bench.kernel_work(n, d, T, f, w8)[0] * 1e9
    # W8A16 dequantisation: FP8 the four linears (12 d^2 codes in, 24 d^2 bytes out),
    # INT8 / MXFP8 all five weights plus their scales
    assert kw("dequant_weights", "fp8") == 36 * d * d
    assert kw("dequant_weights", "int8") == 54 * d * d + 60 * d
    assert kw("dequant_weights", "mxfp8") == 54 * d * d + 18 * d * d // 32
    # W8A8: nothing dequantised for FP8, the adaLN weight for MXFP8
    assert kw("dequant_weights", "fp8", True) == 0
    assert kw("dequant_weights", "mxfp8", True) == 18 * d * d + 6 * d * d // 32
    # the adaLN GEMV reads E4M3 codes only for per-tensor FP8
    assert kw("adaln_gemv", "fp8") < kw("adaln_gemv", "mxfp8") == kw("adaln_gemv", "bf16")
    # W8A8: LayerNorm writes codes (+ scales), quant_h / quant_h2 do nothing
    assert kw("ln1_modulate", "fp8", True) == T * d * 5 + T * 4
    assert kw("ln2_modulate", "mxfp8", True) == T * d * 5 + T * d // 32
    for f in ("fp8", "mxfp8"):
        assert kw("quant_h", f, True) == kw("quant_h2", f, True) == 0
        assert kw("quant_attn", f, True) > 0
    # u: quantised by its own pass for FP8, by the fc1 epilogue for MXFP8
    assert kw("quant_u", "fp8", True) == T * 4 * d * 3 + T * 4
    assert kw("quant_u", "mxfp8", True) == 0
    # no quantisation without W8A8, nor for bf16 and INT8 blocks
    for f in ("bf16", "int8", "fp8", "mxfp8"):
        assert kw("quant_attn", f) == kw("quant_u", f) == 0
    # W8A8 INT8: the adaLN weight dequantised; h, h2, attn and u quantised in their own passes
    assert kw("dequant_weights", "int8", True) == 18 * d * d + 24 * d
    assert kw("ln1_modulate", "int8", True) == T * d * 6
    for n in ("quant_h", "quant_h2", "quant_attn"):
        assert kw(n, "int8", True) == T * d * 3 + T * 4
    assert kw("quant_u", "int8", True) == T * 4 * d * 3 + T * 4
