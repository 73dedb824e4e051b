#!/usr/bin/env python3
"""Benchmark of the double-buffered, layerwise weight-streamed DiT stack on one MI355X.

One step = one call of dlo_forward_stack: every block of the stack, for the
workload's number of chained passes, with block N+1's shards streaming into the
free slot while block N computes.  Inputs are seeded synthetic data with the
workload's shapes; the host store is packed before timing; x, cond and the slots
live in HBM when the timed region starts.

Printed: one JSON line (blocks/s as ``value``) with tokens/s, host-to-device
GB/s against the PCIe 5.0 x16 link, bf16 MFMA utilisation against the dense
peak, copy/compute overlap efficiency (all from HIP events recorded by libdlo on
the streams the work runs on), the dominant kernel's roofline position, and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA (TOP/s), published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
LINK_PEAK_GBS = 32.0 * 16 * 128 / 130 / 8   # PCIe 5.0 x16, one direction: 63.0 GB/s


def kernel_work(name, d, T, form="bf16", w8a8=False):
    """Algorithmic work of one launch: (amount, unit, bound).  form: the block's
    weight form ("bf16", "fp8", "int8", "mxfp8"); w8a8: quantised blocks run W8A8
    (the linears' inputs quantised, only the adaLN weight dequantised, and for
    per-tensor FP8 not even that)."""
    fp8 = form == "fp8"
    if name == "dequant_weights":   # codes (+ scales) in, bf16 weights out
        if fp8:     # the four linears, W8A16 only
            return (12 * d * d * 3 if not w8a8 else 0) / 1e9, "GB", "hbm"
        if form == "mxfp8" and w8a8:   # the adaLN weight only
            return (6 * d * d * 3 + 6 * d * d // 32) / 1e9, "GB", "hbm"
        if form == "int8" and w8a8:
            return (6 * d * d * 3 + 6 * d * 4) / 1e9, "GB", "hbm"
        if form == "int8":   # all five weights, fp32 scale per row (15 d rows)
            return (18 * d * d * 3 + 15 * d * 4) / 1e9, "GB", "hbm"
        if form == "mxfp8":  # all five weights, one E8M0 per 32 codes
            return (18 * d * d * 3 + 18 * d * d // 32) / 1e9, "GB", "hbm"
        return 0.0, "GB", "hbm"
    if name in ("quant_h", "quant_h2") and w8a8 and form != "int8":   # written by the fused LayerNorm
        return 0.0, "GB", "hbm"
    if name == "quant_u" and w8a8 and form == "mxfp8":   # written by the fc1 epilogue
        return 0.0, "GB", "hbm"
    if name.startswith("quant_"):   # bf16 rows in, 1-byte codes + fp32 row / E8M0 block scales out
        K = 4 * d if name == "quant_u" else d
        if form == "mxfp8" and w8a8:
            return (T * K * 3 + T * K // 32) / 1e9, "GB", "hbm"
        return ((T * K * 3 + T * 4) if (form in ("fp8", "int8") and w8a8) else 0) / 1e9, "GB", "hbm"
    if name == "adaln_gemv":   # bf16 or E4M3 weight rows, silu(c), bias in, modulation out
        return (6 * d * d * (1 if fp8 else 2) + 6 * d * 4 * 2 + d * 4) / 1e9, "GB", "hbm"
    if name in ("ln1_modulate", "ln2_modulate"):
        if w8a8 and form in ("fp8", "mxfp8"):   # fp32 rows in, E4M3 codes + scales out
            return (T * d * 5 + (T * d // 32 if form == "mxfp8" else T * 4)) / 1e9, "GB", "hbm"
        return (T * d * 4 + T * d * 2) / 1e9, "GB", "hbm"
    flops = {"gemm_qk": 2 * T * d * 2 * d, "gemm_v_t": 2 * T * d * d, "attention": 4 * T * T * d,
             "gemm_out_residual": 2 * T * d * d, "gemm_fc1_gelu": 8 * T * d * d,
             "gemm_fc2_residual": 8 * T * d * d}[name]
    return flops / 1e12, "TFLOP", "mfma"


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dit_block_kernels_super_hbm_traffic.md")
CSRC = os.path.join(ROOT, "layerwise_weight_streaming_amd", "csrc")
TRAFFIC_KEY = {"adaln_gemv": "adaln_gemv", "ln1_modulate": "ln1", "ln2_modulate": "ln1",
               "gemm_qk": "gemm_qk", "gemm_v_t": "gemm_v_t", "attention": "attention",
               "gemm_out_residual": "gemm_out",
               "gemm_fc1_gelu": "gemm_fc1", "gemm_fc2_residual": "gemm_fc2"}


def kernel_source_sha(fname):
    """sha256 of a kernel source file followed by the shared device header."""
    import hashlib
    h = hashlib.sha256()
    for f in (fname, "device_common.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(kernel, workload):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary, or None.

    The summary holds bytes already scaled by the plain-copy calibration and,
    per kernel, the hash of the source file it was counted on; a changed source
    or another workload gives None.
    """
    key = TRAFFIC_KEY.get(kernel)
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    wl, src, val = None, None, None
    for ln in lines:
        f = ln.split()
        if len(f) == 2 and f[0] == "workload":
            wl = f[1]
        elif len(f) == 4 and f[0] == "kernel_source" and f[1] == key:
            src = (f[2], f[3])
        elif len(f) == 3 and f[0] == "traffic_bytes_per_launch" and f[1] == key:
            val = float(f[2])
    if wl != workload or src is None or val is None:
        return None
    try:
        if kernel_source_sha(src[0]) != src[1]:
            return None
    except OSError:
        return None
    return val


def block_flops(d, T):
    return 24 * T * d * d + 4 * T * T * d + 12 * d * d


def union(iv):
    iv = sorted((a, b) for a, b in iv if b > a)
    out = []
    for a, b in iv:
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def length(u):
    return sum(b - a for a, b in u)


def intersect(u, v):
    i = j = 0
    tot = 0.0
    while i < len(u) and j < len(v):
        a, b = max(u[i][0], v[j][0]), min(u[i][1], v[j][1])
        if b > a:
            tot += b - a
        if u[i][1] < v[j][1]:
            i += 1
        else:
            j += 1
    return tot


def clip(u, lo, hi):
    return [[max(a, lo), min(b, hi)] for a, b in u if min(b, hi) > max(a, lo)]


def overlap_metrics(trace, copy_bytes, flops):
    """Steady window: from the start of the second streamed step's copy to the end of
    compute(last - 1).  Resident steps (read_slot -1) have no copy."""
    n = len(trace)
    if n < 3:
        return None
    streamed = [e for e in trace if e["read_slot"] >= 0]
    lo = streamed[1]["t_copy_begin"] if len(streamed) > 1 else trace[1]["t_compute_begin"]
    hi = trace[n - 2]["t_compute_end"]
    C = clip(union([(e["t_compute_begin"], e["t_compute_end"]) for e in trace]), lo, hi)
    M = clip(union([(e["t_copy_begin"], e["t_copy_end"]) for e in streamed[1:]]), lo, hi)
    c, m, W = length(C), length(M), hi - lo
    in_w = [e for e in trace[1:n - 1]]
    bytes_w = sum(copy_bytes[e["block"]] for e in in_w if e["read_slot"] >= 0)
    flops_w = sum(flops[e["block"]] for e in in_w)
    all_copy = length(union([(e["t_copy_begin"], e["t_copy_end"]) for e in streamed]))
    return {
        "window_ms": W, "compute_busy_ms": c, "copy_busy_ms": m, "copy_busy_step_ms": all_copy,
        "overlap_eff": intersect(C, M) / max(min(c, m), 1e-9),
        "wall_eff": max(c, m) / W,
        "h2d_busy_GBps": bytes_w / (max(m, 1e-9) * 1e-3) / 1e9,
        "h2d_delivered_GBps": bytes_w / (W * 1e-3) / 1e9,
        "mfma_util_busy": flops_w / (c * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "mfma_util_wall": flops_w / (W * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "bound": "h2d" if m > c else "compute",
    }


def environment(torch, dev):
    """Software, GPU, host-link and CPU facts of the machine the run is on."""
    env = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        env["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        env["rocm"] = None
    p = torch.cuda.get_device_properties(dev)
    env["gpu"] = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
                  "compute_units": p.multi_processor_count, "hbm_GiB": round(p.total_memory / 2**30, 1)}
    bus = getattr(p, "pci_bus_id", None)
    if bus is not None:
        bdf = "%04x:%02x:%02x.0" % (getattr(p, "pci_domain_id", 0), bus, getattr(p, "pci_device_id", 0))
        link = {"bdf": bdf}
        for key in ("current_link_speed", "current_link_width", "max_link_speed", "max_link_width", "numa_node"):
            try:
                link[key] = open(f"/sys/bus/pci/devices/{bdf}/{key}").read().strip()
            except OSError:
                link[key] = None
        env["pcie"] = link
        try:  # engine clock levels (current one starred), as the driver lists them
            env["sclk_levels"] = open(f"/sys/bus/pci/devices/{bdf}/pp_dpm_sclk").read().split("\n")[:8]
        except OSError:
            env["sclk_levels"] = None
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    env["cpu"] = {"model": model, "threads_available": len(os.sched_getaffinity(0))}
    return env


def measure_link(torch, dev, gib=1, reps=4):
    """Pinned host -> device copy rate of one large buffer (practical link peak)."""
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        dst.copy_(src, non_blocking=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            dst.copy_(src, non_blocking=True)
        e1.record(s)
    s.synchronize()
    ms = e0.elapsed_time(e1)
    del src, dst
    return reps * n / (ms * 1e-3) / 1e9


def mfma_sustained(torch, dev, iters=2000, reps=3):
    """Dense bf16 MFMA rate with register operands and no memory traffic (libdlo's
    dlo_op_mfma_rate), both instruction shapes, median of reps each: the rate the
    chip holds under its power limit, beside the published 2.5 PFLOP/s."""
    import layerwise_weight_streaming_amd as dlo
    g = torch.Generator(device="cpu").manual_seed(7)
    vals = (torch.rand(4096 * 8, generator=g) * 2 - 1).to(torch.bfloat16).to(dev)
    out = torch.empty(dlo.MFMA_RATE_THREADS, dtype=torch.float32, device=dev)
    s = torch.cuda.Stream(device=dev)
    res = {}
    with torch.cuda.stream(s):
        for form in (0, 1):
            dlo.op_mfma_rate(form, vals.data_ptr(), out.data_ptr(), 200, s.cuda_stream)   # warm
    for rep in range(reps):
        for form in (0, 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(s):
                e0.record(s)
                fl = dlo.op_mfma_rate(form, vals.data_ptr(), out.data_ptr(), iters, s.cuda_stream)
                e1.record(s)
            s.synchronize()
            res.setdefault(form, []).append(fl / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    med = {f: float(np.median(v)) for f, v in res.items()}
    return {"mfma_32x32x16_TFLOPs": med[0], "mfma_16x16x32_TFLOPs": med[1],
            "frac_of_published_peak": {"32x32x16": med[0] / PEAK_BF16_TFLOPS, "16x16x32": med[1] / PEAK_BF16_TFLOPS},
            "note": "dense bf16 MFMA chains on register operands, no memory traffic, median of "
                    f"{reps} runs each, taken right after the timed steps"}


def library_gemm(torch, dev, T, d, reps=5):
    """hipBLASLt (through torch) on the block's five GEMM shapes, for context only
    (the path never calls it): A [T, K] times B^T with B [N, K] row-major, as
    libdlo's GEMMs take them; median of reps after a warm call.

    "ms": the bare product (torch.matmul, bf16 out, no epilogue).
    "ms_with_epilogue": the product plus the epilogue libdlo fuses, done the
    cheapest way torch offers: q,k and v: addmm with the bias (hipBLASLt's bias
    epilogue; v without libdlo's transposed store); fc1: _addmm_activation with
    GELU (hipBLASLt's bias + GELU epilogue, the tanh form, cheaper than erf);
    out and fc2: the product in fp32 (mm with out_dtype, else bf16 widened),
    then y += bias and X += gate * y on the fp32 residual (two elementwise
    passes)."""
    shapes = {"gemm_qk": (2 * d, d), "gemm_v_t": (d, d), "gemm_out_residual": (d, d),
              "gemm_fc1_gelu": (4 * d, d), "gemm_fc2_residual": (d, 4 * d)}
    g = torch.Generator(device="cpu").manual_seed(11)

    def med(f):
        f()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize(dev)
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    out = {}
    for name, (N, K) in shapes.items():
        A = (torch.randn(T, K, generator=g) * 0.5).to(torch.bfloat16).to(dev)
        B = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16).to(dev)
        bias = (torch.randn(N, generator=g) * 0.1).to(dev)
        ms = med(lambda: torch.matmul(A, B.t()))
        rec = {"M": T, "N": N, "K": K, "ms": ms, "TFLOPs": 2 * T * N * K / (ms * 1e-3) / 1e12}
        if name.endswith("_residual"):
            X = torch.randn(T, N, generator=g).to(dev)
            gate = (torch.randn(N, generator=g) * 0.1).to(dev)

            def prod32():
                try:
                    return torch.mm(A, B.t(), out_dtype=torch.float32), "mm out_dtype=float32"
                except Exception:
                    return torch.matmul(A, B.t()).float(), "bf16 matmul widened to fp32"
            rec["epilogue"] = prod32()[1] + ", y += bias, X += gate * y"

            def step():
                y = prod32()[0]
                y.add_(bias)
                X.addcmul_(y, gate)
            rec["ms_with_epilogue"] = med(step)
            del X
        elif name == "gemm_fc1_gelu":
            bb = bias.to(torch.bfloat16)
            rec["epilogue"] = "_addmm_activation(use_gelu=True)"
            rec["ms_with_epilogue"] = med(lambda: torch._addmm_activation(bb, A, B.t(), use_gelu=True))
        else:
            bb = bias.to(torch.bfloat16)
            rec["epilogue"] = "addmm (bias)"
            rec["ms_with_epilogue"] = med(lambda: torch.addmm(bb, A, B.t()))
        out[name] = rec
        del A, B
    torch.cuda.empty_cache()
    return out


def cpu_facts():
    """Host CPU model (lscpu, /proc/cpuinfo), usable cores, and the BLAS library numpy runs on."""
    import subprocess
    facts = {"nproc": len(os.sched_getaffinity(0))}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            k, _, v = ln.partition(":")
            if k.strip() in ("Model name", "Vendor ID", "Socket(s)", "Core(s) per socket", "Thread(s) per core"):
                facts["lscpu_" + k.strip().lower().replace(" ", "_").replace("(s)", "s")] = v.strip()
    except Exception:
        pass
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                facts["cpuinfo_model"] = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        facts["blas"] = [{"api": i.get("internal_api"), "version": i.get("version"),
                          "threads": i.get("num_threads"), "arch": i.get("architecture"),
                          "lib": os.path.basename(i.get("filepath", ""))} for i in threadpool_info()]
    except Exception:
        facts["blas"] = None
    return facts


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count()


def cpu_tiny_stack(seed, threads):
    """The oracle's full tiny stack (3 blocks, d = 256, 64 tokens, 2 passes) with the
    BLAS pool limited to ``threads``: blocks/s over repetitions totalling >= 1 s."""
    import synth
    from oracle import forward as of
    from threadpoolctl import threadpool_limits
    w = synth.WORKLOADS["tiny"]
    st = synth.make_stack(w, seed)
    heads = [w.heads(b) for b in range(w.n_blocks)]
    with threadpool_limits(limits=threads):
        reps, t0 = 0, time.perf_counter()
        while True:
            of.forward_stack(st.x, st.c, st.blocks, heads, w.passes)
            reps += 1
            if time.perf_counter() - t0 >= 1.0:
                break
        dt = (time.perf_counter() - t0) / reps
    return {"threads": threads, "blocks_per_s": w.n_blocks * w.passes / dt,
            "tokens_per_s": w.tokens * w.passes / dt, "s_per_stack": dt}


def cpu_baseline(w, seed, n_blocks, rows=4096, full_block=False):
    """The oracle, untouched, on a bounded sample: sampled output rows of the first block.

    dit_block_rows computes LN1 and the k/v projections for every token and the
    rest of the block for ``rows`` query rows; its FLOPs are counted and the
    rate is scaled to whole blocks by the ratio of FLOPs.  full_block: also time
    the oracle's whole first block (dit_block at the workload's full shape) and
    extrapolate it to the stack, labelled as such.
    """
    import synth
    from oracle import forward as of
    cores = blas_threads()
    d, T, H = w.width(0), w.tokens, w.heads(0)
    params = synth.block_params(seed, 0, d)
    x = synth.activations(seed, T, w.D)
    c = synth.conditioning(seed, w.D)
    rows = min(rows, T)
    idx = np.linspace(0, T - 1, rows).astype(np.int64)
    P = of.param_dict(params)
    reps, t0 = 0, time.perf_counter()
    while True:   # at least ~2 s of work, so small blocks are timed over many repetitions
        of.dit_block_rows(x, c, P, H, idx)
        reps += 1
        if time.perf_counter() - t0 >= 2.0 or reps >= 1000:
            break
    dt = (time.perf_counter() - t0) / reps
    f_sample = 2 * T * d * 2 * d + rows * (2 * d * d + 4 * T * d + 2 * d * d + 16 * d * d) + 12 * d * d
    frac = f_sample / block_flops(d, T)
    blocks_per_s = frac / dt
    out = {"value": blocks_per_s, "unit": "blocks/s", "cores": cores, "kind": "oracle",
           # a pass of the n-block stack moves T tokens
           "tokens_per_s": blocks_per_s * T / n_blocks,
           "sample": (f"float64 oracle, first block of the {w.name} stack (d={d}, T={T}): "
                      f"k/v for all tokens + {rows} sampled query rows, {dt:.3g} s per sample "
                      f"(mean of {reps}) for {frac * 100:.2f}% of a block's FLOPs, scaled by that "
                      f"FLOP fraction"),
           "host": cpu_facts(),
           "tiny_full_stack": [cpu_tiny_stack(seed, 1), cpu_tiny_stack(seed, cores)]}
    if full_block:
        t0 = time.perf_counter()
        of.dit_block(x, c, P, H, progress=lambda msg: print(
            f"[bench] cpu full block: {msg} ({time.perf_counter() - t0:.0f} s)", file=sys.stderr, flush=True))
        tb = time.perf_counter() - t0
        out["full_block"] = {"s_per_block": tb, "blocks_per_s": 1.0 / tb,
                             "extrapolated_stack_s": tb * n_blocks * w.passes,
                             "note": (f"one whole block of the {w.name} stack by the float64 oracle at full "
                                      f"shape (d={d}, T={T}); the stack time is extrapolated "
                                      f"({n_blocks} blocks x {w.passes} passes), not run")}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="super")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--k", type=int, default=None)
    ap.add_argument("--blocks", type=int, default=None, help="use only the first N blocks")
    ap.add_argument("--pinned-limit-gib", type=float, default=56.0,
                    help="ceiling on pinned block memory; blocks beyond it are staged")
    ap.add_argument("--store", default="auto", choices=["auto", "pinned", "pageable"])
    ap.add_argument("--weights", default="bf16", choices=["bf16", "fp8", "int8", "mxfp8"],
                    help="fp8: per-tensor E4M3 weights + fp32 scales; int8: int8 weights + fp32 "
                         "scales per row; mxfp8: E4M3 weights + E8M0 scales per 32 (quantized on the host before "
                         "packing), dequantised on the device after each copy")
    ap.add_argument("--compute", default="bf16", choices=["bf16", "fp8"],
                    help="fp8 (needs --weights fp8 or mxfp8): the four linears of each block as W8A8 "
                         "FP8 products (per-row E4M3 inputs, or per-row MXFP8 inputs with hardware "
                         "block scales); attention stays bf16")
    ap.add_argument("--resident-layers", type=int, default=0,
                    help="keep blocks 0 .. R-1 in device memory; stream the rest")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB "
                         "(a known-size kernel to scale HBM counters by)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full-block", action="store_true",
                    help="also time the oracle's whole first block at full shape (minutes for Super)")
    ap.add_argument("--resident-steps", type=int, default=None,
                    help="timed all-resident steps for the run-based cross-check (default min(steps, 5))")
    ap.add_argument("--async-enqueue", action="store_true",
                    help="timed steps with DLO_ASYNC_ENQUEUE (a library thread enqueues each step)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time hipBLASLt (torch.matmul) on the block's GEMM shapes, for context")
    ap.add_argument("--no-verify", action="store_true",
                    help="skip the streamed == resident bit-exact check")
    args = ap.parse_args()

    if args.compute == "fp8" and args.weights not in ("fp8", "mxfp8", "int8"):
        print("--compute fp8 needs --weights fp8, mxfp8 or int8", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the stack is streamed from this host into this "
              "GPU's two slots; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import layerwise_weight_streaming_amd as dlo
    from layerwise_weight_streaming_amd.runner import StackRunner

    def log(*a):
        print("[bench]", *a, file=sys.stderr, flush=True)

    dlo.lib()
    dev = torch.device("cuda", 0)
    if args.copy_probe_mib > 0:
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        log(f"copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")
        del src, dst
    w = synth.WORKLOADS[args.config]
    if args.k:
        w = w.with_(k=args.k)
    n = args.blocks or w.n_blocks
    T, P = w.tokens, w.passes
    quantized = args.weights != "bf16"
    if quantized:
        specs = [(w.width(b), w.heads(b), dlo.block_schema(w.width(b), form=args.weights)) for b in range(n)]
    else:
        specs = [(w.width(b), w.heads(b), [(nm, dt, int(np.prod(s))) for nm, dt, s in synth.block_schema(w.width(b))])
                 for b in range(n)]

    t_setup = time.perf_counter()
    r = StackRunner(specs, w.k, T, w.D, store_mode=args.store,
                    pinned_limit=int(args.pinned_limit_gib * (1 << 30)))
    t_alloc = time.perf_counter() - t_setup
    store_info = r.store.info()
    log(f"{w.name}: {n} blocks, slot {r.plan.slot_bytes / 1e6:.1f} MB, store {store_info} "
        f"allocated in {t_alloc:.1f} s")
    bufs = {}
    t_gen = t_pack = 0.0
    for b in range(n):
        d = w.width(b)
        key = d
        if key not in bufs:
            bufs[key] = {nm: np.empty(s, dtype=np.uint16 if dt == "bf16" else np.float32)
                         for nm, dt, s in synth.block_schema(d)}
        t0 = time.perf_counter()
        ps = synth.block_params(args.seed, b, d, out_buffers=bufs[key])
        if quantized:   # the loader's finalisation: codes + scales by libdlo's quantizer
            ps = dlo.quantize_block(ps, args.weights)
        t1 = time.perf_counter()
        r.pack(b, [(d, w.heads(b), ps)])
        t2 = time.perf_counter()
        t_gen += t1 - t0
        t_pack += t2 - t1
        if b % 32 == 31:
            log(f"packed {b + 1}/{n} blocks")
    del bufs
    x0 = synth.activations(args.seed, T, w.D)
    c0 = synth.conditioning(args.seed, w.D)
    r.set_inputs(x0, c0)
    log(f"generated in {t_gen:.1f} s, packed in {t_pack:.1f} s")

    link = measure_link(torch, dev)
    log(f"pinned H2D microbenchmark: {link:.1f} GB/s")

    R = args.resident_layers
    w8a8 = args.compute == "fp8"
    cflags = dlo.FP8_COMPUTE if w8a8 else 0
    aflags = dlo.ASYNC_ENQUEUE if args.async_enqueue else 0
    if R:
        r.make_resident(R)
        log(f"{R} resident layers placed")
    for i in range(args.warmup):
        r.forward(P, flags=cflags, n_resident=R, want_run=False)
        r.synchronize()
        log(f"warmup step {i + 1} done")

    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    runs = []
    for _ in range(args.steps):
        if runs:
            runs[-1].enqueued()   # ASYNC_ENQUEUE: the previous step's program is fully enqueued
        runs.append(r.forward(P, flags=dlo.TRACE_TIMING | cflags | aflags, n_resident=R))
    runs[-1].enqueued()
    r.synchronize()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.2f} s")

    infos = [r.plan.block_info(b) for b in range(n)]
    copy_bytes = [i["copy_bytes"] for i in infos]
    flops = [block_flops(i["d_model"], T) for i in infos]
    names = dlo.kernel_names()
    per_kernel = np.zeros(len(names))
    launches = 0
    work = np.zeros(len(names))
    ov = []
    step_ms = []   # each step's GPU time: its trace is relative to the step's own start event
    for run in runs:
        tr = run.trace()
        kt = run.kernel_times()
        step_ms.append(max(e["t_compute_end"] for e in tr))
        per_kernel += kt.sum(axis=0)
        launches += kt.shape[0]
        for e, row in zip(tr, kt):
            d, form = infos[e["block"]]["d_model"], infos[e["block"]]["form"]
            for j, nm in enumerate(names):
                work[j] += kernel_work(nm, d, T, form, w8a8)[0]
        m = overlap_metrics(tr, copy_bytes, flops)
        if m:
            ov.append(m)
        run.close()
    avg = {k: float(np.median([m[k] for m in ov])) for k in ov[0] if k != "bound"} if ov else {}
    bound = ov[0]["bound"] if ov else None
    jdom = int(np.argmax(per_kernel))
    dname = names[jdom]
    _, unit, kbound = kernel_work(dname, w.width(0), T)
    avg_ms = per_kernel[jdom] / launches
    achieved = work[jdom] / launches / (avg_ms * 1e-3)
    fp8_mfma = w8a8 and dname.startswith("gemm_") and any(i["form"] in ("fp8", "mxfp8") for i in infos)
    i8_mfma = w8a8 and dname.startswith("gemm_") and any(i["form"] == "int8" for i in infos)
    peak = ((PEAK_INT8_TOPS if i8_mfma else PEAK_FP8_TFLOPS if fp8_mfma else PEAK_BF16_TFLOPS)
            if kbound == "mfma" else PEAK_HBM_GBS)
    roofline = {"kernel": dname, "bound": kbound, "achieved": achieved, "peak": peak,
                "unit": ("TOP/s" if i8_mfma else "TFLOP/s") if kbound == "mfma" else "GB/s",
                "frac": achieved / peak,
                "traffic": counted_traffic(dname, w.name),
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "avg_launch_ms": avg_ms,
                "per_launch": f"{work[jdom] / launches:.4g} {unit}"}

    mfma_ceiling = mfma_sustained(torch, dev)
    log(f"sustained MFMA rate: {mfma_ceiling['mfma_32x32x16_TFLOPs']:.0f} / "
        f"{mfma_ceiling['mfma_16x16x32_TFLOPs']:.0f} TFLOP/s (32x32x16 / 16x16x32)")

    if args.library_gemm:
        lib_gemm = library_gemm(torch, dev, T, w.width(0))
        log("hipBLASLt on the block's GEMM shapes (bare / with the epilogue): " +
            ", ".join(f"{k} {v['ms']:.3f} / {v['ms_with_epilogue']:.3f} ms" for k, v in lib_gemm.items()))

    blocks_done = n * P * args.steps
    result = {
        "metric": "DiT blocks/s with streaming",
        "value": blocks_done / wall,
        "unit": "blocks/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "step_ms": {"per_step": step_ms, "median": float(np.median(step_ms))},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("int8+bf16" if args.weights == "int8" else "fp8e4m3+bf16") if w8a8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "n_blocks": n,
                   "widths": list(w.widths), "head_dim": w.head_dim, "tokens": T, "batch": 1,
                   "k": w.k, "passes": P, "slot_bytes": r.plan.slot_bytes,
                   "block_copy_bytes": max(copy_bytes), "host_store_bytes": sum(copy_bytes),
                   "parallelism": "single GPU", "store": args.store, "resident_layers": R,
                   "weights": args.weights, "compute": args.compute, "async_enqueue": args.async_enqueue,
                   "pinned_blocks": store_info["pinned_blocks"],
                   "staged_blocks": store_info["staged_blocks"]},
        "tokens_per_s": T * P * args.steps / wall,
        "h2d": {"busy_GBps": avg.get("h2d_busy_GBps"), "delivered_GBps": avg.get("h2d_delivered_GBps"),
                "link_peak_GBps": LINK_PEAK_GBS, "measured_link_GBps": link,
                "frac_of_link_peak": (avg.get("h2d_busy_GBps") or 0) / LINK_PEAK_GBS},
        "mfma_util": {"busy": avg.get("mfma_util_busy"), "wall": avg.get("mfma_util_wall"),
                      "peak_TFLOPs": PEAK_BF16_TFLOPS,
                      "basis": ("bf16-equivalent: every block FLOP against the bf16 dense peak, although "
                                "the linears run on 8-bit MFMA" if w8a8 else
                                "every block FLOP against the bf16 dense peak")},
        "overlap_eff": avg.get("overlap_eff"), "wall_eff": avg.get("wall_eff"),
        "bound_resource": bound,
        "steady_window": {k: avg.get(k) for k in ("window_ms", "compute_busy_ms", "copy_busy_ms")},
        "per_kernel_ms_per_block": {nm: per_kernel[j] / launches for j, nm in enumerate(names)},
        "roofline": roofline,
        "mfma_sustained": mfma_ceiling,
        # device weight memory of the streamed path: exactly two slots of the largest block
        "weight_hbm": {"two_slots_bytes": 2 * r.plan.slot_bytes, "allocated_bytes": r.slot_alloc_bytes},
        "setup_s": {"pin_alloc": t_alloc, "generate": t_gen, "pack": t_pack},
        "env": environment(torch, dev),
    }
    if args.library_gemm:
        result["library_gemm"] = {"note": "hipBLASLt through torch, bf16; ms: bare product, "
                                          "ms_with_epilogue: with the epilogue libdlo fuses, by torch; context only",
                                  **lib_gemm}

    if not args.no_verify:
        # the pages' own correctness criterion at full scale: streamed == resident, bit-exact
        log("verify: streamed vs resident, one step each from the same inputs")
        r.set_inputs(x0, c0)
        r.forward(P, flags=cflags, n_resident=R, want_run=False)
        xs = r.x_host()
        r.set_inputs(x0, c0)
        r.make_resident()
        r.synchronize()
        r.forward(P, flags=cflags, resident=True, want_run=False)
        xr = r.x_host()
        result["streamed_equals_resident"] = bool(np.array_equal(xs.view(np.uint32), xr.view(np.uint32)))
        result["finite"] = bool(np.isfinite(xs).all())
        # run-based cross-check of the overlap: an all-resident step is the compute
        # alone; the copy stream's busy time per streamed step is the copy alone.
        # Both step times are GPU times from the same HIP events (first event to the
        # last block's end), medians over timed steps after a warm step each.
        n_res = args.resident_steps if args.resident_steps is not None else min(args.steps, 5)
        res_ms = []
        for _ in range(max(n_res, 1)):
            run = r.forward(P, flags=dlo.TRACE_TIMING | cflags, resident=True)
            res_ms.append(max(e["t_compute_end"] for e in run.trace()))
            run.close()
        r.free_resident()
        t_res = float(np.median(res_ms)) * 1e-3
        t_str = float(np.median(step_ms)) * 1e-3
        t_copy = avg.get("copy_busy_step_ms", 0.0) * 1e-3
        result["cross_check"] = {
            "streamed_step_ms": t_str * 1e3, "resident_step_ms": t_res * 1e3,
            "resident_steps": len(res_ms), "streamed_steps": len(step_ms),
            "copy_busy_step_ms": t_copy * 1e3,
            "run_overlap": (t_copy + t_res - t_str) / max(min(t_copy, t_res), 1e-9),
            "streaming_cost": t_str / t_res - 1.0,
            "basis": "medians of per-step GPU times (HIP events) over the timed streamed and resident steps",
        }
        log(f"verify: equal={result['streamed_equals_resident']}; resident step {t_res * 1e3:.0f} ms "
            f"vs streamed {t_str * 1e3:.0f} ms (medians of {len(res_ms)} and {len(step_ms)} steps)")

    r.close()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle sample)")
        result["cpu_baseline"] = cpu_baseline(w, args.seed, n, full_block=args.cpu_full_block)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
