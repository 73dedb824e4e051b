"""Python binding of libdlo (C ABI in include/dlo.h): argument marshalling only.

Every step of the weight-streaming path -- planning, packing, placement, the
two-slot schedule and every kernel of the block forward -- runs inside
libdlo.so.  Device memory and streams are passed as integer addresses
(``tensor.data_ptr()``, ``torch.cuda.Stream().cuda_stream``); this module never
imports torch.  If the library is not built, importing the binding works but
every call raises ``RuntimeError``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdlo.so")

DLO_OK = 0
STATUS = {0: "DLO_OK", -1: "DLO_E_ARG", -2: "DLO_E_HOSTMEM", -3: "DLO_E_PIN",
          -4: "DLO_E_SLOT_SMALL", -5: "DLO_E_PLAN_MISMATCH", -6: "DLO_E_HIP",
          -7: "DLO_E_STATE", -8: "DLO_E_UNSUPPORTED", -9: "DLO_E_WORKSPACE"}
DTYPES = {"bf16": 0, "f32": 1, "fp8": 2, "i8": 3, "e8m0": 4}   # fp8: OCP E4M3; e8m0: MX block scale
DTYPE_NAMES = {v: k for k, v in DTYPES.items()}
STORE_PINNED, STORE_PAGEABLE, STORE_AUTO = 0, 1, 2
TRACE_DIGEST, TRACE_TIMING, RESIDENT, FP8_COMPUTE, ASYNC_ENQUEUE = 1, 2, 4, 8, 16
EPI_BIAS, EPI_BIAS_GELU, EPI_GATED_RESIDUAL, EPI_BIAS_T = 0, 1, 2, 3
KERNELS_PER_BLOCK = 14
MAX_GROUPS = 3
OP_KIND = {0: "copy", 1: "compute", 2: "record", 3: "wait"}
OP_STREAM = {0: "compute", 1: "copy"}
OP_EVENT = {0: "copied0", 1: "copied1", 2: "computed0", 3: "computed1", 4: "start"}


class DLOError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class Param(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int32), ("numel", ctypes.c_int64),
                ("src", ctypes.c_void_p)]


class Block(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_params", ctypes.c_int32), ("params", ctypes.POINTER(Param))]


class BlockInfo(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_params", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("dtype", ctypes.c_int32 * MAX_GROUPS), ("numel", ctypes.c_int64 * MAX_GROUPS),
                ("shard", ctypes.c_int64 * MAX_GROUPS), ("region", ctypes.c_int64 * MAX_GROUPS),
                ("extent", ctypes.c_int64), ("copy_bytes", ctypes.c_int64),
                ("is_dit", ctypes.c_int32)]


class SchedOp(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("stream", ctypes.c_int32), ("block", ctypes.c_int32),
                ("slot", ctypes.c_int32), ("event", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("step", ctypes.c_int64)]


class ForwardArgs(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_void_p * 2), ("slot_bytes", ctypes.c_int64),
                ("x", ctypes.c_void_p), ("x_row_stride", ctypes.c_int64),
                ("cond", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_int64), ("compute_stream", ctypes.c_void_p),
                ("copy_stream", ctypes.c_void_p), ("tokens", ctypes.c_int32),
                ("passes", ctypes.c_int32), ("flags", ctypes.c_uint32), ("n_resident", ctypes.c_int32),
                ("resident_blocks", ctypes.POINTER(ctypes.c_void_p)),
                ("batch", ctypes.c_int32), ("reserved0", ctypes.c_int32), ("cond_stride", ctypes.c_int64)]


class SlotEvent(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("pass_", ctypes.c_int32), ("block", ctypes.c_int32),
                ("read_slot", ctypes.c_int32), ("prefetch_block", ctypes.c_int32),
                ("prefetch_slot", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("prefetch_bytes", ctypes.c_int64), ("digest_pre", ctypes.c_uint64),
                ("digest_post", ctypes.c_uint64), ("t_copy_begin", ctypes.c_float),
                ("t_copy_end", ctypes.c_float), ("t_compute_begin", ctypes.c_float),
                ("t_compute_end", ctypes.c_float)]


_lib = None

_SIGS = {
    "dlo_last_error": (ctypes.c_char_p, []),
    "dlo_block_schema": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p),
                                        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]),
    "dlo_kernel_name": (ctypes.c_char_p, [ctypes.c_int32]),
    "dlo_plan_blocks": (ctypes.c_int, [ctypes.POINTER(Block), ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_void_p)]),
    "dlo_plan_destroy": (None, [ctypes.c_void_p]),
    "dlo_plan_n_blocks": (ctypes.c_int32, [ctypes.c_void_p]),
    "dlo_plan_k": (ctypes.c_int32, [ctypes.c_void_p]),
    "dlo_plan_slot_bytes": (ctypes.c_int64, [ctypes.c_void_p]),
    "dlo_plan_block_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(BlockInfo)]),
    "dlo_plan_param_offset": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_int64)]),
    "dlo_plan_workspace_bytes": (ctypes.c_int64, [ctypes.c_void_p, ctypes.c_int32]),
    "dlo_plan_schedule": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(SchedOp),
                                         ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "dlo_plan_schedule_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(SchedOp), ctypes.c_int64,
                                            ctypes.POINTER(ctypes.c_int64)]),
    "dlo_host_store_create": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint32,
                                             ctypes.POINTER(ctypes.c_void_p)]),
    "dlo_host_store_create_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int64,
                                                ctypes.POINTER(ctypes.c_void_p)]),
    "dlo_host_store_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]),
    "dlo_host_store_destroy": (None, [ctypes.c_void_p]),
    "dlo_pack_host_shards": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(Block)]),
    "dlo_host_store_shard": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                            ctypes.POINTER(ctypes.c_int64)]),
    "dlo_host_store_complete": (ctypes.c_int32, [ctypes.c_void_p]),
    "dlo_forward_stack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ForwardArgs),
                                         ctypes.POINTER(ctypes.c_void_p)]),
    "dlo_place_block": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "dlo_slot_trace": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(SlotEvent), ctypes.c_int64,
                                      ctypes.POINTER(ctypes.c_int64)]),
    "dlo_run_kernel_times": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float),
                                            ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "dlo_run_destroy": (None, [ctypes.c_void_p]),
    "dlo_run_enqueued": (ctypes.c_int, [ctypes.c_void_p]),
    "dlo_op_adaln": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "dlo_op_mfma_rate": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]),
    "dlo_op_adaln_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p]),
    "dlo_op_ln_modulate": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_int32] + [ctypes.c_void_p] * 7),
    "dlo_op_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_void_p]),
    "dlo_op_adaln_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p]),
    "dlo_op_quantize_rows_mxfp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "dlo_op_gemm_mxfp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_void_p]),
    "dlo_op_quantize_rows_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                                ctypes.c_void_p, ctypes.c_void_p]),
    "dlo_op_gemm_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]),
    "dlo_op_quantize_rows_int8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                                 ctypes.c_void_p, ctypes.c_void_p]),
    "dlo_op_gemm_int8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]),
    "dlo_op_v_transpose": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p]),
    "dlo_op_attention": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_void_p]),
    "dlo_block_schema_fp8": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p),
                                            ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]),
    "dlo_quantize_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.POINTER(ctypes.c_float)]),
    "dlo_block_schema_int8": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p),
                                             ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]),
    "dlo_block_schema_mxfp8": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p),
                                              ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]),
    "dlo_quantize_int8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_void_p]),
    "dlo_quantize_mxfp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p]),
    "dlo_op_dequant_int8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]),
    "dlo_op_dequant_mxfp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]),
    "dlo_op_dequant_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]),
    "dlo_op_digest": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_int64), ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_void_p]),
}

EXPORTED = sorted(_SIGS)


def lib():
    """The loaded libdlo.so; raises RuntimeError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libdlo.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != DLO_OK:
        raise DLOError(rc, (lib().dlo_last_error() or b"").decode())


def last_error() -> str:
    return (lib().dlo_last_error() or b"").decode()


FORMS = ("bf16", "fp8", "int8", "mxfp8")   # dlo_block_info.is_dit 1 .. 4


def block_schema(d: int, fp8: bool = False, form: str | None = None):
    """[(name, dtype, numel)] of the DiT block schema or one of its quantised forms
    ("fp8", "int8", "mxfp8") as libdlo defines it."""
    form = form or ("fp8" if fp8 else "bf16")
    fn, count = {"bf16": (lib().dlo_block_schema, 16), "fp8": (lib().dlo_block_schema_fp8, 21),
                 "int8": (lib().dlo_block_schema_int8, 21), "mxfp8": (lib().dlo_block_schema_mxfp8, 21)}[form]
    out = []
    for i in range(count):
        name, dt, n = ctypes.c_char_p(), ctypes.c_int32(), ctypes.c_int64()
        _check(fn(d, i, ctypes.byref(name), ctypes.byref(dt), ctypes.byref(n)))
        out.append((name.value.decode(), DTYPE_NAMES[dt.value], n.value))
    return out


def quantize_fp8(w_bf16):
    """dlo_quantize_fp8 on a host array of bf16 bit patterns -> (E4M3 codes, float32 scale)."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    codes = np.empty(w.shape, dtype=np.uint8)
    scale = ctypes.c_float()
    _check(lib().dlo_quantize_fp8(w.ctypes.data_as(ctypes.c_void_p), w.size,
                                  codes.ctypes.data_as(ctypes.c_void_p), ctypes.byref(scale)))
    return codes, np.float32(scale.value)


def quantize_int8(w_bf16):
    """dlo_quantize_int8 on a host matrix of bf16 bit patterns -> (int8 codes, float32 row scales)."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    if w.ndim != 2:
        raise ValueError("quantize_int8 takes a matrix")
    codes = np.empty(w.shape, dtype=np.int8)
    scales = np.empty(w.shape[0], dtype=np.float32)
    _check(lib().dlo_quantize_int8(w.ctypes.data_as(ctypes.c_void_p), w.shape[0], w.shape[1],
                                   codes.ctypes.data_as(ctypes.c_void_p), scales.ctypes.data_as(ctypes.c_void_p)))
    return codes, scales


def quantize_mxfp8(w_bf16):
    """dlo_quantize_mxfp8 on a host matrix of bf16 bit patterns -> (E4M3 codes, E8M0 scales block-major
    [cols / 32, rows])."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    if w.ndim != 2:
        raise ValueError("quantize_mxfp8 takes a matrix")
    codes = np.empty(w.shape, dtype=np.uint8)
    scales = np.empty((w.shape[1] // 32, w.shape[0]), dtype=np.uint8)
    _check(lib().dlo_quantize_mxfp8(w.ctypes.data_as(ctypes.c_void_p), w.shape[0], w.shape[1],
                                    codes.ctypes.data_as(ctypes.c_void_p), scales.ctypes.data_as(ctypes.c_void_p)))
    return codes, scales


def quantize_block(params, form):
    """A bf16 block's [(name, dtype, array)] -> its quantised form, with libdlo's quantizers
    (the loader's finalisation): "fp8" (per-tensor), "int8" (per-row) or "mxfp8" (32-blocks)."""
    out = []
    for name, dt, arr in params:
        if dt != "bf16":
            out.append((name, dt, arr))
        elif form == "fp8":
            codes, scale = quantize_fp8(arr)
            out += [(name, "fp8", codes), (name + "_scale", "f32", np.array([scale], np.float32))]
        elif form == "int8":
            codes, scales = quantize_int8(arr)
            out += [(name, "i8", codes), (name + "_scale", "f32", scales)]
        elif form == "mxfp8":
            codes, scales = quantize_mxfp8(arr)
            out += [(name, "fp8", codes), (name + "_scale", "e8m0", scales.reshape(-1))]
        else:
            raise ValueError(f"unknown form {form!r}")
    return out


def kernel_names():
    return [lib().dlo_kernel_name(j).decode() for j in range(KERNELS_PER_BLOCK)]


class _BlockArray:
    """ctypes Block[] built from [(d, heads, [(name, dtype, numel_or_array)])]; keeps refs alive."""

    def __init__(self, blocks):
        self._keep = []
        self.arr = (Block * len(blocks))()
        for i, (d, heads, params) in enumerate(blocks):
            ps = (Param * len(params))()
            for j, (name, dt, val) in enumerate(params):
                nm = name.encode()
                self._keep.append(nm)
                ps[j].name = nm
                ps[j].dtype = DTYPES[dt] if isinstance(dt, str) else int(dt)
                if isinstance(val, np.ndarray):
                    a = np.ascontiguousarray(val)
                    self._keep.append(a)
                    ps[j].numel = a.size
                    ps[j].src = a.ctypes.data if a.size else None
                else:
                    ps[j].numel = int(val)
                    ps[j].src = None
            self._keep.append(ps)
            self.arr[i].d_model = d
            self.arr[i].n_heads = heads
            self.arr[i].n_params = len(params)
            self.arr[i].params = ps


class Plan:
    """dlo_plan_blocks: blocks = [(d_model, n_heads, [(name, dtype, numel or ndarray)])]."""

    def __init__(self, blocks, k: int):
        ba = _BlockArray(blocks)
        h = ctypes.c_void_p()
        _check(lib().dlo_plan_blocks(ba.arr, len(blocks), k, ctypes.byref(h)))
        self.h = h
        self.k = k

    def close(self):
        if self.h:
            lib().dlo_plan_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def n_blocks(self):
        return lib().dlo_plan_n_blocks(self.h)

    @property
    def slot_bytes(self):
        return lib().dlo_plan_slot_bytes(self.h)

    def block_info(self, b):
        bi = BlockInfo()
        _check(lib().dlo_plan_block_info(self.h, b, ctypes.byref(bi)))
        g = bi.n_groups
        return {"d_model": bi.d_model, "n_heads": bi.n_heads, "n_params": bi.n_params,
                "n_groups": g, "dtype": [DTYPE_NAMES[bi.dtype[i]] for i in range(g)],
                "numel": list(bi.numel[:g]), "shard": list(bi.shard[:g]),
                "region": list(bi.region[:g]), "extent": bi.extent,
                "copy_bytes": bi.copy_bytes, "is_dit": bool(bi.is_dit), "fp8": bi.is_dit == 2,
                "form": FORMS[bi.is_dit - 1] if bi.is_dit else None}

    def param_offset(self, b, p):
        v = ctypes.c_int64()
        _check(lib().dlo_plan_param_offset(self.h, b, p, ctypes.byref(v)))
        return v.value

    def workspace_bytes(self, tokens):
        v = lib().dlo_plan_workspace_bytes(self.h, tokens)
        if v < 0:
            raise DLOError(-1, last_error())
        return v

    def schedule(self, passes, n_resident=0):
        """The enqueued program as oracle-style tuples (dlo_plan_schedule_ex)."""
        n = ctypes.c_int64()
        _check(lib().dlo_plan_schedule_ex(self.h, passes, n_resident, None, 0, ctypes.byref(n)))
        ops = (SchedOp * n.value)()
        _check(lib().dlo_plan_schedule_ex(self.h, passes, n_resident, ops, n.value, ctypes.byref(n)))
        out = []
        for o in ops:
            kind, stream = OP_KIND[o.kind], OP_STREAM[o.stream]
            if kind == "copy":
                out.append((kind, stream, o.block, o.slot))
            elif kind == "compute":
                out.append((kind, stream, o.block, o.slot, o.step))
            else:
                out.append((kind, stream, OP_EVENT[o.event]))
        return out


class HostStore:
    """dlo_host_store_create_ex + dlo_pack_host_shards.

    mode: "pinned" (every block pinned), "pageable" (every block staged through two
    pinned buffers), or "auto" (pin blocks up to ``pinned_limit`` bytes, stage the rest).
    ``pinned=True/False`` is shorthand for "pinned" / "pageable".
    """

    def __init__(self, plan: Plan, pinned: bool = True, mode: str = None, pinned_limit: int = 0):
        if mode is None:
            mode = "pinned" if pinned else "pageable"
        flags = {"pinned": STORE_PINNED, "pageable": STORE_PAGEABLE, "auto": STORE_AUTO}[mode]
        h = ctypes.c_void_p()
        _check(lib().dlo_host_store_create_ex(plan.h, flags, int(pinned_limit), ctypes.byref(h)))
        self.h = h
        self.plan = plan
        self.mode = mode

    def info(self):
        pb, by, sb = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
        _check(lib().dlo_host_store_info(self.h, ctypes.byref(pb), ctypes.byref(by), ctypes.byref(sb)))
        return {"pinned_blocks": pb.value, "pinned_bytes": by.value, "staged_blocks": sb.value}

    def close(self):
        if self.h:
            lib().dlo_host_store_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def pack(self, b_begin, blocks):
        """blocks[i] = (d, heads, [(name, dtype, ndarray)]) for block b_begin + i."""
        ba = _BlockArray(blocks)
        _check(lib().dlo_pack_host_shards(self.h, b_begin, b_begin + len(blocks), ba.arr))

    @property
    def complete(self):
        return bool(lib().dlo_host_store_complete(self.h))

    def shard(self, b, g, r):
        """A copy of shard r of group g of block b, as bytes (uint8 array)."""
        p, n = ctypes.c_void_p(), ctypes.c_int64()
        _check(lib().dlo_host_store_shard(self.h, b, g, r, ctypes.byref(p), ctypes.byref(n)))
        if n.value == 0:
            return np.zeros(0, dtype=np.uint8)
        return np.ctypeslib.as_array(ctypes.cast(p, ctypes.POINTER(ctypes.c_uint8)),
                                     shape=(n.value,)).copy()


class Run:
    def __init__(self, h):
        self.h = h

    def close(self):
        if self.h:
            lib().dlo_run_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def enqueued(self):
        """dlo_run_enqueued: joins an ASYNC_ENQUEUE run's enqueue (returns at once otherwise)."""
        _check(lib().dlo_run_enqueued(self.h))

    def trace(self):
        n = ctypes.c_int64()
        _check(lib().dlo_slot_trace(self.h, None, 0, ctypes.byref(n)))
        recs = (SlotEvent * n.value)()
        _check(lib().dlo_slot_trace(self.h, recs, n.value, ctypes.byref(n)))
        return [{f: getattr(r, f) for f, _ in SlotEvent._fields_ if f != "pad"} for r in recs]

    def kernel_times(self):
        """[steps, KERNELS_PER_BLOCK] milliseconds (needs TRACE_TIMING)."""
        n = ctypes.c_int64()
        _check(lib().dlo_run_kernel_times(self.h, None, 0, ctypes.byref(n)))
        buf = (ctypes.c_float * n.value)()
        _check(lib().dlo_run_kernel_times(self.h, buf, n.value, ctypes.byref(n)))
        return np.frombuffer(buf, dtype=np.float32).reshape(-1, KERNELS_PER_BLOCK).copy()


def forward_stack(plan, store, *, x, x_row_stride, cond, workspace, workspace_bytes,
                  compute_stream, copy_stream, tokens, passes, slots=(0, 0), slot_bytes=0,
                  flags=0, resident_blocks=None, n_resident=0, want_run=True, batch=1, cond_stride=0):
    """dlo_forward_stack; device pointers and streams as integers."""
    a = ForwardArgs()
    a.slot[0], a.slot[1] = slots
    a.slot_bytes = slot_bytes
    a.x, a.x_row_stride, a.cond = x, x_row_stride, cond
    a.workspace, a.workspace_bytes = workspace, workspace_bytes
    a.compute_stream, a.copy_stream = compute_stream, copy_stream
    a.tokens, a.passes, a.flags = tokens, passes, flags
    a.n_resident = n_resident
    a.batch, a.cond_stride = batch, cond_stride
    keep = None
    if resident_blocks is not None:
        keep = (ctypes.c_void_p * len(resident_blocks))(*resident_blocks)
        a.resident_blocks = ctypes.cast(keep, ctypes.POINTER(ctypes.c_void_p))
    h = ctypes.c_void_p()
    _check(lib().dlo_forward_stack(plan.h, store.h if store is not None else None, ctypes.byref(a),
                                   ctypes.byref(h) if want_run else None))
    return Run(h) if want_run else None


def place_block(plan, store, b, dst, dst_bytes, stream):
    _check(lib().dlo_place_block(plan.h, store.h, b, dst, dst_bytes, stream))


def op_adaln(W, b, cond, rows, d, out, workspace, workspace_bytes, stream):
    _check(lib().dlo_op_adaln(W, b, cond, rows, d, out, workspace, workspace_bytes, stream))


def op_adaln_noalloc(W, b, cond, rows, d, out, stream):
    _check(lib().dlo_op_adaln_noalloc(W, b, cond, rows, d, out, stream))


NOALLOC_MAX_D = 8192
MFMA_RATE_THREADS = 256 * 512


def op_mfma_rate(form, in_ptr, out_ptr, iters, stream):
    """Enqueues the sustained-MFMA-rate probe; returns the FLOPs it performs."""
    fl = ctypes.c_double(0.0)
    _check(lib().dlo_op_mfma_rate(form, in_ptr, out_ptr, iters, ctypes.byref(fl), stream))
    return fl.value


def op_ln_modulate(x, ldx, T, d, gamma, beta, eps, shift, scale, out, stream):
    _check(lib().dlo_op_ln_modulate(x, ldx, T, d, gamma, beta, eps, shift, scale, out, stream))


def op_gemm(A, lda, B, ldb, M, N, K, bias, gate, C, ldc, epilogue, stream):
    _check(lib().dlo_op_gemm(A, lda, B, ldb, M, N, K, bias, gate, C, ldc, epilogue, stream))


def op_adaln_fp8(W, w_scale, b, cond, rows, d, out, workspace, workspace_bytes, stream):
    _check(lib().dlo_op_adaln_fp8(W, w_scale, b, cond, rows, d, out, workspace, workspace_bytes, stream))


def op_quantize_rows_mxfp8(x, ldx, M, K, codes, ldq, scales, lds, stream):
    _check(lib().dlo_op_quantize_rows_mxfp8(x, ldx, M, K, codes, ldq, scales, lds, stream))


def op_gemm_mxfp8(A, lda, a_scales, lds_a, B, ldb, b_scales, lds_b, M, N, K, bias, gate, C, ldc, epilogue, stream):
    _check(lib().dlo_op_gemm_mxfp8(A, lda, a_scales, lds_a, B, ldb, b_scales, lds_b, M, N, K, bias, gate, C, ldc,
                                   epilogue, stream))


def op_quantize_rows_fp8(x, ldx, M, K, codes, ldq, scales, stream):
    _check(lib().dlo_op_quantize_rows_fp8(x, ldx, M, K, codes, ldq, scales, stream))


def op_gemm_fp8(A, lda, a_scale, B, ldb, b_scale, M, N, K, bias, gate, C, ldc, epilogue, stream):
    _check(lib().dlo_op_gemm_fp8(A, lda, a_scale, B, ldb, b_scale, M, N, K, bias, gate, C, ldc, epilogue,
                                 stream))


def op_quantize_rows_int8(x, ldx, M, K, codes, ldq, scales, stream):
    _check(lib().dlo_op_quantize_rows_int8(x, ldx, M, K, codes, ldq, scales, stream))


def op_gemm_int8(A, lda, a_scale, B, ldb, b_scale, M, N, K, bias, gate, C, ldc, epilogue, stream):
    _check(lib().dlo_op_gemm_int8(A, lda, a_scale, B, ldb, b_scale, M, N, K, bias, gate, C, ldc, epilogue,
                                  stream))


def v_t_stride(T):
    """Row stride (elements) of the feature-major V^T the attention reads: T rounded up to 64."""
    return (T + 63) // 64 * 64


def op_v_transpose(qkv, ldqkv, T, d, vt, ldvt, stream):
    _check(lib().dlo_op_v_transpose(qkv, ldqkv, T, d, vt, ldvt, stream))


def op_attention(qkv, ldqkv, vt, ldvt, T, H, dh, out, ldo, stream):
    _check(lib().dlo_op_attention(qkv, ldqkv, vt, ldvt, T, H, dh, out, ldo, stream))


def op_dequant_fp8(codes, n, scale, out, stream):
    _check(lib().dlo_op_dequant_fp8(codes, n, scale, out, stream))


def op_dequant_int8(codes, rows, cols, scales, out, stream):
    _check(lib().dlo_op_dequant_int8(codes, rows, cols, scales, out, stream))


def op_dequant_mxfp8(codes, rows, cols, scales, out, stream):
    _check(lib().dlo_op_dequant_mxfp8(codes, rows, cols, scales, out, stream))


def op_digest(base, offsets, lengths, out, stream):
    n = len(offsets)
    o = (ctypes.c_int64 * max(n, 1))(*offsets)
    l_ = (ctypes.c_int64 * max(n, 1))(*lengths)
    _check(lib().dlo_op_digest(base, o, l_, n, out, stream))
