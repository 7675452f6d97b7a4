"""ctypes binding of libwq (argument marshalling only).

Each function has the name and argument order of the C entry point declared
in include/wq.h.  Buffers are torch tensors on the GPU (or raw device
addresses as ints, or None for a nullable pointer); sizes are ints; `stream`
defaults to torch's current stream on the current device.  Every step of the
computation runs in the HIP library; a non-OK status raises WQError.

The library is loaded from this package directory (built in-tree by
``weight_only_quantized_wq_amd.build``).  Loading fails loudly if it is
missing: there is no fallback implementation.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwq.so")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32

_SIGNATURES = {
    "wq_quantize_int8": [_P, _I64, _I64, _P, _P, _P],
    "wq_quantize_int4g32": [_P, _I64, _I64, _P, _P, _P],
    "wq_quantize_int4": [_P, _I64, _I64, _I32, _P, _P, _P],
    "wq_gemv_bf16": [_P, _P, _I64, _I64, _P, _P, _P],
    "wq_gemv_int8": [_P, _P, _P, _I64, _I64, _P, _P, _P],
    "wq_gemv_int4g32": [_P, _P, _P, _I64, _I64, _P, _P, _P],
    "wq_gemv_int4": [_P, _P, _P, _I64, _I64, _I32, _P, _P, _P],
    "wq_gemm_smallM": [_P, _I64, _P, _P, _I64, _I64, _P, _P, _P],
    "wq_gemm_smallM_int8": [_P, _I64, _P, _P, _I64, _I64, _P, _P, _P],
    "wq_gemm_smallM_int4": [_P, _I64, _P, _P, _I64, _I64, _I32, _P, _P, _P],
    "moe_top2_gemv": [_P, _P, _I64, _P, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P],
}

WQ_FORMAT = {"bf16": 1, "int8": 2, "int4g32": 3, "int4g64": 4, "int4g128": 5, "int4g256": 6, "int4pc": 7}


class wq_matrix(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("aux", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("y_f32", ctypes.c_void_p), ("y_bf16", ctypes.c_void_p)]


class wq_step_plan(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("m", ctypes.c_int32), ("count", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("total_batches", ctypes.c_int64), ("workspace", ctypes.c_void_p)]


class wq_moe_layer(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("logits", ctypes.c_void_p), ("w13", ctypes.c_void_p),
                ("s13", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("s2", ctypes.c_void_p),
                ("work", ctypes.c_void_p), ("y_f32", ctypes.c_void_p), ("y_bf16", ctypes.c_void_p),
                ("sel", ctypes.c_void_p), ("gates", ctypes.c_void_p)]


class wq_moe_plan(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int64), ("f", ctypes.c_int64), ("e", ctypes.c_int32), ("count", ctypes.c_int32),
                ("grid13", ctypes.c_int32), ("grid2", ctypes.c_int32), ("workspace", ctypes.c_void_p)]


WQ_STATUS = {0: "WQ_OK", 1: "WQ_ERR_NULL", 2: "WQ_ERR_SHAPE", 3: "WQ_ERR_ALIGN", 4: "WQ_ERR_DEVICE",
             5: "WQ_ERR_LAUNCH"}


class WQError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.fn = fn
        self.status = status
        self.detail = detail
        super().__init__(f"{fn}: {WQ_STATUS.get(status, status)}: {detail}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libwq.so not found at {LIB_PATH}; build it first with "
            "`python -m weight_only_quantized_wq_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.wq_decode_step_workspace_bytes.argtypes = [ctypes.c_int32]
    lib.wq_decode_step_workspace_bytes.restype = ctypes.c_int64
    lib.wq_decode_step_prepare.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(wq_matrix), ctypes.c_int32,
                                           _P, _I64, ctypes.POINTER(wq_step_plan)]
    lib.wq_decode_step_prepare.restype = ctypes.c_int
    lib.wq_decode_step_run.argtypes = [ctypes.POINTER(wq_step_plan), _P]
    lib.wq_decode_step_run.restype = ctypes.c_int
    lib.wq_moe_step_workspace_bytes.argtypes = [ctypes.c_int32]
    lib.wq_moe_step_workspace_bytes.restype = ctypes.c_int64
    lib.wq_moe_step_prepare.argtypes = [_I64, _I64, _I64, ctypes.POINTER(wq_moe_layer), ctypes.c_int32, _P, _I64,
                                        ctypes.POINTER(wq_moe_plan)]
    lib.wq_moe_step_prepare.restype = ctypes.c_int
    lib.wq_moe_step_run.argtypes = [ctypes.POINTER(wq_moe_plan), _P]
    lib.wq_moe_step_run.restype = ctypes.c_int
    lib.wq_status_string.argtypes = [ctypes.c_int]
    lib.wq_status_string.restype = ctypes.c_char_p
    lib.wq_last_error.argtypes = []
    lib.wq_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def _ptr(t):
    """Device address of a tensor (or None / int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not getattr(t, "is_cuda", False):
        raise ValueError("libwq buffers must be GPU tensors (device memory)")
    if not t.is_contiguous():
        raise ValueError("libwq buffers must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, *args):
    rc = getattr(lib, name)(*args)
    if rc != 0:
        raise WQError(name, rc, lib.wq_last_error().decode(errors="replace"))


def status_string(status):
    return lib.wq_status_string(int(status)).decode()


def last_error():
    return lib.wq_last_error().decode(errors="replace")


def wq_quantize_int8(w, n, k, q, scale, stream=None):
    _call("wq_quantize_int8", _ptr(w), n, k, _ptr(q), _ptr(scale), _stream(stream))


def wq_quantize_int4g32(w, n, k, qpacked, sz, stream=None):
    _call("wq_quantize_int4g32", _ptr(w), n, k, _ptr(qpacked), _ptr(sz), _stream(stream))


def wq_quantize_int4(w, n, k, group, qpacked, sz, stream=None):
    _call("wq_quantize_int4", _ptr(w), n, k, group, _ptr(qpacked), _ptr(sz), _stream(stream))


def wq_gemv_bf16(x, w, n, k, y_f32=None, y_bf16=None, stream=None):
    _call("wq_gemv_bf16", _ptr(x), _ptr(w), n, k, _ptr(y_f32), _ptr(y_bf16), _stream(stream))


def wq_gemv_int8(x, q, scale, n, k, y_f32=None, y_bf16=None, stream=None):
    _call("wq_gemv_int8", _ptr(x), _ptr(q), _ptr(scale), n, k, _ptr(y_f32), _ptr(y_bf16), _stream(stream))


def wq_gemv_int4g32(x, qpacked, sz, n, k, y_f32=None, y_bf16=None, stream=None):
    _call("wq_gemv_int4g32", _ptr(x), _ptr(qpacked), _ptr(sz), n, k, _ptr(y_f32), _ptr(y_bf16),
          _stream(stream))


def wq_gemv_int4(x, qpacked, sz, n, k, group, y_f32=None, y_bf16=None, stream=None):
    _call("wq_gemv_int4", _ptr(x), _ptr(qpacked), _ptr(sz), n, k, group, _ptr(y_f32), _ptr(y_bf16),
          _stream(stream))


def wq_gemm_smallM(x, m, qpacked, sz, n, k, y_f32=None, y_bf16=None, stream=None):
    _call("wq_gemm_smallM", _ptr(x), m, _ptr(qpacked), _ptr(sz), n, k, _ptr(y_f32), _ptr(y_bf16),
          _stream(stream))


def wq_gemm_smallM_int4(x, m, qpacked, sz, n, k, group, y_f32=None, y_bf16=None, stream=None):
    """m token rows x [m, k] through int4 weights with groups of `group` inputs -> y [m, n]."""
    _call("wq_gemm_smallM_int4", _ptr(x), m, _ptr(qpacked), _ptr(sz), n, k, group, _ptr(y_f32), _ptr(y_bf16),
          _stream(stream))


def wq_gemm_smallM_int8(x, m, q, scale, n, k, y_f32=None, y_bf16=None, stream=None):
    """m token rows x [m, k] through int8 per-row weights -> y [m, n]."""
    _call("wq_gemm_smallM_int8", _ptr(x), m, _ptr(q), _ptr(scale), n, k, _ptr(y_f32), _ptr(y_bf16),
          _stream(stream))


def moe_top2_gemv(x, logits, e, w13, s13, w2, s2, dim, f, work, y_f32=None, y_bf16=None, sel=None,
                  gates=None, stream=None):
    _call("moe_top2_gemv", _ptr(x), _ptr(logits), e, _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), dim, f,
          _ptr(work), _ptr(y_f32), _ptr(y_bf16), _ptr(sel), _ptr(gates), _stream(stream))


def wq_decode_step_workspace_bytes(count):
    return int(lib.wq_decode_step_workspace_bytes(count))


def wq_decode_step_prepare(format, m, mats, workspace, workspace_bytes=None):
    """mats: sequence of (x, w, aux, n, k, y_f32, y_bf16) with tensors (or None).
    `format` is a WQ_FORMAT code or name ("bf16", "int8", "int4g32", "int4g64",
    "int4g128", "int4g256", "int4pc": one group per row).  Returns the
    wq_step_plan."""
    fmt = WQ_FORMAT.get(format, format)
    arr = (wq_matrix * len(mats))()
    for i, (x, w, aux, n, k, y32, y16) in enumerate(mats):
        arr[i] = wq_matrix(_ptr(x), _ptr(w), _ptr(aux), n, k, _ptr(y32), _ptr(y16))
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    plan = wq_step_plan()
    rc = lib.wq_decode_step_prepare(fmt, m, arr, len(mats), _ptr(workspace), workspace_bytes, ctypes.byref(plan))
    if rc != 0:
        raise WQError("wq_decode_step_prepare", rc, lib.wq_last_error().decode(errors="replace"))
    return plan


def wq_decode_step_run(plan, stream=None):
    rc = lib.wq_decode_step_run(ctypes.byref(plan), _stream(stream))
    if rc != 0:
        raise WQError("wq_decode_step_run", rc, lib.wq_last_error().decode(errors="replace"))


def wq_moe_step_workspace_bytes(count):
    return int(lib.wq_moe_step_workspace_bytes(count))


def wq_moe_step_prepare(e, dim, f, layers, workspace, workspace_bytes=None):
    """layers: sequence of (x, logits, w13, s13, w2, s2, work, y_f32, y_bf16, sel, gates) with tensors (or
    None).  Returns the wq_moe_plan."""
    arr = (wq_moe_layer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = wq_moe_layer(*[_ptr(t) for t in L])
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    plan = wq_moe_plan()
    rc = lib.wq_moe_step_prepare(e, dim, f, arr, len(layers), _ptr(workspace), workspace_bytes, ctypes.byref(plan))
    if rc != 0:
        raise WQError("wq_moe_step_prepare", rc, lib.wq_last_error().decode(errors="replace"))
    return plan


def wq_moe_step_run(plan, stream=None):
    rc = lib.wq_moe_step_run(ctypes.byref(plan), _stream(stream))
    if rc != 0:
        raise WQError("wq_moe_step_run", rc, lib.wq_last_error().decode(errors="replace"))
