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
    "moe_top2_gemv_noalloc": [_P, _P, _I64, _P, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _P],
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


class _HostBuffer:
    """Stand-in returned by _ptr for a tensor that is not in device memory;
    _call (and the plan builders) refuse it after every buffer's extent has
    been checked."""


def _ptr(t, nbytes=None, what="buffer"):
    """Device address of a tensor (or None / int passthrough).

    With `nbytes`, a tensor must hold at least that many bytes (the extent the
    C call will read or write for the sizes it is given); a shorter one raises
    ValueError before any call, since the kernels would access memory past
    it.  Raw integer addresses are passed through unchecked.  A tensor that is
    not on the GPU yields a _HostBuffer, which the call refuses once all
    arguments have been checked."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if nbytes is not None and nbytes > 0:
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise ValueError(f"libwq: {what} holds {have} bytes; the sizes given need {nbytes}")
    if not getattr(t, "is_cuda", False):
        return _HostBuffer()
    if not t.is_contiguous():
        raise ValueError(f"libwq: {what} must be contiguous")
    return t.data_ptr()


def _refuse_host(args):
    if any(isinstance(a, _HostBuffer) for a in args):
        raise ValueError("libwq buffers must be GPU tensors (device memory)")


def _nonneg(*v):
    """True when every size is a non-negative int (else the C call reports the error)."""
    return all(isinstance(a, int) and a >= 0 for a in v)


def _int4_sz_bytes(n, k, group):
    """Bytes of the (scale, zero) words of an int4 matrix with groups of `group` (0 if undefined)."""
    if not _nonneg(n, k, group) or group == 0 or k % group:
        return 0
    return n * (k // group) * 4


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, *args):
    _refuse_host(args)
    rc = getattr(lib, name)(*args)
    if rc != 0:
        raise WQError(name, rc, lib.wq_last_error().decode(errors="replace"))


def status_string(status):
    return lib.wq_status_string(int(status)).decode()


def last_error():
    return lib.wq_last_error().decode(errors="replace")


def wq_quantize_int8(w, n, k, q, scale, stream=None):
    ok = _nonneg(n, k)
    _call("wq_quantize_int8", _ptr(w, ok and 4 * n * k, "w"), n, k, _ptr(q, ok and n * k, "q"),
          _ptr(scale, ok and 2 * n, "scale"), _stream(stream))


def wq_quantize_int4g32(w, n, k, qpacked, sz, stream=None):
    ok = _nonneg(n, k)
    _call("wq_quantize_int4g32", _ptr(w, ok and 4 * n * k, "w"), n, k, _ptr(qpacked, ok and n * k // 2, "qpacked"),
          _ptr(sz, _int4_sz_bytes(n, k, 32), "sz"), _stream(stream))


def wq_quantize_int4(w, n, k, group, qpacked, sz, stream=None):
    ok = _nonneg(n, k)
    _call("wq_quantize_int4", _ptr(w, ok and 4 * n * k, "w"), n, k, group, _ptr(qpacked, ok and n * k // 2, "qpacked"),
          _ptr(sz, _int4_sz_bytes(n, k, group), "sz"), _stream(stream))


def wq_gemv_bf16(x, w, n, k, y_f32=None, y_bf16=None, stream=None):
    ok = _nonneg(n, k)
    _call("wq_gemv_bf16", _ptr(x, ok and 2 * k, "x"), _ptr(w, ok and 2 * n * k, "w"), n, k,
          _ptr(y_f32, ok and 4 * n, "y_f32"), _ptr(y_bf16, ok and 2 * n, "y_bf16"), _stream(stream))


def wq_gemv_int8(x, q, scale, n, k, y_f32=None, y_bf16=None, stream=None):
    ok = _nonneg(n, k)
    _call("wq_gemv_int8", _ptr(x, ok and 2 * k, "x"), _ptr(q, ok and n * k, "q"), _ptr(scale, ok and 2 * n, "scale"),
          n, k, _ptr(y_f32, ok and 4 * n, "y_f32"), _ptr(y_bf16, ok and 2 * n, "y_bf16"), _stream(stream))


def wq_gemv_int4g32(x, qpacked, sz, n, k, y_f32=None, y_bf16=None, stream=None):
    ok = _nonneg(n, k)
    _call("wq_gemv_int4g32", _ptr(x, ok and 2 * k, "x"), _ptr(qpacked, ok and n * k // 2, "qpacked"),
          _ptr(sz, _int4_sz_bytes(n, k, 32), "sz"), n, k, _ptr(y_f32, ok and 4 * n, "y_f32"),
          _ptr(y_bf16, ok and 2 * n, "y_bf16"), _stream(stream))


def wq_gemv_int4(x, qpacked, sz, n, k, group, y_f32=None, y_bf16=None, stream=None):
    ok = _nonneg(n, k)
    _call("wq_gemv_int4", _ptr(x, ok and 2 * k, "x"), _ptr(qpacked, ok and n * k // 2, "qpacked"),
          _ptr(sz, _int4_sz_bytes(n, k, group), "sz"), n, k, group, _ptr(y_f32, ok and 4 * n, "y_f32"),
          _ptr(y_bf16, ok and 2 * n, "y_bf16"), _stream(stream))


def wq_gemm_smallM(x, m, qpacked, sz, n, k, y_f32=None, y_bf16=None, stream=None):
    ok = _nonneg(m, n, k)
    _call("wq_gemm_smallM", _ptr(x, ok and 2 * m * k, "x"), m, _ptr(qpacked, ok and n * k // 2, "qpacked"),
          _ptr(sz, _int4_sz_bytes(n, k, 32), "sz"), n, k, _ptr(y_f32, ok and 4 * m * n, "y_f32"),
          _ptr(y_bf16, ok and 2 * m * n, "y_bf16"), _stream(stream))


def wq_gemm_smallM_int4(x, m, qpacked, sz, n, k, group, y_f32=None, y_bf16=None, stream=None):
    """m token rows x [m, k] through int4 weights with groups of `group` inputs -> y [m, n]."""
    ok = _nonneg(m, n, k)
    _call("wq_gemm_smallM_int4", _ptr(x, ok and 2 * m * k, "x"), m, _ptr(qpacked, ok and n * k // 2, "qpacked"),
          _ptr(sz, _int4_sz_bytes(n, k, group), "sz"), n, k, group, _ptr(y_f32, ok and 4 * m * n, "y_f32"),
          _ptr(y_bf16, ok and 2 * m * n, "y_bf16"), _stream(stream))


def wq_gemm_smallM_int8(x, m, q, scale, n, k, y_f32=None, y_bf16=None, stream=None):
    """m token rows x [m, k] through int8 per-row weights -> y [m, n]."""
    ok = _nonneg(m, n, k)
    _call("wq_gemm_smallM_int8", _ptr(x, ok and 2 * m * k, "x"), m, _ptr(q, ok and n * k, "q"),
          _ptr(scale, ok and 2 * n, "scale"), n, k, _ptr(y_f32, ok and 4 * m * n, "y_f32"),
          _ptr(y_bf16, ok and 2 * m * n, "y_bf16"), _stream(stream))


def _moe_bytes(e, dim, f):
    """Extent of each buffer of one MoE layer (zeros when the sizes are invalid: the C call reports them)."""
    if not _nonneg(e, dim, f):
        e = dim = f = 0
    return {"x": 2 * dim, "logits": 4 * e, "w13": e * 2 * f * dim, "s13": e * 2 * f * 2, "w2": e * dim * f,
            "s2": e * dim * 2, "work": 8 * f, "y_f32": 4 * dim, "y_bf16": 2 * dim, "sel": 8, "gates": 8}


def moe_top2_gemv(x, logits, e, w13, s13, w2, s2, dim, f, work, y_f32=None, y_bf16=None, sel=None,
                  gates=None, stream=None):
    b = _moe_bytes(e, dim, f)
    _call("moe_top2_gemv", _ptr(x, b["x"], "x"), _ptr(logits, b["logits"], "logits"), e, _ptr(w13, b["w13"], "w13"),
          _ptr(s13, b["s13"], "s13"), _ptr(w2, b["w2"], "w2"), _ptr(s2, b["s2"], "s2"), dim, f,
          _ptr(work, b["work"], "work"), _ptr(y_f32, b["y_f32"], "y_f32"), _ptr(y_bf16, b["y_bf16"], "y_bf16"),
          _ptr(sel, b["sel"], "sel"), _ptr(gates, b["gates"], "gates"), _stream(stream))


def moe_top2_gemv_noalloc(x, logits, e, w13, s13, w2, s2, dim, f, y_f32=None, y_bf16=None, sel=None,
                          gates=None, stream=None):
    """moe_top2_gemv with the SwiGLU intermediate in the library's static device scratch (f <= 16384)."""
    b = _moe_bytes(e, dim, f)
    _call("moe_top2_gemv_noalloc", _ptr(x, b["x"], "x"), _ptr(logits, b["logits"], "logits"), e,
          _ptr(w13, b["w13"], "w13"), _ptr(s13, b["s13"], "s13"), _ptr(w2, b["w2"], "w2"), _ptr(s2, b["s2"], "s2"),
          dim, f, _ptr(y_f32, b["y_f32"], "y_f32"), _ptr(y_bf16, b["y_bf16"], "y_bf16"), _ptr(sel, b["sel"], "sel"),
          _ptr(gates, b["gates"], "gates"), _stream(stream))


def wq_decode_step_workspace_bytes(count):
    return int(lib.wq_decode_step_workspace_bytes(count))


def wq_decode_step_prepare(format, m, mats, workspace, workspace_bytes=None):
    """mats: sequence of (x, w, aux, n, k, y_f32, y_bf16) with tensors (or None).
    `format` is a WQ_FORMAT code or name ("bf16", "int8", "int4g32", "int4g64",
    "int4g128", "int4g256", "int4pc": one group per row).  Returns the
    wq_step_plan."""
    fmt = WQ_FORMAT.get(format, format)
    name = {v: k for k, v in WQ_FORMAT.items()}.get(fmt)
    ptrs = []
    for i, (x, w, aux, n, k, y32, y16) in enumerate(mats):
        ok = name is not None and _nonneg(m, n, k)
        if ok and name == "bf16":
            wb, ab = 2 * n * k, 0
        elif ok and name == "int8":
            wb, ab = n * k, 2 * n
        elif ok:
            wb, ab = n * k // 2, _int4_sz_bytes(n, k, k if name == "int4pc" else int(name[5:]))
        else:
            wb = ab = 0
        ptrs.append((_ptr(x, ok and 2 * m * k, f"matrix {i} x"), _ptr(w, wb, f"matrix {i} w"),
                     _ptr(aux, ab, f"matrix {i} aux"), n, k, _ptr(y32, ok and 4 * m * n, f"matrix {i} y_f32"),
                     _ptr(y16, ok and 2 * m * n, f"matrix {i} y_bf16")))
    _refuse_host([a for p in ptrs for a in p] + [_ptr(workspace)])
    arr = (wq_matrix * len(mats))()
    for i, p in enumerate(ptrs):
        arr[i] = wq_matrix(*p)
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
    b = _moe_bytes(e, dim, f)
    keys = ("x", "logits", "w13", "s13", "w2", "s2", "work", "y_f32", "y_bf16", "sel", "gates")
    ptrs = [[_ptr(t, b[kk], f"layer {i} {kk}") for t, kk in zip(L, keys)] for i, L in enumerate(layers)]
    _refuse_host([a for p in ptrs for a in p] + [_ptr(workspace)])
    arr = (wq_moe_layer * len(layers))()
    for i, p in enumerate(ptrs):
        arr[i] = wq_moe_layer(*p)
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
