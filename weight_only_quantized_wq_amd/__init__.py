"""Weight-only quantized decode matvecs for AMD MI355X (gfx950).

The compute lives in libwq.so (hand-written HIP kernels behind a C ABI,
include/wq.h); this package is its thin Python binding.  The library is
loaded on first use of any binding name and the load fails loudly if it has
not been built (``python -m weight_only_quantized_wq_amd.build``); the build
module itself imports without it.
"""

_EXPORTS = (
    "LIB_PATH", "WQError", "WQ_STATUS", "lib", "status_string", "last_error",
    "wq_quantize_int8", "wq_quantize_int4g32", "wq_quantize_int4",
    "wq_gemv_bf16", "wq_gemv_int8", "wq_gemv_int4g32", "wq_gemv_int4", "wq_gemm_smallM", "wq_gemm_smallM_int4", "wq_gemm_smallM_int8",
    "moe_top2_gemv", "moe_top2_gemv_noalloc",
    "WQ_FORMAT", "wq_matrix", "wq_step_plan",
    "wq_decode_step_workspace_bytes", "wq_decode_step_prepare", "wq_decode_step_run",
    "wq_moe_layer", "wq_moe_plan", "wq_moe_step_workspace_bytes", "wq_moe_step_prepare", "wq_moe_step_run",
)

__all__ = list(_EXPORTS)


def __getattr__(name):
    if name in _EXPORTS:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
