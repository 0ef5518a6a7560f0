"""Exact long-accumulator GEMM for AMD MI355X (gfx950).

The det-train operations (page "det-train", sections "Usage" and "Method"):
det_gemm, det_gemm_partial, det_combine, det_finalize and the DetLinear
module.  The kernels live in libdetgemm.so (C ABI: include/detgemm.h); this
package only marshals torch tensors into it.
"""
from ._lib import K_MAX, LSB_EXPONENT, NUM_DIGITS, DetGemmError  # noqa: F401
from .api import (det_combine, det_finalize, det_gemm, det_gemm_noalloc, det_gemm_partial,  # noqa: F401
                  exact_dot, exact_dot_digits, exact_sqdiff_digits, exact_sum_squares, gemm_any_k,
                  device_status, gemm_path, get_gemm_path, has_nonfinite, last_gemm_plan, round_f32_to_bf16,
                  set_gemm_path)
from .linear import DetLinear  # noqa: F401
from .loss import exact_mse_loss  # noqa: F401

__all__ = ["det_gemm", "det_gemm_noalloc", "det_gemm_partial", "det_combine", "det_finalize", "DetLinear",
           "round_f32_to_bf16", "has_nonfinite", "set_gemm_path", "last_gemm_plan", "gemm_path", "get_gemm_path",
           "device_status",
           "gemm_any_k", "exact_dot", "exact_dot_digits", "exact_sqdiff_digits", "exact_sum_squares",
           "exact_mse_loss",
           "NUM_DIGITS", "LSB_EXPONENT", "K_MAX", "DetGemmError"]
