"""ctypes binding of libdetgemm.so (the C ABI declared in include/detgemm.h).

Loading fails loudly when the library has not been built: there is no
fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdetgemm.so")

DET_OK, DET_EINVAL, DET_EKLIMIT, DET_EDTYPE, DET_ENONFINITE, DET_EHIP, DET_ERANGE = 0, 1, 2, 3, 4, 5, 6
DET_F32, DET_BF16 = 0, 1
DET_PATH_AUTO, DET_PATH_ACCUMULATOR, DET_PATH_SLICES, DET_PATH_AUTO_HOST = 0, 1, 2, 3
NUM_DIGITS = 18
LSB_EXPONENT = -298
K_MAX = 1 << 19

_lib = None


class DetGemmError(RuntimeError):
    """The HIP runtime reported an error inside the library."""


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(hipcc for gfx950).  There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, c_int = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int
    sigs = {
        "det_num_digits": ([], c_int),
        "det_lsb_exponent": ([], c_int),
        "det_k_max": ([], i64),
        "det_last_error": ([], ctypes.c_char_p),
        "det_gemm": ([c_int, vp, i64, i64, vp, i64, i64, i64, i64, i64, vp, i64, i64, vp], c_int),
        "det_gemm_partial": ([c_int, vp, i64, i64, vp, i64, i64, i64, i64, i64, vp, vp], c_int),
        "det_gemm_workspace_bytes": ([c_int, c_int, i64, i64, i64], i64),
        "det_gemm_ws": ([c_int, vp, i64, i64, vp, i64, i64, i64, i64, i64, vp, i64, i64, vp, ctypes.c_size_t,
                         vp], c_int),
        "det_gemm_noalloc": ([c_int, vp, i64, i64, vp, i64, i64, i64, i64, i64, vp, i64, i64, vp], c_int),
        "det_gemm_noalloc_max_bytes": ([], ctypes.c_size_t),
        "det_gemm_partial_ws": ([c_int, vp, i64, i64, vp, i64, i64, i64, i64, i64, vp, vp, ctypes.c_size_t, vp],
                                c_int),
        "det_combine": ([ctypes.POINTER(vp), c_int, vp, i64, vp], c_int),
        "det_finalize": ([vp, vp, i64, vp], c_int),
        "det_round_f32_to_bf16": ([vp, vp, i64, vp], c_int),
        "det_mse_grad": ([c_int, vp, vp, i64, ctypes.c_float, vp, vp, vp, vp], c_int),
        "det_check_finite": ([c_int, vp, i64, i64, i64, i64, vp, vp], c_int),
        "det_dot_partial": ([c_int, vp, i64, vp, i64, i64, vp, c_int, vp], c_int),
        "det_sqdiff_partial": ([c_int, vp, i64, vp, i64, i64, vp, c_int, vp], c_int),
        "det_set_gemm_path": ([c_int, c_int], c_int),
        "det_set_kernel_events": ([vp, vp], None),
        "det_device_status": ([vp, c_int, ctypes.POINTER(c_int)], c_int),
        "det_device_status_word": ([], vp),
        "det_get_gemm_path": ([ctypes.POINTER(c_int), ctypes.POINTER(c_int)], None),
        "det_last_gemm_plan": ([ctypes.POINTER(c_int), ctypes.POINTER(c_int), ctypes.POINTER(i64),
                                ctypes.POINTER(i64)], None),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if lib.det_num_digits() != NUM_DIGITS or lib.det_lsb_exponent() != LSB_EXPONENT:
        raise ImportError("libdetgemm.so layout constants do not match the binding")
    _lib = lib
    return lib


def last_error() -> str:
    return load().det_last_error().decode(errors="replace")


def check(status: int) -> None:
    """Map a det_status to a Python exception."""
    if status == DET_OK:
        return
    msg = last_error()
    if status == DET_EHIP:
        raise DetGemmError(msg)
    raise ValueError(msg)
