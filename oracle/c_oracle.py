"""ctypes wrapper around the plain C oracle (exact_oracle.c).

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's cpu_baseline leg.  Same definition as ``oracle.exact`` (det-train
page, "Method" section), written independently in C for large shapes.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB, build

NUM_DIGITS = 18
_ERRORS = {-1: "K exceeds 2^19", -2: "non-finite input", -3: "product outside the digit range",
           -4: "digit sum overflows int64", -5: "invalid argument", -6: "out of memory"}
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        c_long, c_int, vp = ctypes.c_long, ctypes.c_int, ctypes.c_void_p
        lib.oracle_partial_full.argtypes = [c_int, vp, c_long, vp, c_long, c_long, c_long, c_long,
                                            vp, c_int]
        lib.oracle_partial_pairs.argtypes = [c_int, vp, c_long, vp, c_long, c_long, vp, vp, c_long,
                                             vp, c_int]
        lib.oracle_finalize.argtypes = [vp, c_long, vp]
        lib.oracle_finalize.restype = None
        lib.oracle_combine.argtypes = [vp, c_int, c_long, vp]
        _lib = lib
    return _lib


def _check(rc: int) -> None:
    if rc != 0:
        raise ValueError(f"C oracle: {_ERRORS.get(rc, rc)}")


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise ValueError("operands must be uint32 (f32 bits) or uint16 (bf16 bits)")


def _threads(n):
    return n if n else (os.cpu_count() or 1)


def partial(x_bits: np.ndarray, w_bits: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Raw digits [M, N, 18] of x [M, K] against w [N, K]."""
    x = np.ascontiguousarray(x_bits)
    w = np.ascontiguousarray(w_bits)
    if x.dtype != w.dtype or x.shape[1] != w.shape[1]:
        raise ValueError("x and w must share dtype and K")
    M, K = x.shape
    N = w.shape[0]
    out = np.empty((M, N, NUM_DIGITS), dtype=np.int64)
    _check(load().oracle_partial_full(_dt(x), x.ctypes.data, K, w.ctypes.data, K, M, N, K,
                                      out.ctypes.data, _threads(nthreads)))
    return out


def partial_pairs(x_bits: np.ndarray, w_bits: np.ndarray, rows, cols,
                  nthreads: int = 0) -> np.ndarray:
    """Raw digits [P, 18] of the outputs (rows[p], cols[p])."""
    x = np.ascontiguousarray(x_bits)
    w = np.ascontiguousarray(w_bits)
    if x.dtype != w.dtype or x.shape[1] != w.shape[1]:
        raise ValueError("x and w must share dtype and K")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D of equal length")
    if rows.size and (rows.min() < 0 or rows.max() >= x.shape[0] or cols.min() < 0
                      or cols.max() >= w.shape[0]):
        raise ValueError("output index out of range")
    K = x.shape[1]
    out = np.empty((rows.size, NUM_DIGITS), dtype=np.int64)
    _check(load().oracle_partial_pairs(_dt(x), x.ctypes.data, K, w.ctypes.data, K, K,
                                       rows.ctypes.data, cols.ctypes.data, rows.size,
                                       out.ctypes.data, _threads(nthreads)))
    return out


def finalize(digits: np.ndarray) -> np.ndarray:
    """fp32 bit patterns (uint32) of digit arrays [..., 18]."""
    d = np.ascontiguousarray(digits, dtype=np.int64)
    if d.shape[-1:] != (NUM_DIGITS,):
        raise ValueError("digit arrays must end in a dimension of 18")
    out = np.empty(d.shape[:-1], dtype=np.uint32)
    load().oracle_finalize(d.ctypes.data, d.size // NUM_DIGITS, out.ctypes.data)
    return out


def combine(parts) -> np.ndarray:
    """Digit-wise int64 sum with an overflow check."""
    if len(parts) == 0:
        raise ValueError("combine needs at least one digit array")
    arrs = [np.ascontiguousarray(p, dtype=np.int64) for p in parts]
    for a in arrs:
        if a.shape != arrs[0].shape:
            raise ValueError("digit arrays must have equal shapes")
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    out = np.empty_like(arrs[0])
    _check(load().oracle_combine(ptrs, len(arrs), out.size, out.ctypes.data))
    return out


def gemm(x_bits: np.ndarray, w_bits: np.ndarray, nthreads: int = 0) -> np.ndarray:
    return finalize(partial(x_bits, w_bits, nthreads))


def gemm_pairs(x_bits, w_bits, rows, cols, nthreads: int = 0) -> np.ndarray:
    return finalize(partial_pairs(x_bits, w_bits, rows, cols, nthreads))
