"""The det-train operations on torch tensors ("Usage" section of the det-train
page): det_gemm, det_gemm_partial, det_combine, det_finalize.

Argument marshalling only: every step runs in libdetgemm.so's HIP kernels on
the tensors' device, enqueued on the current torch stream.  torch provides the
device memory and the stream.

Shapes: x is [M, K], w is [N, K] (any strides, e.g. the K-slices x[:, a:b] or
transposed views), both float32 or both bfloat16, K <= 2^19.  det_gemm
returns float32 [M, N]; det_gemm_partial returns the raw long-accumulator
digits int64 [M, N, 18] (digit j weighs 2^(32j-298)).

Non-finite inputs are rejected with ValueError when ``check_finite`` is true;
its default comes from the environment variable DETGEMM_CHECK_FINITE ("1",
the default, or "0").  The check costs one small kernel and a device sync.
Unchecked calls still note an Inf or NaN operand (and combine and finalize a
digit outside +-2^62) in the GPU's sticky device status, read with
device_status().
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

from . import _lib

_DT = {torch.float32: _lib.DET_F32, torch.bfloat16: _lib.DET_BF16}


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _call(dev: torch.device, fn, *args) -> None:
    """One library call with the operands' device current (the library's
    launches, events and copies go to the calling thread's current device)."""
    with torch.cuda.device(dev):
        _lib.check(fn(*args))


def _want_check(flag: Optional[bool]) -> bool:
    if flag is not None:
        return bool(flag)
    return os.environ.get("DETGEMM_CHECK_FINITE", "1") != "0"


def _operands(x: torch.Tensor, w: torch.Tensor):
    if not isinstance(x, torch.Tensor) or not isinstance(w, torch.Tensor):
        raise TypeError("x and w must be tensors")
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x must be [M, K] and w must be [N, K]")
    if x.shape[1] != w.shape[1]:
        raise ValueError(f"K mismatch: x has {x.shape[1]}, w has {w.shape[1]}")
    if x.dtype != w.dtype or x.dtype not in _DT:
        raise ValueError(f"x and w must both be float32 or both bfloat16 (got {x.dtype}, {w.dtype})")
    if x.shape[1] > _lib.K_MAX:
        raise ValueError(f"K = {x.shape[1]} exceeds the limit 2^19 per call")
    if x.device.type != "cuda" or w.device != x.device:
        raise ValueError("x and w must be on the same GPU device")
    return _DT[x.dtype]


def has_nonfinite(t: torch.Tensor) -> bool:
    """True if a float32/bfloat16 tensor (<= 2-D, any strides) holds Inf or NaN."""
    if t.dtype not in _DT or t.device.type != "cuda":
        raise ValueError("has_nonfinite needs a float32/bfloat16 GPU tensor")
    t2 = t.reshape(1, -1) if t.dim() < 2 else t
    if t2.dim() != 2:
        t2 = t2.reshape(-1, t2.shape[-1])
    flag = torch.zeros(1, dtype=torch.int32, device=t.device)
    _call(t.device, _lib.load().det_check_finite,
          _DT[t.dtype], ctypes.c_void_p(t2.data_ptr()), t2.shape[0], t2.shape[1],
          t2.stride(0), t2.stride(1), ctypes.c_void_p(flag.data_ptr()), _stream(t.device))
    return bool(flag.item())


def _reject_nonfinite(x, w, check_finite):
    if _want_check(check_finite) and x.numel() and w.numel():
        if has_nonfinite(x) or has_nonfinite(w):
            raise ValueError("x or w holds Inf or NaN; the exact accumulator takes finite inputs only")


def _workspace(dt: int, partial: bool, M: int, N: int, K: int, device: torch.device, use: bool):
    """Scratch for the decoded copy of w, for long K the carried digits, and
    for det_gemm the digit arrays of the matrix-core path (torch's caching
    allocator provides it)."""
    nbytes = _lib.load().det_gemm_workspace_bytes(dt, int(partial), M, N, K) if use else 0
    if nbytes <= 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def det_gemm(x: torch.Tensor, w: torch.Tensor, *, check_finite: Optional[bool] = None,
             out: Optional[torch.Tensor] = None, workspace: bool = True) -> torch.Tensor:
    """y = x w^T with every product exact and one rounding to fp32.

    ``workspace=False`` decodes w inside the GEMM kernel instead of once up
    front; the result is bit-identical either way."""
    dt = _operands(x, w)
    _reject_nonfinite(x, w, check_finite)
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    elif out.shape != (M, N) or out.dtype != torch.float32 or out.device != x.device:
        raise ValueError("out must be float32 [M, N] on the operands' device")
    lib = _lib.load()
    ops = (dt, ctypes.c_void_p(x.data_ptr()), x.stride(0), x.stride(1),
           ctypes.c_void_p(w.data_ptr()), w.stride(0), w.stride(1), M, N, K,
           ctypes.c_void_p(out.data_ptr()), out.stride(0), out.stride(1))
    ws, nbytes = _workspace(dt, False, M, N, K, x.device, workspace)
    if ws is None:
        _call(x.device, lib.det_gemm, *ops, _stream(x.device))
    else:
        _call(x.device, lib.det_gemm_ws, *ops, ctypes.c_void_p(ws.data_ptr()), nbytes, _stream(x.device))
    return out


def det_gemm_noalloc(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """det_gemm into a caller-provided float32 [M, N] ``out``, allocating
    nothing: the library's static device scratch holds the decoded operands
    (C ABI det_gemm_noalloc; sizes up to its 64 MiB).  Bit-identical to
    det_gemm.  Inputs must be finite; an Inf or NaN is not checked for here
    (the check would allocate) but is noted in the device status (see
    device_status).  Calls that overlap in time on one GPU race."""
    dt = _operands(x, w)
    M, K = x.shape
    N = w.shape[0]
    if out.shape != (M, N) or out.dtype != torch.float32 or out.device != x.device:
        raise ValueError("out must be float32 [M, N] on the operands' device")
    lib = _lib.load()
    _call(x.device, lib.det_gemm_noalloc, dt, ctypes.c_void_p(x.data_ptr()), x.stride(0), x.stride(1),
          ctypes.c_void_p(w.data_ptr()), w.stride(0), w.stride(1), M, N, K,
          ctypes.c_void_p(out.data_ptr()), out.stride(0), out.stride(1), _stream(x.device))
    return out


def det_gemm_partial(x: torch.Tensor, w: torch.Tensor, *, check_finite: Optional[bool] = None,
                     workspace: bool = True) -> torch.Tensor:
    """Raw long-accumulator digits of x w^T: int64 [M, N, 18]."""
    dt = _operands(x, w)
    _reject_nonfinite(x, w, check_finite)
    M, K = x.shape
    N = w.shape[0]
    acc = torch.empty((M, N, _lib.NUM_DIGITS), dtype=torch.int64, device=x.device)
    lib = _lib.load()
    ops = (dt, ctypes.c_void_p(x.data_ptr()), x.stride(0), x.stride(1),
           ctypes.c_void_p(w.data_ptr()), w.stride(0), w.stride(1), M, N, K,
           ctypes.c_void_p(acc.data_ptr()))
    ws, nbytes = _workspace(dt, True, M, N, K, x.device, workspace)
    if ws is None:
        _call(x.device, lib.det_gemm_partial, *ops, _stream(x.device))
    else:
        _call(x.device, lib.det_gemm_partial_ws, *ops, ctypes.c_void_p(ws.data_ptr()), nbytes,
              _stream(x.device))
    return acc


def _check_acc(a: torch.Tensor, what: str) -> None:
    if a.dtype != torch.int64 or a.dim() < 1 or a.shape[-1] != _lib.NUM_DIGITS:
        raise ValueError(f"{what} must be int64 digit arrays [..., 18]")
    if a.device.type != "cuda":
        raise ValueError(f"{what} must be on a GPU")


def det_combine(parts: Sequence[torch.Tensor]) -> torch.Tensor:
    """Digit-wise int64 sum of accumulator arrays of equal shape."""
    parts = list(parts)
    if not parts:
        raise ValueError("det_combine needs at least one digit array")
    for p in parts:
        _check_acc(p, "det_combine inputs")
        if p.shape != parts[0].shape or p.device != parts[0].device:
            raise ValueError("det_combine inputs must share shape and device")
    parts = [p.contiguous() for p in parts]
    out = torch.empty_like(parts[0])
    ptrs = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    _call(out.device, _lib.load().det_combine, ptrs, len(parts), ctypes.c_void_p(out.data_ptr()),
          out.numel() // _lib.NUM_DIGITS, _stream(out.device))
    return out


def det_finalize(acc: torch.Tensor) -> torch.Tensor:
    """Round each accumulator once to fp32: [..., 18] int64 -> [...] float32."""
    _check_acc(acc, "det_finalize input")
    acc = acc.contiguous()
    y = torch.empty(acc.shape[:-1], dtype=torch.float32, device=acc.device)
    _call(acc.device, _lib.load().det_finalize, ctypes.c_void_p(acc.data_ptr()),
          ctypes.c_void_p(y.data_ptr()), y.numel(), _stream(acc.device))
    return y


K_ANY_MAX = 1 << 30


def gemm_any_k(x: torch.Tensor, w: torch.Tensor, *, check_finite: Optional[bool] = None) -> torch.Tensor:
    """det_gemm for any K: up to 2^19 one call; beyond, K-slices of at most
    2^19 as raw digits, added with det_combine and rounded once with
    det_finalize ("Usage": the partials of K-slices compose into the whole
    sum).  Bit-identical to one exact sum rounded once.  K up to 2^30, where
    the added digits still fit det_combine's int64 bound."""
    K = x.shape[1] if x.dim() == 2 else -1
    if K <= _lib.K_MAX:
        return det_gemm(x, w, check_finite=check_finite)
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError(f"K mismatch: x is {tuple(x.shape)}, w is {tuple(w.shape)}")
    if K > K_ANY_MAX:
        raise ValueError(f"K = {K} exceeds 2^30, the limit of composed K-slices")
    _operands(x[:, :1], w[:, :1])
    _reject_nonfinite(x, w, check_finite)
    parts = [det_gemm_partial(x[:, a:min(a + _lib.K_MAX, K)], w[:, a:min(a + _lib.K_MAX, K)],
                              check_finite=False)
             for a in range(0, K, _lib.K_MAX)]
    return det_finalize(det_combine(parts))


DOT_MAX_PRODUCTS = 1 << 30


def _vector(t: torch.Tensor, what: str):
    """A tensor as (tensor, element increment) for the dot entry points: a
    1-D view keeps its stride, anything else is flattened (a copy only when
    its elements are not evenly spaced)."""
    if t.dtype not in _DT:
        raise ValueError(f"{what} must be float32 or bfloat16 (got {t.dtype})")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be on a GPU")
    if t.dim() != 1:
        t = t.reshape(-1)
    return t, (t.stride(0) if t.numel() > 1 else 1)


def _dot_digits(fn, a: torch.Tensor, b: Optional[torch.Tensor], check_finite) -> torch.Tensor:
    va, ia = _vector(a, "a")
    vb, ib = _vector(b, "b") if b is not None else (None, 0)
    if vb is not None and vb.dtype != va.dtype:
        raise ValueError("a and b must share a dtype")
    if _want_check(check_finite) and va.numel():
        if has_nonfinite(va) or (vb is not None and has_nonfinite(vb)):
            raise ValueError("a or b holds Inf or NaN; the exact accumulator takes finite inputs only")
    acc = torch.empty(_lib.NUM_DIGITS, dtype=torch.int64, device=va.device)
    bp = ctypes.c_void_p(vb.data_ptr()) if vb is not None else None
    _call(va.device, fn, _DT[va.dtype], ctypes.c_void_p(va.data_ptr()), ia, bp, ib, va.numel(),
          ctypes.c_void_p(acc.data_ptr()), 0, _stream(va.device))
    return acc


def exact_dot_digits(a: torch.Tensor, b: torch.Tensor, *, check_finite: Optional[bool] = None) -> torch.Tensor:
    """Raw digits (int64 [18]) of sum_i a_i * b_i, every product exact: the
    digits det_gemm_partial gives for the 1 x 1 GEMM of the flattened
    operands, so they compose with det_combine and round with det_finalize."""
    if a.shape != b.shape:
        raise ValueError("exact_dot needs operands of one shape")
    if a.numel() > DOT_MAX_PRODUCTS:
        raise ValueError(f"{a.numel()} elements exceed 2^30 products per accumulator")
    return _dot_digits(_lib.load().det_dot_partial, a, b, check_finite)


def exact_dot(a: torch.Tensor, b: torch.Tensor, *, check_finite: Optional[bool] = None) -> torch.Tensor:
    """sum_i a_i * b_i over all elements, every product exact and the sum
    rounded once to fp32; a 0-d float32 tensor.  a and b: same shape, both
    float32 or both bfloat16, at most 2^30 elements."""
    return det_finalize(exact_dot_digits(a, b, check_finite=check_finite)).reshape(())


def exact_sqdiff_digits(a: torch.Tensor, b: Optional[torch.Tensor] = None, *,
                        check_finite: Optional[bool] = None) -> torch.Tensor:
    """Raw digits (int64 [18]) of sum_i (a_i - b_i)^2 with no rounding of the
    differences (sum_i a_i^2 without b)."""
    if b is not None and a.shape != b.shape:
        raise ValueError("a and b must have one shape")
    if a.numel() > DOT_MAX_PRODUCTS // (3 if b is not None else 1):
        raise ValueError(f"{a.numel()} elements exceed 2^30 products per accumulator")
    return _dot_digits(_lib.load().det_sqdiff_partial, a, b, check_finite)


def exact_sum_squares(y: torch.Tensor, *, check_finite: Optional[bool] = None) -> torch.Tensor:
    """sum_i y_i^2 exactly, rounded once to fp32; a 0-d float32 tensor."""
    return det_finalize(exact_sqdiff_digits(y, check_finite=check_finite)).reshape(())


_PATHS = {"auto": _lib.DET_PATH_AUTO, "accumulator": _lib.DET_PATH_ACCUMULATOR,
          "slices": _lib.DET_PATH_SLICES, "auto_host": _lib.DET_PATH_AUTO_HOST}
_PATH_NAMES = {v: k for k, v in _PATHS.items()}


def set_gemm_path(path: str = "auto", slices: int = 0) -> None:
    """Choose how det_gemm forms the exact sum (process-wide; see
    det_set_gemm_path in include/detgemm.h): "auto" (default: the device
    picks, the host never waits), "auto_host" (the host waits for the span
    histogram and picks), "accumulator" (the digit accumulator always) or
    "slices" (int8 digit GEMMs on the matrix cores, with `slices` = 2..7
    digits per operand or 0 to let the call choose).  Every path gives the
    same bits."""
    if path not in _PATHS:
        raise ValueError(f"path must be one of {sorted(_PATHS)}")
    _lib.check(_lib.load().det_set_gemm_path(_PATHS[path], int(slices)))


def last_gemm_plan() -> dict:
    """What this thread's last det_gemm call did: the path, the digits per
    operand (0 on the accumulator path) and how many rows of x and of w the
    matrix-core pass listed (rows that span more than S digits).  Waits for
    that call's plan when the device made it."""
    path, slices = ctypes.c_int(), ctypes.c_int()
    rows, cols = ctypes.c_int64(), ctypes.c_int64()
    _lib.load().det_last_gemm_plan(ctypes.byref(path), ctypes.byref(slices), ctypes.byref(rows),
                                   ctypes.byref(cols))
    return {"path": _PATH_NAMES.get(path.value, str(path.value)), "slices": slices.value,
            "fallback_rows": rows.value, "fallback_cols": cols.value}


def get_gemm_path() -> tuple:
    """The current process-wide (path, slices) setting of set_gemm_path."""
    path, slices = ctypes.c_int(), ctypes.c_int()
    _lib.load().det_get_gemm_path(ctypes.byref(path), ctypes.byref(slices))
    return _PATH_NAMES.get(path.value, "auto"), slices.value


class gemm_path:
    """Context manager: set_gemm_path(path, slices) inside; the setting that
    was in force before is restored on exit (contexts nest)."""

    def __init__(self, path: str, slices: int = 0):
        self.path, self.slices = path, slices
        self._saved = []

    def __enter__(self):
        self._saved.append(get_gemm_path())
        set_gemm_path(self.path, self.slices)
        return self

    def __exit__(self, *exc):
        path, slices = self._saved.pop()
        set_gemm_path(path, slices)
        return False


def device_status(device=None, clear: bool = True) -> set:
    """The sticky device status of `device` (default: the current one) after
    the work enqueued so far on its current stream: a set holding
    "nonfinite" (an operand held Inf or NaN) and/or "range" (a digit outside
    +-2^62 reached combine or finalize).  Waits for the stream; with `clear`
    the status is reset after it is read (det_device_status)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    flags = ctypes.c_int()
    with torch.cuda.device(dev):
        st = _lib.load().det_device_status(_stream(dev), int(bool(clear)), ctypes.byref(flags))
    if st not in (_lib.DET_OK, _lib.DET_ENONFINITE, _lib.DET_ERANGE):
        _lib.check(st)
    return {name for bit, name in ((1, "nonfinite"), (2, "range")) if flags.value & bit}


def mse_grad(y: torch.Tensor, t: Optional[torch.Tensor], g: torch.Tensor, need_dy: bool = True,
             need_dt: bool = False):
    """(dy, dt) of the exact mean squared error sum((y - t)^2) / n with
    incoming gradient g (a one-element tensor): dy = RNE_dtype(RNE32(RNE32(y -
    t) * c) * g), c = 2/n rounded to fp32, dt = -dy before the dtype rounding
    (det_mse_grad).  Either is None when not needed."""
    import numpy as np
    if y.dtype not in _DT or y.device.type != "cuda":
        raise ValueError("mse_grad takes float32 or bfloat16 GPU tensors")
    if t is not None and (t.shape != y.shape or t.dtype != y.dtype or t.device != y.device):
        raise ValueError("y and t must share shape, dtype and device")
    n = y.numel()
    c = float(np.float32(2.0) / np.float32(max(n, 1)))         # one IEEE fp32 division
    yc = y.contiguous()
    tc = t.contiguous() if t is not None else None
    gv = g.reshape(-1)[:1].to(device=y.device, dtype=torch.float32).contiguous()
    dy = torch.empty_like(yc) if need_dy else None
    dt = torch.empty_like(yc) if need_dt else None
    ptr = lambda v: ctypes.c_void_p(v.data_ptr()) if v is not None else None      # noqa: E731
    _call(y.device, _lib.load().det_mse_grad, _DT[y.dtype], ptr(yc), ptr(tc), n, c, ptr(gv), ptr(dy), ptr(dt),
          _stream(y.device))
    return (dy.reshape(y.shape) if dy is not None else None, dt.reshape(y.shape) if dt is not None else None)


def round_f32_to_bf16(t: torch.Tensor) -> torch.Tensor:
    """Round float32 to bfloat16, nearest with ties to even (HIP kernel)."""
    if t.dtype != torch.float32 or t.device.type != "cuda":
        raise ValueError("round_f32_to_bf16 needs a float32 GPU tensor")
    t = t.contiguous()
    out = torch.empty(t.shape, dtype=torch.bfloat16, device=t.device)
    _call(t.device, _lib.load().det_round_f32_to_bf16, ctypes.c_void_p(t.data_ptr()),
          ctypes.c_void_p(out.data_ptr()), t.numel(), _stream(t.device))
    return out
