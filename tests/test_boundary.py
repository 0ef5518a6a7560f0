"""The C-ABI library on the CPU: it loads, exports every entry point that
include/detgemm.h declares, and rejects bad arguments before touching a GPU.
No compute call runs here."""
import ctypes
import os
import re

import pytest
import torch

from bitwise_deterministic_exact_amd import _lib
import bitwise_deterministic_exact_amd as det

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "detgemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(det_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_pages_entry_points():
    names = declared_functions()
    for want in ("det_gemm", "det_gemm_partial", "det_combine", "det_finalize"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} missing from libdetgemm.so"


def test_layout_constants():
    lib = _lib.load()
    assert lib.det_num_digits() == 18
    assert lib.det_lsb_exponent() == -298
    assert lib.det_k_max() == 1 << 19


def _call_gemm(dt=0, x=1 << 20, w=1 << 20, M=4, N=4, K=4, y=1 << 20, strides=(4, 1, 4, 1, 4, 1)):
    lib = _lib.load()
    xs, xk, ws, wk, ys, yn = strides
    return lib.det_gemm(dt, ctypes.c_void_p(x), xs, xk, ctypes.c_void_p(w), ws, wk, M, N, K,
                        ctypes.c_void_p(y), ys, yn, None)


def test_c_abi_rejects_bad_arguments_without_a_gpu():
    # every case fails in host-side validation, before any HIP call
    assert _call_gemm(K=(1 << 19) + 1) == _lib.DET_EKLIMIT
    assert "2^19" in _lib.last_error()
    assert _call_gemm(dt=7) == _lib.DET_EDTYPE
    assert _call_gemm(M=-1) == _lib.DET_EINVAL
    assert _call_gemm(x=0) == _lib.DET_EINVAL
    assert _call_gemm(y=0) == _lib.DET_EINVAL
    assert _call_gemm(strides=(4, -1, 4, 1, 4, 1)) == _lib.DET_EINVAL
    assert _call_gemm(x=(1 << 20) + 2) == _lib.DET_EINVAL          # misaligned f32
    lib = _lib.load()
    assert lib.det_gemm_partial(0, ctypes.c_void_p(1 << 20), 4, 1, ctypes.c_void_p(1 << 20), 4, 1,
                                4, 4, 4, None, None) == _lib.DET_EINVAL
    assert lib.det_combine(None, 0, None, 4, None) == _lib.DET_EINVAL
    ptrs = (ctypes.c_void_p * 1)(None)
    assert lib.det_combine(ptrs, 1, ctypes.c_void_p(1 << 20), 4, None) == _lib.DET_EINVAL
    # out may equal a part, but may not partly overlap one (n = 4 outputs = 576 bytes)
    base = 1 << 30
    ptrs = (ctypes.c_void_p * 2)(base, base + 8)
    assert lib.det_combine(ptrs, 2, ctypes.c_void_p(base), 4, None) == _lib.DET_EINVAL
    assert "overlaps" in _lib.last_error()
    ptrs = (ctypes.c_void_p * 2)(base - 576 + 8, base + 4096)
    assert lib.det_combine(ptrs, 2, ctypes.c_void_p(base), 4, None) == _lib.DET_EINVAL
    ptrs = (ctypes.c_void_p * 33)(*([base] * 33))
    assert lib.det_combine(ptrs, 33, ctypes.c_void_p(base), 4, None) == _lib.DET_EINVAL
    assert lib.det_finalize(None, None, 5, None) == _lib.DET_EINVAL
    assert lib.det_finalize(None, None, -1, None) == _lib.DET_EINVAL
    assert lib.det_round_f32_to_bf16(None, None, 3, None) == _lib.DET_EINVAL
    assert lib.det_check_finite(9, None, 1, 1, 1, 1, None, None) == _lib.DET_EDTYPE
    # exact dot products: 2^30 products per accumulator, 3 per squared difference
    v, acc = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)
    assert lib.det_dot_partial(0, v, 1, v, 1, (1 << 30) + 1, acc, 0, None) == _lib.DET_EKLIMIT
    assert lib.det_sqdiff_partial(0, v, 1, v, 1, (1 << 30) // 3 + 1, acc, 0, None) == _lib.DET_EKLIMIT
    assert lib.det_sqdiff_partial(0, v, 1, None, 0, (1 << 30) + 1, acc, 0, None) == _lib.DET_EKLIMIT
    assert lib.det_dot_partial(0, v, 1, v, 1, 8, None, 0, None) == _lib.DET_EINVAL
    assert lib.det_dot_partial(0, v, 1, v, 1, 8, ctypes.c_void_p((1 << 21) + 4), 0, None) == _lib.DET_EINVAL
    assert lib.det_dot_partial(0, v, -1, v, 1, 8, acc, 0, None) == _lib.DET_EINVAL
    assert lib.det_dot_partial(0, v, 1, None, 1, 8, acc, 0, None) == _lib.DET_EINVAL
    assert lib.det_dot_partial(0, ctypes.c_void_p((1 << 20) + 2), 1, v, 1, 8, acc, 0, None) == _lib.DET_EINVAL
    assert lib.det_dot_partial(5, v, 1, v, 1, 8, acc, 0, None) == _lib.DET_EDTYPE


def _ru(v, m):
    return (v + m - 1) // m * m


def _slice_room(M, N, K):
    """det_gemm_ws's room for the matrix-core path, as include/detgemm.h states it."""
    return (_ru(32 * (M + N) + 160, 256) + 7 * (_ru(M, 128) + _ru(N, 128)) * _ru(K, 128)
            + 1024 * (M + N) + 16 * min(1 << 22, 2 * M * N) + (16 * M * N if K > (1 << 14) else 0))


def test_workspace_size_and_checks():
    lib = _lib.load()
    assert lib.det_gemm_workspace_bytes(0, 0, 3, 0, 5) == 0
    assert lib.det_gemm_workspace_bytes(0, 0, 3, 5, 0) == 0
    assert lib.det_gemm_workspace_bytes(0, 0, 0, 5, 5) == 0
    # decoded w: 4-byte significand and exponent word per element (det_gemm),
    # 4 + 2 bytes (det_gemm_partial), rows padded to 64 and K to 16; decoded
    # x of one K block (at most 2^15): 8 bytes per element, rows padded to 2;
    # det_gemm also reserves the matrix-core path's digit arrays
    assert lib.det_gemm_workspace_bytes(0, 0, 1, 1, 1) == 8 * 64 * 16 + 8 * 2 * 16 + _slice_room(1, 1, 1)
    assert lib.det_gemm_workspace_bytes(1, 1, 9, 4096, 4096) == 6 * 4096 * 4096 + 8 * 10 * 4096
    assert (lib.det_gemm_workspace_bytes(0, 0, 9, 65, 17)
            == 8 * 128 * 32 + 8 * 10 * 32 + _slice_room(9, 65, 17))
    # det_gemm with K beyond one block also carries 144 bytes of digits per output
    assert (lib.det_gemm_workspace_bytes(0, 0, 7, 64, 40000)
            == 8 * 64 * 40000 + 8 * 8 * 32768 + 144 * 7 * 64 + _slice_room(7, 64, 40000))
    assert lib.det_gemm_workspace_bytes(0, 1, 7, 64, 40000) == 6 * 64 * 40000 + 8 * 8 * 32768
    vp = ctypes.c_void_p
    args = (0, vp(1 << 20), 4, 1, vp(1 << 20), 4, 1, 4, 4, 4, vp(1 << 20), 4, 1)
    need = lib.det_gemm_workspace_bytes(0, 0, 4, 4, 4)
    acc_need = need - _slice_room(4, 4, 4)              # the accumulator path alone
    assert lib.det_gemm_ws(*args, None, need, None) == _lib.DET_EINVAL
    assert lib.det_gemm_ws(*args, vp((1 << 20) + 8), need, None) == _lib.DET_EINVAL   # misaligned
    assert lib.det_gemm_ws(*args, vp(1 << 20), acc_need - 1, None) == _lib.DET_EINVAL  # too small
    assert "workspace" in _lib.last_error()
    # the matrix-core path, forced, needs its room too
    try:
        assert lib.det_set_gemm_path(_lib.DET_PATH_SLICES, 0) == _lib.DET_OK
        assert lib.det_gemm_ws(*args, vp(1 << 20), need - 1, None) == _lib.DET_EINVAL
        assert "matrix-core" in _lib.last_error()
    finally:
        assert lib.det_set_gemm_path(_lib.DET_PATH_AUTO, 0) == _lib.DET_OK


def test_gemm_path_settings():
    lib = _lib.load()
    assert lib.det_set_gemm_path(4, 0) == _lib.DET_EINVAL
    assert lib.det_set_gemm_path(-1, 0) == _lib.DET_EINVAL
    for bad in (1, 8, -1):
        assert lib.det_set_gemm_path(_lib.DET_PATH_SLICES, bad) == _lib.DET_EINVAL
    assert "slices" in _lib.last_error()
    for path in (_lib.DET_PATH_ACCUMULATOR, _lib.DET_PATH_SLICES, _lib.DET_PATH_AUTO, _lib.DET_PATH_AUTO_HOST):
        for S in (0, 2, 7):
            assert lib.det_set_gemm_path(path, S) == _lib.DET_OK
    lib.det_set_gemm_path(_lib.DET_PATH_AUTO, 0)
    lib.det_last_gemm_plan(None, None, None, None)       # null pointers are skipped
    with pytest.raises(ValueError):
        det.set_gemm_path("fast")
    with pytest.raises(ValueError):
        det.set_gemm_path("slices", 9)
    # contexts restore the setting that was in force before them, and nest
    assert det.get_gemm_path() == ("auto", 0)
    det.set_gemm_path("slices", 5)
    with det.gemm_path("accumulator"):
        assert det.get_gemm_path() == ("accumulator", 0)
        with det.gemm_path("auto_host"):
            assert det.get_gemm_path() == ("auto_host", 0)
        with det.gemm_path("slices", 3):
            assert det.get_gemm_path() == ("slices", 3)
        assert det.get_gemm_path() == ("accumulator", 0)
    assert det.get_gemm_path() == ("slices", 5)
    with pytest.raises(KeyError):
        with det.gemm_path("auto"):
            raise KeyError("restored on an exception too")
    assert det.get_gemm_path() == ("slices", 5)
    det.set_gemm_path("auto")
    assert det.get_gemm_path() == ("auto", 0)
    plan = det.last_gemm_plan()
    assert set(plan) == {"path", "slices", "fallback_rows", "fallback_cols"}


def test_c_abi_empty_problems_are_no_ops():
    # nothing to do: no launch, status OK even with null pointers
    lib = _lib.load()
    assert _call_gemm(M=0, x=0, y=0) == _lib.DET_OK
    assert _call_gemm(N=0, w=0, y=0) == _lib.DET_OK
    assert lib.det_finalize(None, None, 0, None) == _lib.DET_OK
    assert lib.det_round_f32_to_bf16(None, None, 0, None) == _lib.DET_OK


def test_python_layer_validates_before_launch():
    meta = dict(device="meta")
    x = torch.empty(3, (1 << 19) + 1, dtype=torch.float32, **meta)
    with pytest.raises(ValueError, match="2\\^19"):
        det.det_gemm(x, x)
    with pytest.raises(ValueError, match="K mismatch"):
        det.det_gemm(torch.empty(3, 4, **meta), torch.empty(3, 5, **meta))
    with pytest.raises(ValueError, match="float32"):
        det.det_gemm(torch.empty(3, 4, dtype=torch.float16, **meta),
                     torch.empty(3, 4, dtype=torch.float16, **meta))
    with pytest.raises(ValueError, match="float32"):
        det.det_gemm(torch.empty(3, 4, dtype=torch.float32, **meta),
                     torch.empty(3, 4, dtype=torch.bfloat16, **meta))
    with pytest.raises(ValueError):
        det.det_gemm(torch.empty(3, 4), torch.empty(3, 4))          # CPU tensors
    with pytest.raises(ValueError):
        det.det_combine([])
    with pytest.raises(ValueError):
        det.det_finalize(torch.empty(3, 17, dtype=torch.int64))
    with pytest.raises(ValueError):
        det.DetLinear(4, 4, k_shards=0)
    # K-slice composition: up to 2^30, operands checked before any launch
    with pytest.raises(ValueError, match="2\\^30"):
        det.gemm_any_k(torch.empty(1, (1 << 30) + 1, **meta), torch.empty(1, (1 << 30) + 1, **meta))
    with pytest.raises(ValueError, match="K mismatch"):
        det.gemm_any_k(torch.empty(1, (1 << 19) + 5, **meta), torch.empty(1, (1 << 19) + 4, **meta))
    with pytest.raises(ValueError, match="same GPU"):
        det.gemm_any_k(torch.empty(2, (1 << 19) + 5, **meta), torch.empty(2, (1 << 19) + 5, **meta))
    with pytest.raises(ValueError, match="one shape"):
        det.exact_dot(torch.empty(3, **meta), torch.empty(4, **meta))
    with pytest.raises(ValueError, match="one shape"):
        det.exact_mse_loss(torch.empty(3, **meta), torch.empty(4, **meta))
    with pytest.raises(ValueError, match="float32 or bfloat16"):
        det.exact_mse_loss(torch.empty(3, dtype=torch.float16, **meta))


def test_detlinear_bias_parameter():
    layer = det.DetLinear(6, 5, bias=True)
    assert layer.bias.shape == (5,) and layer.bias.dtype == torch.float32
    assert "bias=True" in repr(layer)
    assert all(abs(v) <= 1.0 / 6 ** 0.5 for v in layer.bias.tolist())
    assert det.DetLinear(6, 5).bias is None
    assert "bias=False" in repr(det.DetLinear(6, 5))
    assert det.DetLinear(6, 5, bias=True, dtype=torch.bfloat16).bias.dtype == torch.bfloat16


def test_shard_bounds_cover_k_once():
    from bitwise_deterministic_exact_amd.linear import shard_bounds
    for k in (1, 3, 4, 7, 192, 4096):
        for s in (1, 2, 3, 4, 16):
            b = shard_bounds(k, s)
            assert b[0][0] == 0 and b[-1][1] == k
            assert all(lo < hi for lo, hi in b)
            assert all(b[i][1] == b[i + 1][0] for i in range(len(b) - 1))
            assert len(b) == min(s, k)


def test_no_cpu_fallback_in_the_product():
    # the product path never imports the oracle and has no CPU compute path
    pkg = os.path.join(ROOT, "bitwise_deterministic_exact_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "oracle" not in src.replace("oracle_", ""), fn
