"""The device status of the C ABI: Inf and NaN operands, and digits outside
+-2^62, are noted by the kernels of every entry point that reads them and
reported by det_device_status (DET_ENONFINITE, DET_ERANGE); finite operands
and digits in range leave it clear.  The inputs are in-bounds for every
kernel (the digit grids cover the exponent field's all-ones value); the
results of a flagged call are unspecified and not compared."""
import ctypes

import pytest
import torch

import bitwise_deterministic_exact_amd as det
from bitwise_deterministic_exact_amd import _lib
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

BAD = (float("inf"), float("-inf"), float("nan"))


def _status():
    return det.device_status(clear=True)


def _operands(dt, M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(dt).cuda()
    w = torch.randn(N, K, generator=g).to(dt).cuda()
    return x, w


def _entry_points(x, w):
    """every GEMM-shaped entry point, unchecked (check_finite=False)"""
    M, N = x.shape[0], w.shape[0]
    return {
        "det_gemm_ws accumulator": lambda: det.det_gemm(x, w, check_finite=False),
        "det_gemm (no workspace)": lambda: det.det_gemm(x, w, check_finite=False, workspace=False),
        "det_gemm_partial_ws": lambda: det.det_gemm_partial(x, w, check_finite=False),
        "det_gemm_partial (no workspace)": lambda: det.det_gemm_partial(x, w, check_finite=False, workspace=False),
        "det_gemm_noalloc": lambda: det.det_gemm_noalloc(x, w, torch.empty(M, N, device="cuda")),
        "det_gemm_ws matrix-core S=3": lambda: _sliced(x, w, 3),
        "det_gemm_ws matrix-core S=7": lambda: _sliced(x, w, 7),
        "det_dot_partial": lambda: det.exact_dot_digits(x.reshape(-1), x.reshape(-1).flip(0), check_finite=False),
        "det_sqdiff_partial": lambda: det.exact_sqdiff_digits(x.reshape(-1), x.reshape(-1).flip(0),
                                                              check_finite=False),
    }


def _sliced(x, w, S):
    with det.gemm_path("slices", S):
        return det.det_gemm(x, w, check_finite=False)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_nonfinite_operands_set_the_status(dt):
    _status()
    x, w = _operands(dt, 37, 70, 300, 11)
    for name, call in _entry_points(x, w).items():
        announce(f"device status, finite operands: {name} {dt}")
        call()
        assert _status() == set(), name
    for bad in BAD:
        for side in ("x", "w"):
            xb, wb = x.clone(), w.clone()
            (xb if side == "x" else wb)[5, 123] = bad
            for name, call in _entry_points(xb, wb).items():
                if side == "w" and ("dot" in name or "sqdiff" in name):
                    continue                                   # the dot products read x only
                announce(f"device status, {bad} in {side}: {name} {dt}")
                call()
                assert _status() == {"nonfinite"}, (name, side, bad)
                assert _status() == set(), "det_device_status(clear=1) leaves the status clear"


def test_status_is_sticky_and_readable_without_waiting():
    _status()
    x, w = _operands(torch.float32, 8, 9, 20, 12)
    x[1, 2] = float("nan")
    det.det_gemm(x, w, check_finite=False)
    det.det_gemm(x.nan_to_num(), w, check_finite=False)        # a later clean call keeps it set
    lib = _lib.load()
    ptr = lib.det_device_status_word()
    assert ptr
    # the word read by a device copy on the stream, without det_device_status
    words = torch.empty(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipMemcpyDtoDAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert hip.hipMemcpyDtoDAsync(words.data_ptr(), ptr, 16, stream.cuda_stream) == 0
    assert words.cpu().tolist() == [1, 0, 0, 0]
    assert det.device_status(clear=False) == {"nonfinite"}
    flags = ctypes.c_int()
    st = lib.det_device_status(ctypes.c_void_p(stream.cuda_stream), 1, ctypes.byref(flags))
    assert st == _lib.DET_ENONFINITE and flags.value == 1
    assert "Inf or NaN" in _lib.last_error()
    st = lib.det_device_status(ctypes.c_void_p(stream.cuda_stream), 1, ctypes.byref(flags))
    assert st == _lib.DET_OK and flags.value == 0


def _finalize_flags(digits):
    acc = torch.tensor(digits, dtype=torch.int64).reshape(-1, 18).cuda()
    det.det_finalize(acc)
    return _status()


def test_finalize_digits_out_of_range_set_the_status():
    _status()
    edge = 2 ** 62
    for j in (0, 9, 17):
        for v, want in ((edge, set()), (-edge, set()), (edge + 1, {"range"}), (-edge - 1, {"range"}),
                        (2 ** 63 - 1, {"range"}), (-2 ** 63, {"range"})):
            announce(f"finalize digit {j} = {v}")
            d = [0] * 18
            d[j] = v
            assert _finalize_flags([d, [1] * 18]) == want, (j, v)


def _combine_flags(parts):
    ps = [torch.tensor(p, dtype=torch.int64).reshape(-1, 18).cuda() for p in parts]
    out = det.det_combine(ps)
    torch.cuda.synchronize()
    return _status(), out.cpu()


def test_combine_out_of_range_sets_the_status():
    _status()
    edge = 2 ** 62
    row = lambda v: [v] + [0] * 17                              # noqa: E731
    # in range: parts and total within +-2^62, although int64 partial sums of
    # (2^62, 2^62, -2^62) pass 2^63
    for parts in ([row(edge), row(-edge)], [row(edge - 5), row(5)], [row(edge), row(edge), row(-edge)]):
        announce(f"combine in range {[p[0] for p in parts]}")
        flags, out = _combine_flags(parts)
        assert flags == set()
        assert out[0, 0].item() == sum(p[0] for p in parts)
    # out of range: a total beyond 2^62, a part beyond it, and four parts of
    # 2^62 whose int64 sum wraps to 0
    for parts in ([row(edge), row(1)], [row(edge + 1), row(-5)], [row(edge)] * 4, [row(-edge)] * 3):
        announce(f"combine out of range {[p[0] for p in parts]}")
        flags, _ = _combine_flags(parts)
        assert flags == {"range"}
