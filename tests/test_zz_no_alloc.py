"""det_gemm_noalloc (the entry point with a static device scratch) against
det_gemm_ws, through the C ABI: two calls in a row sharing the scratch, the
second smaller, each bit for bit; and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import c_oracle
from tests.gpu_util import announce, f32_bits, mismatch_report, to_device
from workloads import random_operands
import bitwise_deterministic_exact_amd as det
from bitwise_deterministic_exact_amd import _lib

pytestmark = pytest.mark.gpu


def _noalloc(x, w, y, dt):
    lib = _lib.load()
    M, K = x.shape
    N = w.shape[0]
    return lib.det_gemm_noalloc(0 if dt == "f32" else 1, ctypes.c_void_p(x.data_ptr()), x.stride(0), x.stride(1),
                                ctypes.c_void_p(w.data_ptr()), w.stride(0), w.stride(1), M, N, K,
                                ctypes.c_void_p(y.data_ptr()), y.stride(0), y.stride(1),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_noalloc_matches_workspace_entry_point(dt):
    rng = np.random.default_rng(41 if dt == "f32" else 42)
    # first call: two K blocks (the digits carried between them live in the
    # scratch) and two epochs per block; second call smaller, same scratch
    cases = [(40, 60, 40000, "wide"), (17, 33, 5000, "normal")]
    inputs, outs = [], []
    for (M, N, K, kind) in cases:
        xb, wb = random_operands(rng, M, N, K, dt, kind)
        x, w = to_device(xb, dt), to_device(wb, dt)
        inputs.append((xb, wb, x, w))
        outs.append(torch.full((M, N), float("nan"), dtype=torch.float32, device=x.device))
    torch.cuda.synchronize()
    for (xb, wb, x, w), y in zip(inputs, outs):
        announce(f"det_gemm_noalloc {dt} M={x.shape[0]} N={w.shape[0]} K={x.shape[1]}")
        assert _noalloc(x, w, y, dt) == _lib.DET_OK, _lib.last_error()
    torch.cuda.synchronize()
    for (xb, wb, x, w), y in zip(inputs, outs):
        want = f32_bits(det.det_gemm(x, w, workspace=True))       # the existing entry point, det_gemm_ws
        got = f32_bits(y)
        assert np.array_equal(got, want), mismatch_report(got, want)
        oracle_y = c_oracle.gemm(xb, wb)
        assert np.array_equal(got, oracle_y), mismatch_report(got, oracle_y)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lib = _lib.load()
    assert lib.det_gemm_noalloc_max_bytes() == 64 << 20
    x = torch.zeros((4096, 4096), dtype=torch.float32, device="cuda")
    y = torch.empty((4096, 4096), dtype=torch.float32, device="cuda")
    assert _noalloc(x, x, y, "f32") == _lib.DET_EINVAL
    assert "scratch" in _lib.last_error()
    with pytest.raises(ValueError):
        det.det_gemm_noalloc(x, x, y)
