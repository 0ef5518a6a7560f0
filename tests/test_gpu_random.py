"""Seeded random sweep of the GPU entry points against the oracle, bit for
bit: many small shapes (ragged against every tile), both dtypes, every value
kind the workloads know, transposed and sliced views, both det_gemm paths and
the automatic choice, the partials, and their composition over random K cuts."""
import numpy as np
import pytest
import torch

import bitwise_deterministic_exact_amd as det
from oracle import c_oracle
from tests.gpu_util import announce, f32_bits, mismatch_report, to_device
from workloads import random_operands, to_bf16_bits

pytestmark = pytest.mark.gpu

KINDS = ["normal", "uniform", "int", "wide", "special"]


@pytest.fixture(autouse=True)
def _auto_path_after():
    yield
    det.set_gemm_path("auto", 0)


def _view(t: torch.Tensor, how: int) -> torch.Tensor:
    """The same values as another memory layout: contiguous, column-major,
    or a slice of a wider buffer."""
    if how == 0:
        return t
    if how == 1:
        return t.t().contiguous().t()
    pad = torch.zeros(t.shape[0], t.shape[1] + 5, dtype=t.dtype, device=t.device)
    pad[:, 3:3 + t.shape[1]] = t
    return pad[:, 3:3 + t.shape[1]]


@pytest.mark.parametrize("seed", range(8))
def test_random_gemms_and_partials(seed):
    rng = np.random.default_rng(700 + seed)
    for case in range(25):
        dt = ["f32", "bf16"][int(rng.integers(0, 2))]
        kind = KINDS[int(rng.integers(0, len(KINDS)))]
        M, N, K = (int(v) for v in rng.integers(1, 200, 3))
        xb, wb = random_operands(rng, M, N, K, dt, kind)
        path = ["auto", "accumulator", "slices"][int(rng.integers(0, 3))]
        S = int(rng.integers(2, 8)) if path == "slices" and rng.random() < 0.5 else 0
        vx, vw = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        announce(f"seed {seed} case {case}: {dt} {kind} M={M} N={N} K={K} path={path} S={S} views={vx},{vw}")
        x, w = _view(to_device(xb, dt), vx), _view(to_device(wb, dt), vw)
        want = c_oracle.gemm(xb, wb)
        det.set_gemm_path(path, S)
        got = f32_bits(det.det_gemm(x, w))
        assert np.array_equal(got, want), mismatch_report(got, want)
        # raw digits, and their composition over random K cuts
        digits = c_oracle.partial(xb, wb)
        whole = det.det_gemm_partial(x, w).cpu().numpy()
        assert np.array_equal(whole, digits)
        cuts = sorted(set(int(c) for c in rng.integers(1, K, size=min(3, K - 1)))) if K > 1 else []
        bounds = list(zip([0] + cuts, cuts + [K]))
        parts = [det.det_gemm_partial(x[:, a:b], w[:, a:b]) for a, b in bounds]
        combined = det.det_combine(parts)
        assert np.array_equal(combined.cpu().numpy(), digits)
        assert np.array_equal(f32_bits(det.det_finalize(combined)), want)


def _scaled_operands(rng, M, N, K, dt, kind):
    """N(0,1) operands with rows scaled by random powers of two ("rowscaled"),
    or with one element in 500 scaled far up or down ("outlier"): rows of
    different spans for the matrix-core path's digits, listed rows and tails."""
    xb, wb = random_operands(rng, M, N, K, "f32", "normal")
    x, w = xb.view(np.float32).copy(), wb.view(np.float32).copy()
    if kind == "rowscaled":
        x *= np.exp2(rng.integers(-30, 31, size=(M, 1))).astype(np.float32)
        w *= np.exp2(rng.integers(-30, 31, size=(N, 1))).astype(np.float32)
    else:
        for a in (x, w):
            n = max(1, a.size // 500)
            idx = rng.integers(0, a.size, size=n)
            a.flat[idx] *= np.exp2(rng.integers(-60, 61, size=n)).astype(np.float32)
    if dt == "bf16":
        return to_bf16_bits(x), to_bf16_bits(w)
    return x.view(np.uint32), w.view(np.uint32)


@pytest.mark.parametrize("seed", range(3))
def test_random_larger_shapes(seed):
    """Larger ragged shapes whose K crosses the f32 accumulator's 4096-long
    epochs and the 2^14 / 2^15 K blocks of both paths, every path and digit
    count, with and without the workspace, against the oracle."""
    rng = np.random.default_rng(900 + seed)
    for case in range(6):
        dt = ["f32", "bf16"][int(rng.integers(0, 2))]
        kind = (KINDS + ["rowscaled", "outlier"])[int(rng.integers(0, len(KINDS) + 2))]
        M, N = (int(np.exp(rng.uniform(np.log(40), np.log(400)))) for _ in range(2))
        K = int(np.exp(rng.uniform(np.log(3000), np.log(70000))))
        K = min(K, int(4e8 // (M * N)))
        path = ["auto", "accumulator", "slices"][int(rng.integers(0, 3))]
        S = int(rng.integers(2, 8)) if path == "slices" and rng.random() < 0.5 else 0
        ws = bool(rng.random() < 0.75)
        vx, vw = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        announce(f"seed {seed} case {case}: {dt} {kind} M={M} N={N} K={K} path={path} S={S} "
                 f"workspace={ws} views={vx},{vw}")
        if kind in ("rowscaled", "outlier"):
            xb, wb = _scaled_operands(rng, M, N, K, dt, kind)
        else:
            xb, wb = random_operands(rng, M, N, K, dt, kind)
        x, w = _view(to_device(xb, dt), vx), _view(to_device(wb, dt), vw)
        want = c_oracle.gemm(xb, wb)
        det.set_gemm_path(path, S)
        got = f32_bits(det.det_gemm(x, w, workspace=ws))
        assert np.array_equal(got, want), mismatch_report(got, want)
        det.set_gemm_path("auto", 0)
        digits = c_oracle.partial(xb, wb)
        whole = det.det_gemm_partial(x, w, workspace=ws).cpu().numpy()
        assert np.array_equal(whole, digits)
