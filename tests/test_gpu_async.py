"""det_gemm's default path decides on the device: the host never waits, the
call can be captured in a HIP graph, and one captured graph follows the data
(the matrix-core pass for narrow-span operands, the digit accumulator for
wide ones) with the oracle's bits every time.  DET_PATH_AUTO_HOST, the
opt-in that waits for the span histogram, gives the same bits."""
import numpy as np
import pytest
import torch

from oracle import c_oracle
import bitwise_deterministic_exact_amd as det
from tests.gpu_util import announce, f32_bits, mismatch_report, to_device
from workloads import random_operands

pytestmark = pytest.mark.gpu


def _sampled_oracle(xb, wb, step=(37, 41)):
    M, N = xb.shape[0], wb.shape[0]
    rr, cc = np.meshgrid(np.arange(0, M, step[0]), np.arange(3, N, step[1]), indexing="ij")
    return rr.ravel(), cc.ravel(), c_oracle.gemm_pairs(xb, wb, rr.ravel(), cc.ravel())


def test_auto_path_does_not_wait_for_the_device():
    rng = np.random.default_rng(700)
    xb, wb = random_operands(rng, 512, 512, 1024, "bf16", "normal")
    x, w = to_device(xb, "bf16"), to_device(wb, "bf16")
    y = torch.empty(512, 512, device="cuda")
    det.det_gemm(x, w, check_finite=False, out=y)         # workspace and plan buffers exist
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for path in ("auto", "slices", "accumulator"):
        announce(f"host does not wait: path {path}")
        with det.gemm_path(path):
            torch.cuda._sleep(200_000_000)                  # the stream is busy for a while
            det.det_gemm(x, w, check_finite=False, out=y)
            busy = not stream.query()
            torch.cuda.synchronize()
        assert busy, f"det_gemm on path {path} returned only after the stream had drained"
    rr, cc, want = _sampled_oracle(xb, wb)
    assert np.array_equal(f32_bits(y)[rr, cc], want)


def test_one_captured_graph_follows_the_data():
    # the same shape with narrow-span (N(0,1)) and wide-range operands: the
    # plan made at replay picks the matrix cores for the first and the
    # accumulator for the second, inside one graph
    rng = np.random.default_rng(701)
    M = N = K = 512
    cases = []
    for kind in ("normal", "wide", "normal", "special"):
        xb, wb = random_operands(rng, M, N, K, "f32", kind)
        cases.append((kind, xb, wb))
    # N(0,1) with every 7th row of x and 9th of w wide-range: the matrix
    # cores for the rest, and the device-counted recompute of those rows
    # (far more than 256 tails each) inside the same graph
    xn, wn = random_operands(rng, M, N, K, "f32", "normal")
    xw, ww = random_operands(rng, M, N, K, "f32", "wide")
    xn[::7], wn[::9] = xw[::7], ww[::9]
    cases.append(("mixed", xn, wn))
    x = torch.empty(M, K, device="cuda")
    w = torch.empty(N, K, device="cuda")
    y = torch.empty(M, N, device="cuda")
    x.copy_(to_device(cases[0][1], "f32"))
    w.copy_(to_device(cases[0][2], "f32"))
    with det.gemm_path("auto"):
        det.det_gemm(x, w, check_finite=False, out=y)     # warm up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            det.det_gemm(x, w, check_finite=False, out=y)
    torch.cuda.synchronize()
    for rep in range(2):
        for kind, xb, wb in cases:
            announce(f"graph replay {rep}: {kind} operands")
            x.copy_(to_device(xb, "f32"))
            w.copy_(to_device(wb, "f32"))
            y.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = f32_bits(y)
            with det.gemm_path("accumulator"):
                eager = f32_bits(det.det_gemm(x, w, check_finite=False))
            assert np.array_equal(got, eager), mismatch_report(got, eager)
            rr, cc, want = _sampled_oracle(xb, wb)
            assert np.array_equal(got[rr, cc], want)
    # eager, the mixed operands take the matrix cores with listed rows
    with det.gemm_path("auto"):
        det.det_gemm(x, w, check_finite=False)
        plan = det.last_gemm_plan()
    assert plan["path"] == "slices" and plan["fallback_rows"] > 0 and plan["fallback_cols"] > 0, plan


@pytest.mark.parametrize("dt,kind", [("bf16", "normal"), ("f32", "normal"), ("f32", "wide")])
def test_device_and_host_choices_agree(dt, kind):
    rng = np.random.default_rng(702 + ["normal", "wide"].index(kind) + (dt == "bf16"))
    xb, wb = random_operands(rng, 512, 640, 768, dt, kind)
    x, w = to_device(xb, dt), to_device(wb, dt)
    out = {}
    for path in ("auto", "auto_host"):
        announce(f"{path} {dt} {kind}")
        with det.gemm_path(path):
            out[path] = (f32_bits(det.det_gemm(x, w, check_finite=False)), det.last_gemm_plan())
    assert np.array_equal(out["auto"][0], out["auto_host"][0])
    assert out["auto"][1] == out["auto_host"][1], (out["auto"][1], out["auto_host"][1])
    assert out["auto"][1]["path"] == ("accumulator" if kind == "wide" else "slices")
    rr, cc, want = _sampled_oracle(xb, wb)
    assert np.array_equal(out["auto"][0][rr, cc], want)
