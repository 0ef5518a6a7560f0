"""GPU parity on the five workload configurations, at their full sizes and in
the launch configuration the benchmark times.

The oracle checks every output of the small configurations, of the 4096^3
wide-range one and of the DetLinear forward (each under a minute on the
host's cores). Where it cannot finish the whole output in that time (the
2^19-long K, the DetLinear backward) it checks sampled outputs one by one,
and the whole output is checked through properties that hold at any size:
det_gemm equals det_finalize of det_gemm_partial, and K-sharded compositions
equal the unsharded digits bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import c_oracle
from tests.gpu_util import announce, digest, f32_bits, mismatch_report, tensor_bits, to_device
import workloads as W
import bitwise_deterministic_exact_amd as det

pytestmark = pytest.mark.gpu


def _sample(rng, M, N, count):
    return rng.integers(0, M, count), rng.integers(0, N, count)


def test_c1_f32_64x64x256_two_shards():
    wl = W.c1_small_f32()
    xb, wb = wl.bits()
    announce("C1 f32 64x64x256, shards [0,100) and [100,256)")
    x, w = to_device(xb, "f32"), to_device(wb, "f32")
    want_d = c_oracle.partial(xb, wb)
    want_y = c_oracle.finalize(want_d)
    y = det.det_gemm(x, w)
    assert np.array_equal(f32_bits(y), want_y), mismatch_report(f32_bits(y), want_y)
    d = det.det_gemm_partial(x, w)
    assert np.array_equal(d.cpu().numpy(), want_d)
    a1 = det.det_gemm_partial(x[:, :100], w[:, :100])
    a2 = det.det_gemm_partial(x[:, 100:], w[:, 100:])
    acc = det.det_combine([a1, a2])
    assert torch.equal(acc, d)                                    # digit for digit
    assert torch.equal(det.det_finalize(acc).view(torch.int32), y.view(torch.int32))
    assert np.array_equal(a1.cpu().numpy(), c_oracle.partial(xb[:, :100], wb[:, :100]))


def test_c2_bf16_1024_cancelling_columns():
    wl = W.c2_bf16_cancel()
    xb, wb = wl.bits()
    announce("C2 bf16 1024^3 with 10% negated w columns: full oracle check")
    x, w = to_device(xb, "bf16"), to_device(wb, "bf16")
    want_d = c_oracle.partial(xb, wb)
    want_y = c_oracle.finalize(want_d)
    got_y = f32_bits(det.det_gemm(x, w))
    assert np.array_equal(got_y, want_y), mismatch_report(got_y, want_y)
    got_d = det.det_gemm_partial(x, w).cpu().numpy()
    assert np.array_equal(got_d, want_d)
    # the forced-cancellation variant: x columns copied alongside, so every
    # negated pair of products cancels exactly
    targets = np.array([int(v) for v in wl.note.split("targets=[")[1].split("]")[0].split(",")])
    sources = np.array([int(v) for v in wl.note.split("sources=[")[1].split("]")[0].split(",")])
    xc = xb.copy()
    xc[:, targets] = xc[:, sources]
    keep = np.setdiff1d(np.arange(xb.shape[1]), np.concatenate([targets, sources]))
    y_cancel = f32_bits(det.det_gemm(to_device(xc, "bf16"), w))
    y_rest = f32_bits(det.det_gemm(to_device(np.ascontiguousarray(xc[:, keep]), "bf16"),
                                   to_device(np.ascontiguousarray(wb[:, keep]), "bf16")))
    assert np.array_equal(y_cancel, y_rest)


@pytest.fixture(scope="module")
def c3():
    announce("C3 generating f32 4096^3 wide-range inputs")
    wl = W.c3_wide_f32()
    xb, wb = wl.bits()
    return xb, wb, to_device(xb, "f32"), to_device(wb, "f32")


def test_c3_f32_4096_wide_range(c3):
    xb, wb, x, w = c3
    announce("C3 det_gemm and det_gemm_partial 4096^3")
    y = det.det_gemm(x, w, check_finite=False)
    d = det.det_gemm_partial(x, w, check_finite=False)
    # every output against the oracle (6.9e10 exact products on the host's
    # cores, about half a minute): raw digits and the rounded fp32
    announce("C3 the oracle's 4096 x 4096 raw digits (all outputs)")
    want_d = c_oracle.partial(xb, wb)
    got_d = d.cpu().numpy()
    assert np.array_equal(got_d, want_d), mismatch_report(got_d.reshape(-1, 18), want_d.reshape(-1, 18))
    got_y = f32_bits(y)
    want_y = c_oracle.finalize(want_d)
    assert np.array_equal(got_y, want_y), mismatch_report(got_y.ravel(), want_y.ravel())
    del got_d, want_d
    # whole output: fused rounding == finalize of the raw digits
    assert torch.equal(det.det_finalize(d).view(torch.int32), y.view(torch.int32))
    # most outputs overflow (products reach 2^142); check both kinds are present
    yb = f32_bits(y)
    assert np.count_nonzero((yb & 0x7FFFFFFF) == 0x7F800000) > 0
    del d


def test_c3_sharded_equals_unsharded(c3):
    xb, wb, x, w = c3
    announce("C3 3-way K-shard composition vs unsharded digits")
    whole = det.det_gemm_partial(x[:512], w, check_finite=False)
    parts = [det.det_gemm_partial(x[:512, a:b], w[:, a:b], check_finite=False)
             for a, b in [(0, 1000), (1000, 3333), (3333, 4096)]]
    assert torch.equal(det.det_combine(parts), whole)
    y = det.det_gemm(x[:512], w, check_finite=False)
    assert torch.equal(det.det_finalize(whole).view(torch.int32), y.view(torch.int32))


def test_c4_ksharded_2048_k2e19_fold_tree():
    announce("C4 generating f32 2048 x 2048, K = 2^19 (8 GiB of operands)")
    wl = W.c4_ksharded_f32()
    xb, wb = wl.bits()
    x, w = to_device(xb, "f32"), to_device(wb, "f32")
    K = x.shape[1]
    announce("C4 unsharded partial")
    whole = det.det_gemm_partial(x, w, check_finite=False)
    announce(f"C4 16 shards at {wl.cuts[:3]}..., fold tree of {len(wl.fold)} combines")
    parts = [det.det_gemm_partial(x[:, a:b], w[:, a:b], check_finite=False)
             for a, b in W.shard_bounds(K, wl.cuts)]
    folded = W.apply_fold(parts, wl.fold, det.det_combine)
    assert torch.equal(folded, whole)
    assert torch.equal(det.det_combine(parts), whole)
    del parts
    y_sharded = det.det_finalize(folded)
    y = det.det_gemm(x, w, check_finite=False)
    assert torch.equal(y_sharded.view(torch.int32), y.view(torch.int32))
    # a seeded 1 % sample of the outputs (41943 of 2048^2, each with all 2^19
    # products) against the oracle; the whole output is covered by the
    # sharded == unsharded digit equality above
    count = 2048 * 2048 // 100
    announce(f"C4 {count} sampled outputs (1 %) against the oracle")
    flat = np.random.default_rng(41).choice(2048 * 2048, count, replace=False)
    rows, cols = flat // 2048, flat % 2048
    want_d = c_oracle.partial_pairs(xb, wb, rows, cols)
    got_d = whole[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    assert np.array_equal(got_d, want_d), mismatch_report(got_d, want_d)
    assert np.array_equal(f32_bits(y)[rows, cols], c_oracle.finalize(want_d))
    # repeat: identical digest
    assert digest(f32_bits(det.det_gemm(x, w, check_finite=False))) == digest(f32_bits(y))


def test_c5_detlinear_4096_bf16_8192_tokens():
    wl = W.c5_detlinear_bf16()
    xb, Wb = wl.x, wl.w
    announce("C5 DetLinear 4096->4096 bf16, 8192 tokens, forward + backward")
    layer = det.DetLinear(4096, 4096, device="cuda", dtype=torch.bfloat16)
    with torch.no_grad():
        layer.weight.copy_(to_device(Wb, "bf16"))
    x = to_device(xb, "bf16").requires_grad_(True)
    y = layer(x)
    loss = y.square().mean()
    loss.backward()
    rng = np.random.default_rng(51)
    # forward: y = x W^T, K = 4096, every output against the oracle (1.4e11
    # exact products on the host's cores, well under a minute)
    announce("C5 the oracle's forward, all 8192 x 4096 outputs")
    want = c_oracle.gemm(xb, Wb)
    yb = f32_bits(y)
    assert np.array_equal(yb, want), mismatch_report(yb.ravel(), want.ravel())
    # dY = 2 y / numel = y * 2^-24 exactly (powers of two), rounded to bf16
    g32 = (yb.view(np.float32) * np.float32(2.0 ** -24)).astype(np.float32)
    gb = torch.from_numpy(g32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # dX = dY W, K = 4096 (out); dW = dY^T x, K = 8192 (tokens)
    WT = np.ascontiguousarray(Wb.T)
    gT = np.ascontiguousarray(gb.T)
    xT = np.ascontiguousarray(xb.T)
    dx_bits = tensor_bits(x.grad)
    dw_bits = tensor_bits(layer.weight.grad)
    # every output of dX (8192 x 4096, K = 4096) and of dW (4096 x 4096, K =
    # 8192) against the oracle's fp32 result rounded to bf16 (nearest-even,
    # torch's CPU cast): 1.4e11 exact products each on the host's cores
    announce("C5 the oracle's dX = dY W, all 8192 x 4096 outputs")
    dx32 = c_oracle.gemm(gb, WT).view(np.float32)
    want_dx = torch.from_numpy(dx32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(dx_bits, want_dx), mismatch_report(dx_bits.ravel(), want_dx.ravel())
    del dx32, want_dx
    announce("C5 the oracle's dW = dY^T x, all 4096 x 4096 outputs")
    dw32 = c_oracle.gemm(gT, xT).view(np.float32)
    want_dw = torch.from_numpy(dw32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(dw_bits, want_dw), mismatch_report(dw_bits.ravel(), want_dw.ravel())
    del dw32, want_dw
    # the same step again gives identical bytes
    x2 = to_device(xb, "bf16").requires_grad_(True)
    layer.weight.grad = None
    layer(x2).square().mean().backward()
    assert np.array_equal(tensor_bits(x2.grad), dx_bits)
    assert np.array_equal(tensor_bits(layer.weight.grad), dw_bits)
    # the exact loss (the step bench.py times) gives the same gradients: its
    # dY = 2 y / 2^25 is the same power-of-two scaling of y
    x3 = to_device(xb, "bf16").requires_grad_(True)
    layer.weight.grad = None
    loss = det.exact_mse_loss(layer(x3))
    loss.backward()
    assert np.array_equal(tensor_bits(x3.grad), dx_bits)
    assert np.array_equal(tensor_bits(layer.weight.grad), dw_bits)
    flat = yb.reshape(-1)                          # sum y^2 over K-slices within the oracle's 2^19
    parts = [c_oracle.partial(flat[a:a + 400_000].reshape(1, -1), flat[a:a + 400_000].reshape(1, -1))
             for a in range(0, flat.size, 400_000)]
    s_exact = c_oracle.finalize(c_oracle.combine(parts)).reshape(-1)[0]     # rounded once
    want_loss = np.float32(np.array([s_exact], dtype=np.uint32).view(np.float32)[0] / np.float32(yb.size))
    assert f32_bits(loss.reshape(1))[0] == want_loss.view(np.uint32)
