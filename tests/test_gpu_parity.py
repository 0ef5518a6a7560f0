"""GPU parity: the HIP path against the oracle, element by element and bit for
bit, at sizes the oracle finishes in seconds (several 16x16 output tiles and
16-wide K chunks, ragged tails, empty and degenerate shapes, strided views).

Everything is called through the C ABI (via the thin Python binding)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from oracle import c_oracle
from tests import pins
from tests.gpu_util import announce, digest, f32_bits, mismatch_report, tensor_bits, to_device
from workloads import random_operands, shard_bounds
import bitwise_deterministic_exact_amd as det
from bitwise_deterministic_exact_amd import _lib

pytestmark = pytest.mark.gpu

KINDS = ["normal", "uniform", "wide", "special", "int"]
SHAPES = [(1, 1, 1), (3, 5, 1), (16, 16, 16), (17, 33, 47), (31, 17, 100), (64, 48, 257),
          (5, 70, 33), (40, 3, 16)]


def _gemm(xb, wb, dt):
    return f32_bits(det.det_gemm(to_device(xb, dt), to_device(wb, dt)))


def _partial(xb, wb, dt):
    return det.det_gemm_partial(to_device(xb, dt), to_device(wb, dt)).cpu().numpy()


def test_golden_fixtures_on_gpu():
    announce("golden digits and rounding fixtures")
    assert pins.check_golden_digits(
        _partial, lambda d: f32_bits(det.det_finalize(torch.from_numpy(d).cuda()))) == []
    assert pins.check_golden_rounding(_gemm) == []


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", KINDS)
def test_random_shapes_bit_exact(kind, dt):
    rng = np.random.default_rng(100 + 2 * KINDS.index(kind) + (dt == "bf16"))
    for (M, N, K) in SHAPES:
        announce(f"random {kind} {dt} M={M} N={N} K={K}")
        xb, wb = random_operands(rng, M, N, K, dt, kind)
        want_d = c_oracle.partial(xb, wb)
        want_y = c_oracle.finalize(want_d)
        x, w = to_device(xb, dt), to_device(wb, dt)
        got_d = det.det_gemm_partial(x, w).cpu().numpy()
        assert np.array_equal(got_d, want_d), mismatch_report(got_d, want_d)
        got_y = f32_bits(det.det_gemm(x, w))
        assert np.array_equal(got_y, want_y), mismatch_report(got_y, want_y)
        fin = f32_bits(det.det_finalize(torch.from_numpy(want_d).cuda()))
        assert np.array_equal(fin, want_y), mismatch_report(fin, want_y)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_workspace_and_inkernel_decode_agree(dt):
    # the two ways of decoding w (once into a workspace, or in the GEMM
    # kernel) against the oracle, on strided and transposed w
    rng = np.random.default_rng(29 if dt == "f32" else 30)
    for kind in ("wide", "special", "normal"):
        announce(f"workspace vs in-kernel decode {kind} {dt}")
        xb, wb = random_operands(rng, 37, 70, 130, dt, kind)
        x, w = to_device(xb, dt), to_device(wb, dt)
        want_d = c_oracle.partial(xb, wb)
        want_y = c_oracle.finalize(want_d)
        wt = w.t().contiguous().t()
        for ww in (w, wt, to_device(np.ascontiguousarray(np.pad(wb, ((0, 0), (3, 0)))), dt)[:, 3:]):
            for use in (True, False):
                assert np.array_equal(f32_bits(det.det_gemm(x, ww, workspace=use)), want_y), (use,)
                got = det.det_gemm_partial(x, ww, workspace=use).cpu().numpy()
                assert np.array_equal(got, want_d), (use,)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_long_k_counter_folds(dt):
    # K long enough for several epochs of cell folds and digit carries inside
    # the kernels (f32: a fold every 4096 k; bf16: every 512 k; the partial's
    # counters: a block every 2^15 k), all signs and magnitudes
    rng = np.random.default_rng(33 if dt == "f32" else 34)
    for kind, K in (("wide", 5000), ("wide", 8200), ("normal", 9000), ("normal", 70001), ("special", 3000)):
        announce(f"long K {kind} {dt} K={K}")
        xb, wb = random_operands(rng, 5, 66, K, dt, kind)
        x, w = to_device(xb, dt), to_device(wb, dt)
        want_d = c_oracle.partial(xb, wb)
        want_y = c_oracle.finalize(want_d)
        for use in (True, False):
            got_y = f32_bits(det.det_gemm(x, w, workspace=use))
            assert np.array_equal(got_y, want_y), mismatch_report(got_y, want_y)
            got_d = det.det_gemm_partial(x, w, workspace=use).cpu().numpy()
            assert np.array_equal(got_d, want_d), mismatch_report(got_d, want_d)


def test_small_against_python_oracle():
    rng = np.random.default_rng(21)
    for dt in ("f32", "bf16"):
        for kind in ("wide", "special"):
            announce(f"python oracle {kind} {dt}")
            xb, wb = random_operands(rng, 9, 7, 37, dt, kind)
            assert np.array_equal(_partial(xb, wb, dt), oracle.partial(xb, wb, dt))
            assert np.array_equal(_gemm(xb, wb, dt), oracle.gemm(xb, wb, dt))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_empty_and_degenerate(dt):
    rng = np.random.default_rng(22)
    for (M, N, K) in [(0, 5, 3), (5, 0, 3), (0, 0, 0), (4, 6, 0)]:
        announce(f"empty {dt} M={M} N={N} K={K}")
        xb, wb = random_operands(rng, M, N, K, dt, "normal")
        x, w = to_device(xb, dt), to_device(wb, dt)
        y = det.det_gemm(x, w)
        assert y.shape == (M, N)
        assert np.all(f32_bits(y) == 0)                      # K = 0: +0.0
        d = det.det_gemm_partial(x, w)
        assert d.shape == (M, N, 18) and int(d.abs().sum()) == 0
    # all-zero and cancelling operands give +0.0; all products -0 give +0.0
    z = torch.zeros(3, 40, device="cuda", dtype=torch.float32 if dt == "f32" else torch.bfloat16)
    assert np.all(f32_bits(det.det_gemm(z, -z)) == 0)
    a = torch.from_numpy(np.linspace(-3, 3, 40, dtype=np.float32)).reshape(1, 40).cuda()
    a = a.to(z.dtype)
    both = torch.cat([a, -a], dim=1)
    ones = torch.ones_like(both)
    assert np.all(f32_bits(det.det_gemm(both, ones)) == 0)


def test_strided_and_transposed_views():
    rng = np.random.default_rng(23)
    for dt in ("f32", "bf16"):
        announce(f"views {dt}")
        xb, wb = random_operands(rng, 37, 29, 90, dt, "wide")
        xbig, wbig = to_device(xb, dt), to_device(wb, dt)
        # K-slices (row stride 90, start offset 17 elements: misaligned for bf16)
        xs, ws = xbig[:, 17:83], wbig[:, 17:83]
        want = c_oracle.partial(xb[:, 17:83], wb[:, 17:83])
        assert np.array_equal(det.det_gemm_partial(xs, ws).cpu().numpy(), want)
        # transposed storage: x^T stored [K, M] and used as a [M, K] view
        xt = xbig.t().contiguous().t()
        wt = wbig.t().contiguous().t()
        assert xt.stride() == (1, 37)
        want_y = c_oracle.gemm(xb, wb)
        assert np.array_equal(f32_bits(det.det_gemm(xt, wt)), want_y)
        assert np.array_equal(f32_bits(det.det_gemm(xbig, wt)), want_y)
        # every other row and column
        xe, we = xbig[::2, ::3], wbig[1::2, ::3]
        want_y = c_oracle.gemm(np.ascontiguousarray(xb[::2, ::3]), np.ascontiguousarray(wb[1::2, ::3]))
        assert np.array_equal(f32_bits(det.det_gemm(xe, we)), want_y)
        # output into a strided view
        out = torch.empty(29, 37, device="cuda", dtype=torch.float32).t()
        det.det_gemm(xbig, wbig, out=out)
        assert np.array_equal(f32_bits(out), c_oracle.gemm(xb, wb))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_k_partitions_and_fold_trees(dt):
    rng = np.random.default_rng(24 if dt == "f32" else 25)
    M, N, K = 40, 36, 600
    xb, wb = random_operands(rng, M, N, K, dt, "wide")
    x, w = to_device(xb, dt), to_device(wb, dt)
    whole = det.det_gemm_partial(x, w)
    want = c_oracle.partial(xb, wb)
    assert np.array_equal(whole.cpu().numpy(), want)
    y_full = f32_bits(det.det_gemm(x, w))
    for nshards in (2, 4, 8, 16):
        announce(f"partition {dt} {nshards}-way")
        cuts = sorted(rng.choice(np.arange(1, K), nshards - 1, replace=False).tolist())
        parts = [det.det_gemm_partial(x[:, a:b], w[:, a:b]) for a, b in shard_bounds(K, cuts)]
        # n-ary combine, then a random fold tree
        assert torch.equal(det.det_combine(parts), whole)
        live = list(parts)
        while len(live) > 1:
            i, j = sorted(rng.choice(len(live), 2, replace=False).tolist())
            b_ = live.pop(j)
            a_ = live.pop(i)
            live.append(det.det_combine([a_, b_]))
        assert torch.equal(live[0], whole)
        assert np.array_equal(f32_bits(det.det_finalize(live[0])), y_full)
    # the K-permuted GEMM has identical digits too
    perm = torch.from_numpy(rng.permutation(K)).cuda()
    assert torch.equal(det.det_gemm_partial(x[:, perm], w[:, perm]), whole)


def test_combine_many_parts_and_aliasing():
    announce("combine of 70 parts, in-place")
    g = torch.Generator().manual_seed(5)
    parts = [torch.randint(-2 ** 40, 2 ** 40, (33, 18), generator=g, dtype=torch.int64).cuda()
             for _ in range(70)]
    want = torch.stack([p.cpu() for p in parts]).sum(0)
    assert torch.equal(det.det_combine(parts).cpu(), want)
    # through the C ABI, with out equal to a part that falls in a later group
    # of 32 (parts[35] of 40), then equal to two parts (one in each group)
    lib = _lib.load()
    for nparts, alias in ((40, (35,)), (40, (3, 38)), (70, (69,))):
        announce(f"combine of {nparts} parts, out == parts{list(alias)}")
        ps = [p.clone() for p in parts[:nparts]]
        for i in alias[1:]:
            ps[i] = ps[alias[0]]
        want = torch.stack([p.cpu() for p in ps]).sum(0)
        out = ps[alias[0]]
        ptrs = (ctypes.c_void_p * nparts)(*[p.data_ptr() for p in ps])
        st = lib.det_combine(ptrs, nparts, ctypes.c_void_p(out.data_ptr()), 33,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == _lib.DET_OK, _lib.last_error()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), want)


def test_finalize_random_digit_arrays():
    announce("finalize on random raw digit arrays")
    rng = np.random.default_rng(26)
    d = rng.integers(-(2 ** 52), 2 ** 52, size=(5000, 18), dtype=np.int64)
    d[::3, 12:] = 0
    d[1::3, :6] = 0
    d[2::5, :] = np.where(rng.random((1000, 18)) < 0.5, -(2 ** 32) + 1, 2 ** 32 - 1)
    d[::7, 17] = 0
    d[::11, 10:] = 0
    d[::11, :10] = rng.integers(-3, 4, size=(455, 10))
    d[::13, :] = 0
    d[::17, 17] = rng.integers(2 ** 40, 2 ** 50, size=295)     # values far beyond fp32: inf
    got = f32_bits(det.det_finalize(torch.from_numpy(d).cuda()))
    want = c_oracle.finalize(d)
    assert np.array_equal(got, want), mismatch_report(got, want)


def test_round_f32_to_bf16_kernel():
    announce("f32 -> bf16 rounding kernel")
    rng = np.random.default_rng(27)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        random_operands(rng, 1, 1, 5000, "f32", "wide")[0].view(np.float32).ravel(),
        ((rng.integers(0, 2 ** 16, 4000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 2.0 ** -149, 3.3895e38, 3.4e38, np.inf, -np.inf], dtype=np.float32)])
    v = v[~np.isnan(v)]
    want = oracle.f32_bits_to_bf16_bits(v.view(np.uint32))
    t = torch.from_numpy(v).cuda()
    got = tensor_bits(det.round_f32_to_bf16(t))
    assert np.array_equal(got, want)
    # 8 elements per thread on 16-byte aligned data, one at a time otherwise,
    # and the last n mod 8 elements one at a time
    for lo, hi in ((4, 4 + 8 * 1000), (1, 5003), (8, 15), (3, 4)):
        got = tensor_bits(det.round_f32_to_bf16(t[lo:hi]))
        assert np.array_equal(got, want[lo:hi]), (lo, hi)


def test_nonfinite_inputs_rejected():
    announce("non-finite inputs")
    x = torch.randn(8, 20, device="cuda")
    w = torch.randn(6, 20, device="cuda")
    assert not det.has_nonfinite(x)
    for bad in (float("inf"), float("-inf"), float("nan")):
        xb = x.clone()
        xb[3, 7] = bad
        assert det.has_nonfinite(xb)
        assert det.has_nonfinite(xb.t())
        with pytest.raises(ValueError, match="Inf or NaN"):
            det.det_gemm(xb, w)
        with pytest.raises(ValueError, match="Inf or NaN"):
            det.det_gemm_partial(w, xb)
        # unchecked: no fault, results unspecified but the call completes
        det.det_gemm(xb, w, check_finite=False)
        torch.cuda.synchronize()


def test_repeat_runs_and_streams_identical():
    rng = np.random.default_rng(28)
    xb, wb = random_operands(rng, 200, 150, 700, "f32", "wide")
    x, w = to_device(xb, "f32"), to_device(wb, "f32")
    announce("repeat runs and a side stream")
    ref = f32_bits(det.det_gemm(x, w))
    d_ref = det.det_gemm_partial(x, w).cpu().numpy()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y2 = det.det_gemm(x, w)
        d2 = det.det_gemm_partial(x, w)
    s.synchronize()
    digests = {digest(f32_bits(det.det_gemm(x, w))) for _ in range(5)}
    digests.add(digest(f32_bits(y2)))
    assert digests == {digest(ref)}
    assert np.array_equal(d2.cpu().numpy(), d_ref)
    assert np.array_equal(ref, c_oracle.gemm(xb, wb))


def test_control_plain_fp32_matmul_is_not_invariant():
    # a control that must differ: torch's fp32 matmul over K-shards vs whole
    announce("fp32 control")
    g = torch.Generator().manual_seed(3)
    x = torch.randn(256, 4096, generator=g).cuda()
    w = torch.randn(256, 4096, generator=g).cuda()
    whole = x @ w.t()
    sharded = sum(x[:, a:b] @ w[:, a:b].t() for a, b in [(0, 1000), (1000, 2500), (2500, 4096)])
    assert not torch.equal(whole, sharded)
    exact = det.det_gemm(x, w)
    shard_parts = [det.det_gemm_partial(x[:, a:b], w[:, a:b]) for a, b in [(0, 1000), (1000, 2500), (2500, 4096)]]
    assert torch.equal(det.det_finalize(det.det_combine(shard_parts)), exact)
