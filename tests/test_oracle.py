"""The oracle against what the det-train page and mathematics fix (CPU only).

Pins: hand-derived digits and rounding boundaries (tests/golden), exact
rational brute force, K = 1 against numpy's IEEE fp64 product and cast,
integer-exact products against numpy's fp64 matmul, closed forms, mpmath's
24-bit rounding, invariance under K permutation / partition / fold order,
bf16-vs-f32 digit identity, the accuracy claim against an fp64 matmul, and
the C oracle against the Python oracle.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import c_oracle
from tests import pins
from workloads import random_operands, f32_bits, to_bf16_bits

KINDS = ["normal", "uniform", "wide", "special", "int"]


def tiny_cases(seed=11, n=3):
    rng = np.random.default_rng(seed)
    cases = []
    for kind in KINDS:
        for dt in ("f32", "bf16"):
            for (M, N, K) in [(2, 3, 5), (3, 2, 16), (1, 1, 1)][:n]:
                x, w = random_operands(rng, M, N, K, dt, kind)
                cases.append((x, w, dt))
    return cases


def test_decode_known_values():
    assert oracle.decode(0x3F800000, "f32") == (0, 1 << 23, -23)
    assert oracle.decode(0xC0200000, "f32") == (1, 5 << 21, -22)      # -2.5 = -5*2^21*2^-22
    assert oracle.decode(0x00000001, "f32") == (0, 1, -149)           # 2^-149
    assert oracle.decode(0x00000000, "f32") == (0, 0, -149)
    assert oracle.decode(0x80000000, "f32") == (1, 0, -149)
    assert oracle.decode(0x7F7FFFFF, "f32") == (0, (1 << 24) - 1, 104)
    assert oracle.decode(0x3F80, "bf16") == (0, 1 << 7, -7)
    assert oracle.decode(0x0001, "bf16") == (0, 1, -133)              # 2^-133
    for bad, dt in [(0x7F800000, "f32"), (0xFFC00000, "f32"), (0x7F80, "bf16"), (0x7FC1, "bf16")]:
        with pytest.raises(ValueError):
            oracle.decode(bad, dt)


def test_golden_digits():
    assert pins.check_golden_digits(oracle.partial, oracle.finalize) == []


def test_golden_digits_c_oracle():
    def part(x, w, dt):
        return c_oracle.partial(x, w)
    assert pins.check_golden_digits(part, c_oracle.finalize) == []


def test_golden_rounding():
    assert pins.check_golden_rounding(oracle.gemm) == []
    assert pins.check_golden_rounding(lambda x, w, dt: oracle.finalize(oracle.partial(x, w, dt))) == []
    assert pins.check_golden_rounding(lambda x, w, dt: c_oracle.gemm(x, w)) == []


def test_fraction_brute_force():
    assert pins.check_fraction(oracle.partial, oracle.gemm, oracle.digits_value, tiny_cases()) == []


def test_k1_against_numpy_fp64():
    rng = np.random.default_rng(3)
    for kind in ("wide", "special", "normal"):
        x, w = random_operands(rng, 300, 200, 1, "f32", kind)
        assert pins.check_k1_numpy(oracle.gemm, x[:, 0], w[:, 0]) == []
        assert pins.check_k1_numpy(lambda a, b, dt: c_oracle.gemm(a, b), x[:, 0], w[:, 0]) == []


def test_integer_exact_and_closed_forms():
    assert pins.check_integer_exact(oracle.gemm, np.random.default_rng(4)) == []
    assert pins.check_integer_exact(lambda a, b, dt: c_oracle.gemm(a, b),
                                    np.random.default_rng(4)) == []


def test_mpmath_rounding():
    rng = np.random.default_rng(5)
    cases = []
    for kind in ("normal", "uniform", "wide"):
        for dt in ("f32", "bf16"):
            x, w = random_operands(rng, 4, 4, 12, dt, kind)
            cases.append((x, w, dt))
    assert pins.check_mpmath(oracle.gemm, cases) == []


def test_partition_and_fold_invariance():
    rng = np.random.default_rng(6)
    for kind in ("wide", "normal", "special"):
        for dt in ("f32", "bf16"):
            x, w = random_operands(rng, 3, 4, 40, dt, kind)
            assert pins.check_partition(oracle.partial, oracle.combine, x, w, dt, rng) == []


def test_c_oracle_partition_and_combine():
    # the C oracle's own partials and combine obey the same partition pin, and
    # its combine equals exact integer sums
    rng = np.random.default_rng(17)
    for dt in ("f32", "bf16"):
        for kind in ("wide", "normal", "special"):
            x, w = random_operands(rng, 3, 4, 41, dt, kind)
            part = lambda a, b, d: c_oracle.partial(a, b)
            assert pins.check_partition(part, c_oracle.combine, x, w, dt, rng) == []
    assert pins.check_combine_exact(c_oracle.combine, rng) == []
    assert pins.check_combine_exact(oracle.combine, rng) == []


def test_swap_and_negation():
    rng = np.random.default_rng(7)
    for dt in ("f32", "bf16"):
        x, w = random_operands(rng, 4, 5, 30, dt, "wide")
        y = oracle.gemm(x, w, dt)
        assert np.array_equal(oracle.gemm(w, x, dt), y.T)
        sign = np.uint32(0x80000000) if dt == "f32" else np.uint16(0x8000)
        yn = oracle.gemm(x ^ sign, w, dt)
        nz = (y & 0x7FFFFFFF) != 0
        assert np.array_equal(yn[nz], y[nz] ^ np.uint32(0x80000000))
        d = oracle.partial(x, w, dt)
        assert np.array_equal(oracle.partial(x ^ sign, w, dt), -d)


def test_power_of_two_scaling():
    # scaling x by 2^5 scales the exact sum by 2^5; away from the subnormal and
    # overflow ranges the rounded result scales exactly too
    rng = np.random.default_rng(8)
    x, w = random_operands(rng, 4, 4, 25, "f32", "normal")
    xs = (x.view(np.float32) * np.float32(32)).view(np.uint32)
    y = oracle.gemm(x, w, "f32").view(np.float32)
    ys = oracle.gemm(xs, w, "f32").view(np.float32)
    assert np.array_equal(ys, y * np.float32(32))


def test_bf16_equals_widened_f32():
    rng = np.random.default_rng(9)
    for kind in KINDS:
        xb, wb = random_operands(rng, 3, 3, 33, "bf16", kind)
        xf = (xb.astype(np.uint32) << 16)
        wf = (wb.astype(np.uint32) << 16)
        assert np.array_equal(oracle.partial(xb, wb, "bf16"), oracle.partial(xf, wf, "f32"))


def test_digit_structure():
    rng = np.random.default_rng(10)
    for dt in ("f32", "bf16"):
        x, w = random_operands(rng, 3, 3, 64, dt, "wide")
        d = oracle.partial(x, w, dt)
        assert np.all(np.abs(d) <= 64 * (2 ** 32 - 1))
        sign_mask = 0x7FFFFFFF if dt == "f32" else 0x7FFF
        d = oracle.partial(x & sign_mask, w & sign_mask, dt)
        assert np.all(d >= 0)
        x1, w1 = random_operands(rng, 20, 20, 1, dt, "wide")
        d1 = oracle.partial(x1, w1, dt)
        assert np.count_nonzero(d1, axis=-1).max() <= (3 if dt == "f32" else 2)


def test_accuracy_against_fp64_matmul():
    # the page's accuracy claim ("Correctness"): the result is the exact sum
    # rounded once, so against an fp64 matmul it sits at the fp32 rounding floor
    rng = np.random.default_rng(12)
    M, N, K = 16, 16, 512
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((N, K), dtype=np.float32)
    y = c_oracle.gemm(f32_bits(x), f32_bits(w)).view(np.float32).astype(np.float64)
    y64 = x.astype(np.float64) @ w.astype(np.float64).T
    absdot = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    gam = K * 2.0 ** -53 / (1 - K * 2.0 ** -53)
    bound = 2.0 ** -24 * np.abs(y64) + 2 * gam * absdot + 2.0 ** -150
    assert np.all(np.abs(y - y64) <= bound)
    rel = np.max(np.abs(y - y64) / np.abs(y64))
    assert rel <= 2.0 ** -24 * 1.0001


def test_c_oracle_matches_python_oracle():
    rng = np.random.default_rng(13)
    for kind in KINDS:
        for dt in ("f32", "bf16"):
            x, w = random_operands(rng, 7, 6, 45, dt, kind)
            dp = oracle.partial(x, w, dt)
            dc = c_oracle.partial(x, w, nthreads=3)
            assert np.array_equal(dp, dc), (kind, dt)
            assert np.array_equal(oracle.finalize(dp), c_oracle.finalize(dc))
            assert np.array_equal(oracle.gemm(x, w, dt), c_oracle.finalize(dc))
            rows = rng.integers(0, 7, size=9)
            cols = rng.integers(0, 6, size=9)
            assert np.array_equal(c_oracle.partial_pairs(x, w, rows, cols), dp[rows, cols])


def test_finalize_on_random_digit_arrays():
    # digit arrays that no GEMM of this size would give (large raw digits of
    # both signs, long carry chains): both finalizers agree with exact
    # rational rounding
    rng = np.random.default_rng(14)
    d = rng.integers(-(2 ** 52), 2 ** 52, size=(300, 18), dtype=np.int64)
    d[::3, 12:] = 0
    d[1::3, :6] = 0
    d[2::5, :] = np.where(rng.random((60, 18)) < 0.5, -(2 ** 32) + 1, 2 ** 32 - 1)
    d[::7, 17] = 0
    d[::11, 10:] = 0
    d[::11, :10] = rng.integers(-3, 4, size=(28, 10))
    yp = oracle.finalize(d)
    yc = c_oracle.finalize(d)
    assert np.array_equal(yp, yc)
    for row, y in zip(d, yp):
        S = Fraction(oracle.digits_value(row.tolist())) * Fraction(2) ** -298
        assert pins.is_correct_rounding(S, int(y)) == ""


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(15)
    v = np.concatenate([
        rng.standard_normal(5000).astype(np.float32),
        random_operands(rng, 1, 1, 3000, "f32", "wide")[0].view(np.float32).ravel(),
        # exact ties: bf16 values plus half a bf16 ulp
        ((rng.integers(0, 2 ** 16, 2000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 2.0 ** -149, -(2.0 ** -149), 3.3895e38, np.inf, -np.inf],
                 dtype=np.float32)])
    v = v[np.isfinite(v) | np.isinf(v)]
    v = v[~np.isnan(v)]
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_bits_to_bf16_bits(v.view(np.uint32))
    assert np.array_equal(got, want)


def test_validation_errors():
    x = np.zeros((2, 3), dtype=np.uint32)
    with pytest.raises(ValueError):
        oracle.partial(x, np.zeros((2, 4), dtype=np.uint32), "f32")
    with pytest.raises(ValueError):
        oracle.partial(x, np.zeros((2, 3), dtype=np.uint16), "f32")
    bad = x.copy()
    bad[1, 2] = 0x7F800000
    with pytest.raises(ValueError):
        oracle.partial(bad, x, "f32")
    with pytest.raises(ValueError):
        c_oracle.partial(bad, x)
    big = np.zeros((1, oracle.K_MAX + 1), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.partial(big, big, "bf16")
    with pytest.raises(ValueError):
        c_oracle.partial(big, big)
    with pytest.raises(ValueError):
        oracle.combine([])
    a = np.full((1, 18), 2 ** 62, dtype=np.int64)
    with pytest.raises(ValueError):
        oracle.combine([a, a])
    with pytest.raises(ValueError):
        c_oracle.combine([a, a])


def test_rne_fraction_matches_ieee_casts():
    # the rational rounding the loss-gradient reference uses, against numpy's
    # IEEE binary32 cast of exactly representable binary64 values: normals,
    # subnormals, halfway ties, values that overflow, and exact zero
    rng = np.random.default_rng(71)
    vals = [0.0, 2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -151, 2.0 ** -126 * (1 - 2.0 ** -30),
            float(np.finfo(np.float32).max), float(np.finfo(np.float32).max) * (1 + 2.0 ** -25),
            float(np.finfo(np.float32).max) * (1 + 2.0 ** -24), 2.0 ** 128, 1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24]
    vals += list(rng.standard_normal(2000) * 2.0 ** rng.integers(-160, 130, 2000))
    for v in vals:
        for s in (1, -1):
            x = s * v
            want = np.float32(x)
            got = pins.rne_fraction(Fraction(x), 24)
            assert float(got) == float(want) and (np.signbit(want) == (x < 0) or want == 0), x
    # bfloat16: 8-bit significand, against torch's CPU cast of float32 values
    import torch
    f = (rng.standard_normal(3000) * 2.0 ** rng.integers(-135, 128, 3000)).astype(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f).to(torch.bfloat16).float().numpy()
    for x, w in zip(f.tolist(), want.tolist()):
        assert float(pins.rne_fraction(Fraction(x), 8)) == w, x
