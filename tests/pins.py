"""Checks that pin the oracle to facts other than itself.

Each ``check_*`` function takes the oracle functions it exercises as
arguments, so the same check can run against the real oracle and against a
deliberately broken copy (tests/test_oracle_mutations.py) to show that the pin
would catch that mistake.  Each returns a list of failure messages (empty when
the pin holds).

Facts used: exact rational arithmetic (``fractions.Fraction``), numpy's IEEE
fp64 multiply and fp64->fp32 cast, mpmath's correctly rounded 24-bit rounding,
closed forms, and the hand-derived fixtures in tests/golden/.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction
from typing import Callable, List

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
LSB_EXP = -298
F32_MAX = Fraction(2 ** 24 - 1) * Fraction(2) ** 104
F32_OVERFLOW_TIE = Fraction(2) ** 128 - Fraction(2) ** 103   # rounds to inf at or above


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def hexbits(vals, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.array([int(v, 16) for v in vals], dtype=np.uint32)
    return np.array([int(v, 16) for v in vals], dtype=np.uint16)


def bits_to_fraction(bits: int, dtype: str) -> Fraction:
    """Exact value of a bit pattern via numpy's own float conversion."""
    if dtype == "f32":
        v = np.array([bits], dtype=np.uint32).view(np.float32)[0]
    else:
        v = np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(v))


def f32_from_bits(b: int) -> np.float32:
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


def is_correct_rounding(S: Fraction, ybits: int) -> str:
    """'' if ybits is the binary32 round-to-nearest-even of S, else a reason.

    Checked by comparing against the neighbouring floats (numpy nextafter),
    independent of any rounding code under test."""
    y = f32_from_bits(ybits)
    if S == 0:
        return "" if ybits == 0 else f"exact zero must give +0, got {ybits:08x}"
    neg = S < 0
    if bool(ybits >> 31) != neg:
        return f"sign of {ybits:08x} differs from the sign of the exact sum"
    A = -S if neg else S
    if A >= F32_OVERFLOW_TIE:
        return "" if (ybits & 0x7FFFFFFF) == 0x7F800000 else "must overflow to inf"
    if not np.isfinite(y):
        return "overflowed although below the overflow threshold"
    Y = abs(Fraction(float(y)))
    up = np.nextafter(np.float32(abs(y)), np.float32(np.inf), dtype=np.float32)
    dn = np.nextafter(np.float32(abs(y)), np.float32(0), dtype=np.float32) if Y > 0 else None
    err = abs(A - Y)
    if np.isfinite(up):
        e_up = abs(A - Fraction(float(up)))
        if e_up < err:
            return "the next float up is nearer"
        if e_up == err and (ybits & 1):
            return "tie not broken to the even significand"
    elif A > Y:
        # y is max finite: only the overflow threshold can push it up
        pass
    if dn is not None:
        e_dn = abs(A - Fraction(float(dn)))
        if e_dn < err:
            return "the next float down is nearer"
        if e_dn == err and (ybits & 1):
            return "tie not broken to the even significand"
    if Y == 0:
        # zero result: A must be at most half the smallest subnormal
        half_min = Fraction(2) ** -150
        if A > half_min:
            return "rounded to zero although above half the smallest subnormal"
    return ""


def exact_dot(xbits, wbits, dtype: str) -> Fraction:
    return sum((bits_to_fraction(int(a), dtype) * bits_to_fraction(int(b), dtype)
                for a, b in zip(xbits, wbits)), Fraction(0))


# ---------------------------------------------------------------- pins

def check_golden_digits(partial: Callable, finalize: Callable) -> List[str]:
    """P4: hand-derived digit arrays and their finalized bits."""
    fails = []
    for case in load_golden("digits.json")["cases"]:
        dt = case["dtype"]
        x = hexbits(case["x"], dt).reshape(1, -1)
        w = hexbits(case["w"], dt).reshape(1, -1)
        d = partial(x, w, dt)[0, 0]
        want = np.zeros(18, dtype=np.int64)
        for j, v in case["digits"].items():
            want[int(j)] = v
        if not np.array_equal(d, want):
            fails.append(f"digits {case['why'][:40]}: got {d.tolist()}")
        y = int(finalize(d.reshape(1, 18))[0])
        if y != int(case["y"], 16):
            fails.append(f"finalize {case['why'][:40]}: got {y:08x} want {case['y']}")
    return fails


def check_golden_rounding(gemm: Callable) -> List[str]:
    """P5: closed-form rounding boundaries."""
    fails = []
    for case in load_golden("rounding.json")["cases"]:
        dt = case.get("dtype", "f32")
        x = hexbits(case["x"], dt).reshape(1, -1)
        w = hexbits(case["w"], dt).reshape(1, -1)
        y = int(gemm(x, w, dt)[0, 0])
        if y != int(case["y"], 16):
            fails.append(f"{case['why'][:50]}: got {y:08x} want {case['y']}")
    return fails


def check_fraction(partial: Callable, gemm: Callable, digits_value: Callable,
                   cases) -> List[str]:
    """P1: digit value equals the exact rational sum; y is correctly rounded."""
    fails = []
    for x, w, dt in cases:
        d = partial(x, w, dt)
        y = gemm(x, w, dt)
        for m in range(x.shape[0]):
            for n in range(w.shape[0]):
                S = exact_dot(x[m], w[n], dt)
                I = digits_value(d[m, n].tolist())
                if Fraction(I) * Fraction(2) ** LSB_EXP != S:
                    fails.append(f"digit value != exact sum at ({m},{n}) {dt}")
                why = is_correct_rounding(S, int(y[m, n]))
                if why:
                    fails.append(f"({m},{n}) {dt}: {why}")
    return fails


def check_k1_numpy(gemm: Callable, xbits: np.ndarray, wbits: np.ndarray) -> List[str]:
    """P2: with K = 1 the result is one rounding of the exact fp64 product,
    which numpy computes (fp64 multiply of fp32 values is exact) and casts."""
    x = xbits.view(np.float32).astype(np.float64)
    w = wbits.view(np.float32).astype(np.float64)
    with np.errstate(over="ignore"):            # products beyond fp32 cast to inf
        want = (x[:, None] * w[None, :]).astype(np.float32).view(np.uint32)
    got = gemm(xbits.reshape(-1, 1), wbits.reshape(-1, 1), "f32")
    bad = np.argwhere(got != want)
    # numpy gives -0.0 for a negative product that is an exact -0 (a zero
    # operand); the accumulator's exact zero is +0.  Only that case may differ.
    fails = []
    for m, n in bad:
        if want[m, n] == 0x80000000 and got[m, n] == 0 and (x[m] == 0 or w[n] == 0):
            continue
        fails.append(f"K=1 ({m},{n}): got {got[m, n]:08x} want {want[m, n]:08x}")
    return fails


def check_integer_exact(gemm: Callable, rng: np.random.Generator) -> List[str]:
    """P3: small integers make every fp64 partial sum exact, so numpy's fp64
    matmul cast to fp32 is the correctly rounded result; closed forms."""
    fails = []
    for (M, N, K) in [(3, 4, 1), (5, 3, 17), (4, 4, 200)]:
        x = rng.integers(-1024, 1025, size=(M, K)).astype(np.float32)
        w = rng.integers(-1024, 1025, size=(N, K)).astype(np.float32)
        want = (x.astype(np.float64) @ w.astype(np.float64).T).astype(np.float32)
        want_bits = want.view(np.uint32).copy()
        want_bits[want == 0] = 0          # exact zero is +0
        got = gemm(x.view(np.uint32), w.view(np.uint32), "f32")
        if not np.array_equal(got, want_bits):
            fails.append(f"integer-exact {M}x{N}x{K} differs")
    # closed forms: ones -> K; x_k = k+1, w = 1 -> K(K+1)/2 rounded to nearest even
    for K in (1, 7, 300, 5000):
        ones = np.ones((1, K), dtype=np.float32).view(np.uint32)
        got = int(gemm(ones, ones, "f32")[0, 0])
        if got != int(np.float32(K).view(np.uint32)):
            fails.append(f"sum of {K} ones")
        ar = np.arange(1, K + 1, dtype=np.float32).reshape(1, K).view(np.uint32)
        tri = K * (K + 1) // 2
        want = np.float32(float(tri))     # exact integer -> fp32 nearest-even (numpy)
        got = int(gemm(ar, ones, "f32")[0, 0])
        if got != int(want.view(np.uint32)):
            fails.append(f"triangular number K={K}: got {got:08x} want {int(want.view(np.uint32)):08x}")
    return fails


def check_mpmath(gemm: Callable, cases) -> List[str]:
    """P8: mpmath rounding to 24 bits (nearest) agrees for normal-range sums."""
    import mpmath
    from mpmath.libmp import from_rational, round_nearest
    fails = []
    for x, w, dt in cases:
        y = gemm(x, w, dt)
        for m in range(x.shape[0]):
            for n in range(w.shape[0]):
                S = exact_dot(x[m], w[n], dt)
                if S == 0:
                    continue
                A = abs(S)
                if not (Fraction(2) ** -126 <= A < Fraction(2) ** 127):
                    continue
                # one correctly rounded division at 24 bits, ties to even
                r = mpmath.mpf(from_rational(S.numerator, S.denominator, 24, round_nearest))
                want = np.float32(float(r))
                if int(want.view(np.uint32)) != int(y[m, n]):
                    fails.append(f"mpmath ({m},{n}) {dt}")
    return fails


def check_partition(partial: Callable, combine: Callable, x, w, dt, rng) -> List[str]:
    """P6: K permutation and any K partition with any fold order give the same
    raw digits (the page's invariance claim, 'Method' and 'Correctness')."""
    fails = []
    whole = partial(x, w, dt)
    K = x.shape[1]
    perm = rng.permutation(K)
    if not np.array_equal(partial(x[:, perm], w[:, perm], dt), whole):
        fails.append("K permutation changed the digits")
    for nshards in (2, 3, 5):
        if K < nshards:
            continue
        cuts = sorted(rng.choice(np.arange(1, K), nshards - 1, replace=False).tolist())
        edges = [0] + cuts + [K]
        parts = [partial(x[:, a:b], w[:, a:b], dt) for a, b in zip(edges[:-1], edges[1:])]
        order = rng.permutation(len(parts))
        acc = parts[order[0]]
        for i in order[1:]:
            acc = combine([acc, parts[i]])
        if not np.array_equal(acc, whole):
            fails.append(f"{nshards}-way partition changed the digits")
        if not np.array_equal(combine(parts), whole):
            fails.append(f"{nshards}-way n-ary combine changed the digits")
    return fails


def check_combine_exact(combine: Callable, rng) -> List[str]:
    """a6 (det-train page, "Method": partials of disjoint K ranges add digit by
    digit): combine is the element-wise sum of all its parts.  Checked against
    Python integers, which cannot wrap, for 1 to 40 parts of both signs and
    several shapes, including a part count that is not a power of two and
    arrays whose length is odd."""
    fails = []
    for nparts, shape in [(1, (2, 3, 18)), (2, (1, 18)), (3, (5, 18)), (7, (3, 1, 18)),
                          (16, (2, 2, 18)), (33, (1, 18)), (40, (4, 18))]:
        parts = [rng.integers(-(2 ** 56), 2 ** 56, size=shape, dtype=np.int64) for _ in range(nparts)]
        parts[0].flat[0] = 2 ** 56 - 1                  # extremes of the drawn range
        parts[-1].flat[-1] = -(2 ** 56)
        got = combine(parts)
        if got.shape != parts[0].shape or got.dtype != np.int64:
            fails.append(f"{nparts} parts: result shape {got.shape} dtype {got.dtype}")
            continue
        want = [sum(int(p.flat[i]) for p in parts) for i in range(parts[0].size)]
        if [int(v) for v in got.reshape(-1)] != want:
            fails.append(f"{nparts} parts of shape {shape}: digit sums differ from the integer sums")
    return fails


def rne_fraction(v: Fraction, p: int, emin: int = -126, emax: int = 127):
    """The exact rational v rounded to the nearest binary float with a p-bit
    significand (ties to even), gradual underflow below 2^emin, and values that
    round to 2^(emax+1) or more returned as +-inf (a float); otherwise a
    Fraction.  p = 24 is binary32, p = 8 bfloat16 (both emin -126, emax 127)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = emin
    if a >= Fraction(2) ** emin:                         # a in [2^e, 2^(e+1))
        e = a.numerator.bit_length() - a.denominator.bit_length() - 1
        while Fraction(2) ** (e + 1) <= a:
            e += 1
        while Fraction(2) ** e > a:
            e -= 1
    ulp = Fraction(2) ** (e - (p - 1))
    q = a / ulp
    r = q.numerator // q.denominator
    rem = q - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    out = r * ulp
    if out >= Fraction(2) ** (emax + 1):
        return float("inf") if v > 0 else float("-inf")
    return out if v > 0 else -out
