"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch each one, so that a passing pin suite says something.

Each mutation patches one function of ``oracle.exact`` for the duration of a
test (pytest's monkeypatch restores it).
"""
import numpy as np
import pytest

import oracle.exact as ex
from tests import pins
from tests.test_oracle import tiny_cases
from workloads import random_operands


def _run(check, *args):
    try:
        return check(*args)
    except Exception as e:           # a pin that makes the oracle raise caught it too
        return [f"{check.__name__} raised {type(e).__name__}: {e}"]


def all_pin_failures():
    rng = np.random.default_rng(3)
    x1, w1 = random_operands(rng, 60, 50, 1, "f32", "wide")
    xp, wp = random_operands(rng, 2, 3, 20, "f32", "wide")
    fails = []
    fails += _run(pins.check_golden_digits, ex.partial, ex.finalize)
    fails += _run(pins.check_golden_rounding, ex.gemm)
    fails += _run(pins.check_golden_rounding, lambda x, w, dt: ex.finalize(ex.partial(x, w, dt)))
    fails += _run(pins.check_fraction, ex.partial, ex.gemm, ex.digits_value, tiny_cases(n=2))
    fails += _run(pins.check_k1_numpy, ex.gemm, x1[:, 0], w1[:, 0])
    fails += _run(pins.check_integer_exact, ex.gemm, np.random.default_rng(4))
    fails += _run(pins.check_partition, ex.partial, ex.combine, xp, wp, "f32", rng)
    return fails


def test_unmutated_oracle_passes_every_pin():
    assert all_pin_failures() == []


def _round_ties_away(I, scale, fmt):
    p, ebits = fmt
    bias = (1 << (ebits - 1)) - 1
    if I == 0:
        return 0
    sign = 1 if I < 0 else 0
    A = abs(I)
    top = A.bit_length() - 1 + scale
    ulp = max(top - (p - 1), 1 - bias - (p - 1))
    q = ulp - scale
    if q <= 0:
        r = A << (-q)
    else:
        r = A >> q
        if A - (r << q) >= (1 << (q - 1)):     # mistake: ties away from zero
            r += 1
    if r == (1 << p):
        r >>= 1
        ulp += 1
    if r < (1 << (p - 1)):
        mag = r
    else:
        b = ulp + (p - 1) + bias
        mag = (((1 << ebits) - 1) << (p - 1)) if b >= (1 << ebits) - 1 else (b << (p - 1)) | (r - (1 << (p - 1)))
    return (sign << (ebits + p - 1)) | mag


def _flush_subnormal_outputs(I, scale, fmt):
    bits = ORIG_ROUND(I, scale, fmt)
    if (bits & 0x7F800000) == 0:                # mistake: flush-to-zero
        return bits & 0x80000000
    return bits


def _overflow_one_late(I, scale, fmt):
    bits = ORIG_ROUND(I, scale, fmt)
    if (bits & 0x7FFFFFFF) == 0x7F800000 and abs(I) < (1 << (128 + 298)):
        return (bits & 0x80000000) | 0x7F7FFFFF  # mistake: threshold at 2^128
    return bits


def _decode_subnormal_off(bits, dtype):
    s, m, e = ORIG_DECODE(bits, dtype)
    if dtype == "f32" and ((bits >> 23) & 0xFF) == 0:
        e -= 1                                  # mistake: subnormal exponent -150
    return s, m, e


def _decode_no_hidden_bit(bits, dtype):
    s, m, e = ORIG_DECODE(bits, dtype)
    if dtype == "f32" and ((bits >> 23) & 0xFF) != 0:
        m &= 0x7FFFFF                           # mistake: hidden bit dropped
    return s, m, e


def _partial_one_unsigned(xrow, wrow):
    xs = [(0, m, e) for (_, m, e) in xrow]      # mistake: product sign dropped
    return ORIG_PARTIAL_ONE(xs, wrow)


def _partial_one_last_dropped(xrow, wrow):
    return ORIG_PARTIAL_ONE(xrow[:-1], wrow[:-1])   # mistake: last k skipped


def _partial_one_w_reversed(xrow, wrow):
    return ORIG_PARTIAL_ONE(xrow, list(wrow)[::-1])  # mistake: w indexed backwards


def _partial_one_carry_normalised(xrow, wrow):
    d = ORIG_PARTIAL_ONE(xrow, wrow)
    carry = 0                                   # mistake: digits carried (not raw)
    out = []
    for v in d:
        v += carry
        out.append(v & 0xFFFFFFFF)
        carry = v >> 32
    out[-1] += carry << 32
    return out


def _exact_sums_off_by_one(x, w, dt):
    return [[I * 2 for I in row] for row in ORIG_EXACT(x, w, dt)]   # mistake: LSB 2^-297


ORIG_ROUND = ex.round_binary
ORIG_DECODE = ex.decode
ORIG_PARTIAL_ONE = ex.partial_one
ORIG_EXACT = ex.exact_sums

MUTATIONS = {
    "ties away from zero": ("round_binary", _round_ties_away),
    "flush subnormal outputs": ("round_binary", _flush_subnormal_outputs),
    "overflow threshold at 2^128": ("round_binary", _overflow_one_late),
    "subnormal input exponent off by one": ("decode", _decode_subnormal_off),
    "hidden bit dropped": ("decode", _decode_no_hidden_bit),
    "product sign dropped": ("partial_one", _partial_one_unsigned),
    "last product dropped": ("partial_one", _partial_one_last_dropped),
    "w read backwards": ("partial_one", _partial_one_w_reversed),
    "digits carried instead of raw": ("partial_one", _partial_one_carry_normalised),
    "digit weight off by one bit": ("exact_sums", _exact_sums_off_by_one),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ex, attr, fn)
    assert all_pin_failures() != [], f"no pin caught: {name}"
