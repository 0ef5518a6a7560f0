"""Exact long-accumulator GEMM, written out with Python integers.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source: the det-train page, "Method" section (digits, limbs, exact products,
one rounding to fp32), "Usage" section (x is [M, K], w is [N, K], K-slices
compose) and "Requirements and limits" section (K <= 2^19, bf16 and f32).

Readings of points the page leaves open:

* Digit layout: 18 signed int64 digits, digit j weighs 2^(32*j - 298).  Every
  fp32 (or bf16) product lies in [2^-298, 2^256); 18*32 = 576 bits leave 19+
  bits of headroom, enough for K = 2^19 products.
* Raw digits: digit j is the sum over products of (sign) * (bits [32j, 32j+32)
  of |product| / 2^-298).  No carries are taken before rounding, so digit
  arrays of K-slices add up digit for digit to the digit array of the whole.
* Rounding: IEEE 754 binary32 round-to-nearest-ties-to-even, with gradual
  underflow, overflow to +-inf, +0.0 for an exact zero, and the sign kept when a
  nonzero sum rounds to zero (so a tiny negative sum gives -0.0).
* Inputs that are Inf or NaN are rejected (the digits cannot hold them).
"""

from __future__ import annotations

from typing import Iterable, List, Sequence, Tuple

import numpy as np

NUM_DIGITS = 18          # digits per output
DIGIT_BITS = 32          # radix 2^32
LSB_EXP = -298           # digit 0 weighs 2^-298 = (2^-149)^2, the smallest product
K_MAX = 1 << 19          # largest K per call ("Requirements and limits")
INT64_MIN = -(1 << 63)
INT64_MAX = (1 << 63) - 1

# binary formats as (significand bits p incl. the hidden bit, exponent bits)
F32_FORMAT = (24, 8)
BF16_FORMAT = (8, 8)


def decode(bits: int, dtype: str) -> Tuple[int, int, int]:
    """Split one fp32 or bf16 bit pattern into (sign, m, ex).

    The value is (-1)^sign * m * 2^ex with m an integer: for normal numbers m
    carries the hidden bit, subnormals keep their raw fraction and the smallest
    exponent, so nothing is flushed.  Inf and NaN raise ValueError.
    """
    if dtype == "f32":
        sign = (bits >> 31) & 1
        e = (bits >> 23) & 0xFF
        f = bits & 0x7FFFFF
        if e == 0xFF:
            raise ValueError("non-finite f32 input (Inf or NaN) is not accepted")
        if e == 0:
            return sign, f, -149
        return sign, f | (1 << 23), e - 150
    if dtype == "bf16":
        sign = (bits >> 15) & 1
        e = (bits >> 7) & 0xFF
        f = bits & 0x7F
        if e == 0xFF:
            raise ValueError("non-finite bf16 input (Inf or NaN) is not accepted")
        if e == 0:
            return sign, f, -133
        return sign, f | (1 << 7), e - 134
    raise ValueError(f"unsupported dtype {dtype!r}")


def _check_operands(x_bits: np.ndarray, w_bits: np.ndarray, dtype: str) -> None:
    want = np.uint32 if dtype == "f32" else np.uint16
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unsupported dtype {dtype!r}")
    if x_bits.dtype != want or w_bits.dtype != want:
        raise ValueError(f"{dtype} operands must be given as {np.dtype(want).name} bit patterns")
    if x_bits.ndim != 2 or w_bits.ndim != 2 or x_bits.shape[1] != w_bits.shape[1]:
        raise ValueError("x must be [M, K] and w must be [N, K] with the same K")
    if x_bits.shape[1] > K_MAX:
        raise ValueError(f"K = {x_bits.shape[1]} exceeds the limit 2^19")


def _decode_rows(a: np.ndarray, dtype: str) -> List[List[Tuple[int, int, int]]]:
    return [[decode(int(b), dtype) for b in row] for row in a.tolist()]


def partial_one(xrow: Sequence[Tuple[int, int, int]],
                wrow: Sequence[Tuple[int, int, int]]) -> List[int]:
    """Raw digits of one output from decoded rows x[m, :] and w[n, :].

    For each k: the exact product is (-1)^s * M * 2^e with M = m_x*m_w and
    e = ex + ew >= -298.  Its offset o = e + 298 picks digit d = o // 32 and
    shift o % 32; T = M * 2^(o % 32) is cut into base-2^32 limbs and limb i is
    added, with the product's sign, into digit d + i.
    """
    digits = [0] * NUM_DIGITS
    for (sx, mx, ex), (sw, mw, ew) in zip(xrow, wrow):
        M = mx * mw
        if M == 0:
            continue
        o = ex + ew - LSB_EXP
        d, s = divmod(o, DIGIT_BITS)
        T = M << s
        neg = sx ^ sw
        i = 0
        while T:
            limb = T & 0xFFFFFFFF
            if limb:
                if d + i >= NUM_DIGITS:
                    raise AssertionError("product outside the digit range")
                digits[d + i] += -limb if neg else limb
            T >>= DIGIT_BITS
            i += 1
    return digits


def partial(x_bits: np.ndarray, w_bits: np.ndarray, dtype: str) -> np.ndarray:
    """det_gemm_partial: raw digits, int64 array of shape [M, N, 18]."""
    _check_operands(x_bits, w_bits, dtype)
    xs = _decode_rows(x_bits, dtype)
    ws = _decode_rows(w_bits, dtype)
    out = np.zeros((len(xs), len(ws), NUM_DIGITS), dtype=np.int64)
    for m, xrow in enumerate(xs):
        for n, wrow in enumerate(ws):
            out[m, n, :] = partial_one(xrow, wrow)
    return out


def exact_sums(x_bits: np.ndarray, w_bits: np.ndarray, dtype: str) -> List[List[int]]:
    """The exact sum of each output as an integer I, value = I * 2^-298.

    Computed straight from the definition (sum of signed exact products),
    without digits, so it checks the digit bookkeeping independently.
    """
    _check_operands(x_bits, w_bits, dtype)
    xs = _decode_rows(x_bits, dtype)
    ws = _decode_rows(w_bits, dtype)
    res = []
    for xrow in xs:
        row = []
        for wrow in ws:
            acc = 0
            for (sx, mx, ex), (sw, mw, ew) in zip(xrow, wrow):
                p = (mx * mw) << (ex + ew - LSB_EXP)
                acc += -p if (sx ^ sw) else p
            row.append(acc)
        res.append(row)
    return res


def digits_value(digits: Iterable[int]) -> int:
    """The integer sum_j digit_j * 2^(32 j) (value in units of 2^-298)."""
    return sum(int(d) << (DIGIT_BITS * j) for j, d in enumerate(digits))


def combine(parts: Sequence[np.ndarray]) -> np.ndarray:
    """det_combine: digit-wise integer sum of digit arrays of equal shape.

    Sums are taken with Python integers and must fit int64 (else ValueError).
    """
    if len(parts) == 0:
        raise ValueError("combine needs at least one digit array")
    shape = parts[0].shape
    if shape[-1:] != (NUM_DIGITS,):
        raise ValueError("digit arrays must end in a dimension of 18")
    for p in parts:
        if p.shape != shape or p.dtype != np.int64:
            raise ValueError("digit arrays must be int64 and of equal shape")
    total = np.zeros(shape, dtype=object)
    for p in parts:
        total = total + p.astype(object)
    flat = total.reshape(-1)
    for v in flat:
        if v < INT64_MIN or v > INT64_MAX:
            raise ValueError("combined digit leaves the int64 range")
    return total.astype(np.int64)


def round_binary(I: int, scale: int, fmt: Tuple[int, int]) -> int:
    """Round I * 2^scale to the nearest binary float (ties to even).

    ``fmt`` = (p, ebits): p significand bits including the hidden bit.  Returns
    the bit pattern.  Gradual underflow; a result at or above 2^(emax+1) after
    rounding is +-inf; zero gives +0; a nonzero value keeps its sign.
    """
    p, ebits = fmt
    bias = (1 << (ebits - 1)) - 1
    emin = 1 - bias
    sign_shift = ebits + p - 1
    if I == 0:
        return 0
    sign = 1 if I < 0 else 0
    A = -I if I < 0 else I
    top = A.bit_length() - 1 + scale            # value in [2^top, 2^(top+1))
    ulp = max(top - (p - 1), emin - (p - 1))    # exponent of the last kept bit
    q = ulp - scale                             # low bits of A to drop
    if q <= 0:
        r = A << (-q)
    else:
        r = A >> q
        rem = A - (r << q)
        half = 1 << (q - 1)
        if rem > half or (rem == half and (r & 1)):
            r += 1
    if r == (1 << p):
        r >>= 1
        ulp += 1
    if r < (1 << (p - 1)):                      # subnormal or zero
        mag = r
    else:
        biased = ulp + (p - 1) + bias
        if biased >= (1 << ebits) - 1:
            mag = ((1 << ebits) - 1) << (p - 1)  # infinity
        else:
            mag = (biased << (p - 1)) | (r - (1 << (p - 1)))
    return (sign << sign_shift) | mag


def finalize(digits: np.ndarray) -> np.ndarray:
    """det_finalize: round the value of each digit array once to fp32.

    Returns the fp32 bit patterns as uint32 with the leading shape of
    ``digits`` (everything but the last dimension of 18).
    """
    digits = np.asarray(digits)
    if digits.shape[-1:] != (NUM_DIGITS,):
        raise ValueError("digit arrays must end in a dimension of 18")
    flat = digits.reshape(-1, NUM_DIGITS).tolist()
    out = np.array([round_binary(digits_value(d), LSB_EXP, F32_FORMAT) for d in flat],
                   dtype=np.uint32)
    return out.reshape(digits.shape[:-1])


def gemm(x_bits: np.ndarray, w_bits: np.ndarray, dtype: str) -> np.ndarray:
    """det_gemm: exact sums rounded once to fp32, as uint32 bit patterns [M, N]."""
    sums = exact_sums(x_bits, w_bits, dtype)
    return np.array([[round_binary(I, LSB_EXP, F32_FORMAT) for I in row] for row in sums],
                    dtype=np.uint32).reshape(len(sums), w_bits.shape[0])


def f32_bits_to_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16, nearest with ties to even (uint32 -> uint16).

    Inf passes through as Inf; NaN is rejected.
    """
    flat = np.asarray(bits, dtype=np.uint32).reshape(-1).tolist()
    out = []
    for b in flat:
        e = (b >> 23) & 0xFF
        if e == 0xFF:
            if b & 0x7FFFFF:
                raise ValueError("NaN cannot be rounded to bf16 here")
            out.append(((b >> 31) << 15) | 0x7F80)
            continue
        s, m, ex = decode(b, "f32")
        r = round_binary(-m if s else m, ex, BF16_FORMAT)
        if r == 0 and s:
            r = 0x8000        # -0.0 stays -0.0
        out.append(r)
    return np.array(out, dtype=np.uint16).reshape(np.shape(bits))
