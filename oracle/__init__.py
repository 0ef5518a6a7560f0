"""Plain, slow CPU oracle for the exact long-accumulator GEMM.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call, link or run anything in
this package.  The product path (the HIP library and its Python binding) never
touches it, and this package imports nothing from the product.

What it computes follows the det-train page ("Method" section): every product
x[m,k]*w[n,k] is exact, its base-2^32 limbs are added into a per-output array of
signed int64 digits (a Kulisch long accumulator), and the exact sum is rounded
once to fp32.  Two implementations live here:

* ``exact``  -- Python integers, the definition written out; small cases only.
* ``c_oracle`` -- the same definition in plain C (``exact_oracle.c``), threaded
  over outputs, for the large configurations and the CPU baseline.

Parity status: every function is pinned by the tests in ``tests/test_oracle*.py``
against exact rational brute force, closed forms, library rounding routines and
invariants; none is "parity unpinned".
"""

from .exact import (  # noqa: F401
    NUM_DIGITS,
    LSB_EXP,
    K_MAX,
    decode,
    partial,
    partial_one,
    exact_sums,
    combine,
    finalize,
    gemm,
    digits_value,
    round_binary,
    f32_bits_to_bf16_bits,
)
