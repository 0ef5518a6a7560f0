"""Plant plausible mistakes in the C oracle's combine (CPU only) and check that
the pins catch each one.

Each mutation is a one-line text change to a copy of oracle/exact_oracle.c,
compiled with gcc into a temporary library; the unmutated copy must pass.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from tests import pins
from workloads import random_operands

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "exact_oracle.c")

MUTATIONS = {
    "none": None,
    "last part dropped": ("for (int p = 0; p < nparts; ++p)", "for (int p = 0; p < nparts - 1; ++p)"),
    "first part dropped": ("for (int p = 0; p < nparts; ++p)", "for (int p = 1; p < nparts; ++p)"),
    "last value skipped": ("for (long i = 0; i < nvals; ++i) {\n    int64_t acc",
                           "for (long i = 0; i + 1 < nvals; ++i) {\n    int64_t acc"),
    "parts subtracted": ("__builtin_add_overflow(acc, parts[p][i], &acc)",
                         "__builtin_sub_overflow(acc, parts[p][i], &acc)"),
}


def _build(tmp_path, name, mutation):
    src = open(SRC).read()
    if mutation is not None:
        old, new = mutation
        assert src.count(old) == 1, f"mutation site for {name!r} not unique"
        src = src.replace(old, new)
    c = tmp_path / "oracle_mut.c"
    c.write_text(src)
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(so), str(c)], check=True)
    lib = ctypes.CDLL(str(so))
    vp = ctypes.c_void_p
    lib.oracle_combine.argtypes = [vp, ctypes.c_int, ctypes.c_long, vp]
    lib.oracle_partial_full.argtypes = [ctypes.c_int, vp, ctypes.c_long, vp, ctypes.c_long, ctypes.c_long,
                                        ctypes.c_long, ctypes.c_long, vp, ctypes.c_int]

    def combine(parts):
        arrs = [np.ascontiguousarray(p, dtype=np.int64) for p in parts]
        ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
        out = np.full_like(arrs[0], 12345)          # anything the combine fails to write shows
        assert lib.oracle_combine(ptrs, len(arrs), out.size, out.ctypes.data) == 0
        return out

    def partial(x, w, dt):
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w)
        M, K = x.shape
        out = np.empty((M, w.shape[0], 18), dtype=np.int64)
        assert lib.oracle_partial_full(0 if x.dtype == np.uint32 else 1, x.ctypes.data, K, w.ctypes.data, K,
                                       M, w.shape[0], K, out.ctypes.data, 1) == 0
        return out
    return partial, combine


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_combine_mutation_is_caught(tmp_path, name):
    partial, combine = _build(tmp_path, name, MUTATIONS[name])
    rng = np.random.default_rng(5)
    x, w = random_operands(rng, 2, 3, 30, "f32", "wide")
    fails = pins.check_combine_exact(combine, rng) + pins.check_partition(partial, combine, x, w, "f32", rng)
    if name == "none":
        assert fails == []
    else:
        assert fails, f"no pin caught the C oracle mutation {name!r}"
