"""GPU parity of det_gemm's matrix-core path against the oracle, bit for bit.

The path forms the exact sum from int8 digit GEMMs when the rows of x and w
span few binades, and recomputes the rows and columns that do not fit on the
digit accumulator; either way the result must be the oracle's correctly
rounded exact sum.  The cases force the path (and the digit count S) so that
small shapes reach it, and cover ragged tiles, K past one 2^14 block, the
recomputed rows and columns (their counts checked against the rule stated in
include/detgemm.h), strided views, all-zero rows, and results that overflow,
underflow or round at ties."""
import threading

import numpy as np
import pytest
import torch

from oracle import c_oracle
from tests import pins
from tests.gpu_util import announce, f32_bits, mismatch_report, to_device
from workloads import f32_bits as np_f32_bits, random_operands, to_bf16_bits
import bitwise_deterministic_exact_amd as det

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _auto_path_after():
    yield
    det.set_gemm_path("auto", 0)


def _needs(bits: np.ndarray, dt: str) -> np.ndarray:
    """Digits each row needs: the least S with (top bit - lowest set bit + 1)
    <= 8S - 2 over the row's nonzero elements, 0 for an all-zero row."""
    b = bits.astype(np.int64)
    if dt == "f32":
        E, F, hid, bias = (b >> 23) & 0xFF, b & 0x7FFFFF, 1 << 23, 150
    else:
        E, F, hid, bias = (b >> 7) & 0xFF, b & 0x7F, 1 << 7, 134
    m = F | np.where(E > 0, hid, 0)
    ex = np.maximum(E, 1) - bias
    nz = m != 0
    mm = np.where(nz, m, 1)
    top = ex + np.floor(np.log2(mm)).astype(np.int64)
    low = ex + np.log2(mm & -mm).astype(np.int64)
    tops = np.where(nz, top, -10**6).max(axis=1)
    lows = np.where(nz, low, 10**6).min(axis=1)
    need = (tops - lows + 10) // 8
    return np.where(nz.any(axis=1), np.minimum(need, 8), 0)


def _run(xb, wb, dt, S, x=None, w=None):
    x = to_device(xb, dt) if x is None else x
    w = to_device(wb, dt) if w is None else w
    det.set_gemm_path("slices", S)
    y = f32_bits(det.det_gemm(x, w))
    return y, det.last_gemm_plan()


def _check(xb, wb, dt, S, label, **kw):
    announce(f"slices {label} {dt} S={S} M={xb.shape[0]} N={wb.shape[0]} K={xb.shape[1]}")
    got, plan = _run(xb, wb, dt, S, **kw)
    want = c_oracle.gemm(xb, wb)
    assert plan["path"] == "slices", plan
    if S:
        assert plan["slices"] == S, plan
        assert plan["fallback_rows"] == int((_needs(xb, dt) > S).sum()), plan
        assert plan["fallback_cols"] == int((_needs(wb, dt) > S).sum()), plan
    assert np.array_equal(got, want), mismatch_report(got, want)
    return plan


SHAPES = [(1, 1, 1), (5, 3, 7), (32, 32, 32), (33, 31, 63), (64, 128, 64), (70, 130, 100),
          (129, 65, 257), (200, 300, 96)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["normal", "uniform", "int"])
def test_forced_digits_ragged_shapes(kind, dt):
    rng = np.random.default_rng(500 + 3 * ["normal", "uniform", "int"].index(kind) + (dt == "bf16"))
    for i, (M, N, K) in enumerate(SHAPES):
        xb, wb = random_operands(rng, M, N, K, dt, kind)
        S = 2 + (i % 6)
        _check(xb, wb, dt, S, kind)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_every_digit_count_on_one_input(dt):
    rng = np.random.default_rng(520 + (dt == "bf16"))
    xb, wb = random_operands(rng, 96, 160, 200, dt, "normal")
    for S in range(2, 8):
        _check(xb, wb, dt, S, "normal")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rows_and_columns_recomputed(dt):
    # wide and special operands: most rows need more digits than S, so most of
    # y comes from the accumulator pass over the listed rows and columns
    rng = np.random.default_rng(530 + (dt == "bf16"))
    for kind in ("wide", "special"):
        xb, wb = random_operands(rng, 45, 77, 90, dt, kind)
        for S in (2, 7):
            _check(xb, wb, dt, S, kind)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_outlier_rows_and_columns(dt):
    # rows and columns with one tiny element planted need more digits than S
    # (f32 N(0,1) rows of 128 fit in 7 digits, bf16 ones in 4): those rows of
    # x and of w go to the accumulator
    rng = np.random.default_rng(540 + (dt == "bf16"))
    M, N, K = 150, 260, 128
    S = 7 if dt == "f32" else 4
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((N, K), dtype=np.float32)
    rows = rng.choice(M, 7, replace=False)
    cols = rng.choice(N, 11, replace=False)
    x[rows, rng.integers(0, K, rows.size)] = np.float32(3.0 * 2.0 ** -60)
    w[cols, rng.integers(0, K, cols.size)] = np.float32(-(2.0 ** -70))
    x[3, :] = 0.0                                   # an all-zero row
    w[5, :] = 0.0                                   # an all-zero column
    conv = np_f32_bits if dt == "f32" else to_bf16_bits
    xb, wb = conv(x), conv(w)
    nx, nw = _needs(xb, dt), _needs(wb, dt)
    assert nx[3] == 0 and nw[5] == 0
    assert all(nx[r] > S for r in rows if r != 3) and all(nw[c] > S for c in cols if c != 5)
    plan = _check(xb, wb, dt, S, "outliers")
    assert plan["fallback_rows"] >= len(set(rows.tolist()) - {3})
    assert plan["fallback_cols"] >= len(set(cols.tolist()) - {5})


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_many_tails_and_many_listed_outputs(dt):
    rng = np.random.default_rng(545 + (dt == "bf16"))
    # wide rows have far more than 256 tails: recomputed on the accumulator
    xb, wb = random_operands(rng, 40, 70, 700, dt, "wide")
    _check(xb, wb, dt, 2, "many tails")
    # N(0,1) rows with some wide rows and some single outliers mixed in:
    # tails added one by one next to rows recomputed whole
    xn, wn = random_operands(rng, 90, 130, 400, dt, "normal")
    xw, ww = random_operands(rng, 90, 130, 400, dt, "wide")
    xb, wb = xn.copy(), wn.copy()
    xb[::7], wb[::9] = xw[::7], ww[::9]
    xb[3::11, 5] = xw[3::11, 5]
    wb[4::13, 17] = ww[4::13, 17]
    _check(xb, wb, dt, 4, "mixed tails")
    # more listed outputs than 2^22: whole rows and columns recomputed
    xb, wb = random_operands(rng, 2100, 2100, 64, dt, "normal")
    plan = _check(xb, wb, dt, 2, "many listed")
    assert plan["fallback_rows"] * 2100 + plan["fallback_cols"] * 2100 > (1 << 22)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_recompute_on_views_and_past_one_k_block(dt):
    # the recompute reads the raw operands through its row and column maps:
    # transposed and padded views, and K past one 2^15 block in one launch
    rng = np.random.default_rng(547 + (dt == "bf16"))
    xb, wb = random_operands(rng, 40, 70, 700, dt, "wide")
    x, w = to_device(xb, dt), to_device(wb, dt)
    xt = x.t().contiguous().t()                              # unit M stride
    wp = to_device(np.ascontiguousarray(np.pad(wb, ((0, 0), (3, 5)))), dt)[:, 3:-5]
    for xx, ww in ((xt, w), (x, wp), (xt, wp)):
        plan = _check(xb, wb, dt, 2, "recompute views", x=xx, w=ww)
        assert plan["fallback_rows"] > 0 and plan["fallback_cols"] > 0
    xb, wb = random_operands(rng, 5, 6, 40000, dt, "wide")
    plan = _check(xb, wb, dt, 2, "recompute long K")
    assert plan["fallback_rows"] > 0


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_k_beyond_one_block(dt):
    # K > 2^14: the 128-bit sums are carried between launches in the workspace
    rng = np.random.default_rng(550 + (dt == "bf16"))
    for K, S in ((16385, 4), (40000, 7 if dt == "f32" else 5)):
        xb, wb = random_operands(rng, 35, 66, K, dt, "normal")
        _check(xb, wb, dt, S, "long K")


def test_chosen_digits_on_normal_data():
    # slices = 0: the call picks S; on N(0,1) data it stays on the matrix cores
    rng = np.random.default_rng(560)
    for dt in ("f32", "bf16"):
        xb, wb = random_operands(rng, 128, 192, 256, dt, "normal")
        plan = _check(xb, wb, dt, 0, "chosen S")
        assert 2 <= plan["slices"] <= 7


def _rows_needing(rng, R, K, S, dt):
    """R rows of K values in which every row needs exactly S digits: its top
    set bit lies 8S - 4 bits above its lowest (one element 2^(8S-4), one 1,
    the others 8-bit integers scaled inside that window, random signs, some
    zeros), all scaled by 2^-20."""
    span = 8 * S - 4
    m = rng.integers(1, 256, size=(R, K)).astype(np.float64)
    e = rng.integers(0, span - 7 + 1, size=(R, K))
    v = np.ldexp(m, e) * rng.choice([-1.0, 1.0], size=(R, K))
    v[rng.random((R, K)) < 0.1] = 0.0
    cols = rng.permuted(np.tile(np.arange(K), (R, 1)), axis=1)
    v[np.arange(R), cols[:, 0]] = 2.0 ** span
    v[np.arange(R), cols[:, 1]] = -1.0
    a = np.ldexp(v, -20).astype(np.float32)
    bits = np_f32_bits(a) if dt == "f32" else to_bf16_bits(a)
    assert np.array_equal(_needs(bits, dt), np.full(R, S))
    return bits


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["auto", "slices"])
def test_device_plan_picks_each_digit_count(path, dt):
    # every row of x and w needs exactly S digits, so the plan made on the
    # device picks that S, at sizes where one launch holds S = 2 .. 6 and at
    # one past them (a launch per S), and with K past one 2^14 block; auto
    # considers the matrix cores from 2^27 MACs on
    rng = np.random.default_rng(565 + 2 * (path == "auto") + (dt == "bf16"))
    M, N, K = (600, 500, 600) if path == "auto" else (70, 130, 100)
    cases = [(S, M, N, K) for S in range(2, 8)] + [(5, 2100, 2100, 64), (3, 130, 70, 17000)]
    for S, M, N, K in cases:
        xb, wb = _rows_needing(rng, M, K, S, dt), _rows_needing(rng, N, K, S, dt)
        announce(f"device plan {path} {dt} S={S} M={M} N={N} K={K}")
        x, w = to_device(xb, dt), to_device(wb, dt)
        det.set_gemm_path(path, 0)
        got = f32_bits(det.det_gemm(x, w))
        plan = det.last_gemm_plan()
        assert plan == {"path": "slices", "slices": S, "fallback_rows": 0, "fallback_cols": 0}, plan
        want = c_oracle.gemm(xb, wb)
        assert np.array_equal(got, want), mismatch_report(got, want)


def _row_scaled(rng, M, K, emin, emax, spread, dt):
    """Rows of N(0,1)-like values with few significant bits, each row scaled
    by its own power of two: narrow spans at extreme magnitudes."""
    e = rng.integers(emin, emax + 1, size=(M, 1))
    v = rng.integers(-(1 << spread), (1 << spread) + 1, size=(M, K)).astype(np.float64)
    a = np.ldexp(v, e).astype(np.float32)
    return np_f32_bits(a) if dt == "f32" else to_bf16_bits(a)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_overflow_underflow_and_ties(dt):
    rng = np.random.default_rng(570 + (dt == "bf16"))
    # products far above 2^128 and far below 2^-149: inf, subnormal, +-0
    xb = _row_scaled(rng, 64, 40, -140, 100, 6, dt)
    wb = _row_scaled(rng, 96, 40, -140, 100, 6, dt)
    _check(xb, wb, dt, 3, "extreme rows")
    # integer sums past 2^24 land on rounding ties
    xb = _row_scaled(rng, 40, 300, 0, 0, 12, dt)
    wb = _row_scaled(rng, 70, 300, 0, 0, 12, dt)
    _check(xb, wb, dt, 3, "integer ties")


def test_golden_rounding_fixtures_on_the_matrix_cores():
    announce("golden rounding fixtures, matrix-core path")
    det.set_gemm_path("slices", 0)
    fails = pins.check_golden_rounding(lambda xb, wb, dt: f32_bits(det.det_gemm(to_device(xb, dt),
                                                                                 to_device(wb, dt))))
    assert fails == []


def test_strided_and_transposed_views():
    rng = np.random.default_rng(580)
    for dt, K in (("f32", 140), ("bf16", 140), ("f32", 300), ("bf16", 300)):
        xb, wb = random_operands(rng, 67, 90, K, dt, "normal")
        x, w = to_device(xb, dt), to_device(wb, dt)
        xt = x.t().contiguous().t()                      # unit M stride
        wt = w.t().contiguous().t()
        xs = to_device(np.ascontiguousarray(np.pad(xb, ((0, 0), (5, 3)))), dt)[:, 5:-3]
        # transposed views with 16-byte aligned columns and a ragged row count:
        # the span check and digits take 16-byte loads, the last rows one at a time
        xp = to_device(np.ascontiguousarray(np.pad(xb.T, ((0, 0), (0, 5)))), dt)[:, :67].t()
        wp = to_device(np.ascontiguousarray(np.pad(wb.T, ((0, 0), (0, 6)))), dt)[:, :90].t()
        assert xp.stride() == (1, 72) and wp.stride() == (1, 96)
        for xx, ww in ((xt, w), (x, wt), (xt, wt), (xs, w), (xp, w), (x, wp), (xp, wp)):
            _check(xb, wb, dt, 4, "views", x=xx, w=ww)


def test_auto_path_matches_accumulator_path():
    # above 2^27 MACs, auto considers the matrix cores; the bits never change
    rng = np.random.default_rng(590)
    for dt, kind in (("bf16", "normal"), ("f32", "normal"), ("f32", "wide")):
        announce(f"auto vs accumulator {dt} {kind} 512^3")
        xb, wb = random_operands(rng, 512, 512, 512, dt, kind)
        x, w = to_device(xb, dt), to_device(wb, dt)
        det.set_gemm_path("accumulator")
        ya = f32_bits(det.det_gemm(x, w))
        assert det.last_gemm_plan()["path"] == "accumulator"
        det.set_gemm_path("auto")
        yb = f32_bits(det.det_gemm(x, w))
        plan = det.last_gemm_plan()
        announce(f"auto plan {plan}")
        assert np.array_equal(ya, yb), mismatch_report(yb, ya)
        rr, cc = np.meshgrid(np.arange(0, 512, 37), np.arange(3, 512, 41), indexing="ij")
        want = c_oracle.gemm_pairs(xb, wb, rr.ravel(), cc.ravel())
        assert np.array_equal(ya[rr.ravel(), cc.ravel()], want)
        if kind == "normal":
            assert plan["path"] == "slices"
        else:
            assert plan["path"] == "accumulator"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_tails_spread_over_many_k_ranges(dt):
    # listed rows whose tails lie in several 1024-long K ranges (each range's
    # wave reserves its own places in the row's list), rows with just under
    # and just over 256 tails, and the same for columns
    rng = np.random.default_rng(600 + (dt == "bf16"))
    M, N, K = 70, 90, 5000
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((N, K), dtype=np.float32)
    tiny = np.float32(2.0 ** -70)                      # below the window at S = 7 (f32) and 4 (bf16)
    for r, n_t in ((3, 5), (10, 200), (11, 256), (12, 257), (40, 600)):
        x[r, rng.choice(K, n_t, replace=False)] = tiny * rng.integers(1, 100, n_t)
    for c, n_t in ((7, 9), (8, 250), (60, 300)):
        w[c, rng.choice(K, n_t, replace=False)] = -tiny * rng.integers(1, 100, n_t)
    conv = np_f32_bits if dt == "f32" else to_bf16_bits
    xb, wb = conv(x), conv(w)
    S = 7 if dt == "f32" else 4
    plan = _check(xb, wb, dt, S, "spread tails")
    assert plan["fallback_rows"] >= 5 and plan["fallback_cols"] >= 3


def test_concurrent_calls_from_two_threads():
    # each thread has its own readback buffers: two threads on their own
    # streams, with different numbers of listed rows, get the oracle's bits
    rng = np.random.default_rng(610)
    cases = []
    for t in range(2):
        xb, wb = random_operands(rng, 300 + 50 * t, 260, 700, "bf16", "normal")
        xw, _ = random_operands(rng, 300 + 50 * t, 260, 700, "bf16", "wide")
        xb[:: 5 + 4 * t] = xw[:: 5 + 4 * t]                 # listed rows, some recomputed
        cases.append((xb, wb))
    want = [c_oracle.gemm(xb, wb) for xb, wb in cases]
    det.set_gemm_path("slices", 4)
    got = [[None] * 6, [None] * 6]
    errors = []

    def run(t):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                x, w = to_device(cases[t][0], "bf16"), to_device(cases[t][1], "bf16")
                for i in range(6):
                    got[t][i] = f32_bits(det.det_gemm(x, w))
        except Exception as e:                              # reported below, in the main thread
            errors.append(e)

    announce("slices from two threads at once")
    threads = [threading.Thread(target=run, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    for t in range(2):
        for i in range(6):
            assert np.array_equal(got[t][i], want[t]), (t, i, mismatch_report(got[t][i], want[t]))
