"""GPU parity of the exact bias, the K-slice composition past 2^19 and the
exact loss reduction against the oracle, bit for bit.

A bias b is one more term of each output's exact sum: y = RNE32(sum_k x*w +
1*b), which the oracle computes as the exact GEMM of [x | 1] and [W | b].
The bias gradient is the exact column sum of dY, the GEMM of dY^T with a row
of ones.  K past 2^19 runs as K-slices of raw digits composed by
det_combine, which the oracle's single exact sum must equal.  The loss is
the exact sum of squared errors rounded once, then divided by n in fp32."""
from fractions import Fraction
import numpy as np
import pytest
import torch

import bitwise_deterministic_exact_amd as det
from oracle import c_oracle
from oracle.exact import f32_bits_to_bf16_bits
from tests import pins
from tests.gpu_util import announce, f32_bits, mismatch_report, tensor_bits, to_device
from workloads import random_operands

pytestmark = pytest.mark.gpu

ONE = {"f32": np.uint32(0x3F800000), "bf16": np.uint16(0x3F80)}
NEG = {"f32": np.uint32(0x80000000), "bf16": np.uint16(0x8000)}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _ones(shape, dt):
    return np.full(shape, ONE[dt], dtype=ONE[dt].dtype)


def _to_param_dtype(bits32: np.ndarray, dt: str) -> np.ndarray:
    return bits32 if dt == "f32" else f32_bits_to_bf16_bits(bits32)


def _layer(dt, IN, OUT, k_shards, Wb, bb):
    layer = det.DetLinear(IN, OUT, bias=True, device="cuda", dtype=TORCH_DT[dt], k_shards=k_shards)
    with torch.no_grad():
        layer.weight.copy_(to_device(Wb, dt))
        layer.bias.copy_(to_device(bb, dt))
    return layer


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("k_shards", [1, 3])
def test_detlinear_bias_forward_backward(dt, k_shards):
    rng = np.random.default_rng(600 + 2 * k_shards + (dt == "bf16"))
    T, IN, OUT = 37, 50, 29
    for kind in ("normal", "wide"):
        announce(f"DetLinear bias {dt} k_shards={k_shards} {kind} T={T} {IN}->{OUT}")
        xb, Wb = random_operands(rng, T, OUT, IN, dt, kind)
        bb = random_operands(rng, 1, OUT, 1, dt, kind)[1].reshape(OUT)
        layer = _layer(dt, IN, OUT, k_shards, Wb, bb)
        x = to_device(xb, dt).requires_grad_(True)
        y = layer(x)
        want = c_oracle.gemm(np.hstack([xb, _ones((T, 1), dt)]), np.hstack([Wb, bb.reshape(OUT, 1)]))
        got = f32_bits(y)
        assert np.array_equal(got, want), mismatch_report(got, want)
        # backward with a given upstream gradient G; dY is G rounded to the
        # parameter dtype
        G = rng.standard_normal((T, OUT), dtype=np.float32)
        gb = _to_param_dtype(G.view(np.uint32), dt)
        y.backward(torch.from_numpy(G).cuda())
        dx = c_oracle.gemm(gb, np.ascontiguousarray(Wb.T))
        dw = c_oracle.gemm(np.ascontiguousarray(gb.T), np.ascontiguousarray(xb.T))
        db = c_oracle.gemm(np.ascontiguousarray(gb.T), _ones((1, T), dt)).reshape(OUT)
        for name, g, w32 in (("dx", x.grad, dx), ("dW", layer.weight.grad, dw), ("db", layer.bias.grad, db)):
            want = _to_param_dtype(w32, dt)
            got = tensor_bits(g)
            assert np.array_equal(got, want), f"{name}: " + mismatch_report(got, want)


def test_detlinear_bias_on_the_matrix_cores():
    # 512 tokens, 512 -> 512 bf16: the forward (K = 513 with the bias term)
    # is large enough for det_gemm to consider the matrix-core path
    rng = np.random.default_rng(610)
    T = IN = OUT = 512
    xb, Wb = random_operands(rng, T, OUT, IN, "bf16", "normal")
    bb = random_operands(rng, 1, OUT, 1, "bf16", "normal")[1].reshape(OUT)
    layer = _layer("bf16", IN, OUT, 1, Wb, bb)
    x = to_device(xb, "bf16")
    announce("DetLinear bias bf16 512^3, auto path")
    y = f32_bits(layer(x))
    plan = det.last_gemm_plan()
    with det.gemm_path("accumulator"):
        ya = f32_bits(layer(x))
    assert np.array_equal(y, ya), mismatch_report(y, ya)
    rr, cc = np.meshgrid(np.arange(0, T, 29), np.arange(1, OUT, 31), indexing="ij")
    xc = np.hstack([xb, _ones((T, 1), "bf16")])
    wc = np.hstack([Wb, bb.reshape(OUT, 1)])
    want = c_oracle.gemm_pairs(xc, wc, rr.ravel(), cc.ravel())
    assert np.array_equal(y[rr.ravel(), cc.ravel()], want)
    announce(f"plan {plan}")
    assert plan["path"] == "slices"


def _oracle_gemm_long(xb, wb):
    """The oracle's exact sum for any K: its raw digits over K-thirds (each
    within its 2^19 limit) added digit for digit, then rounded once."""
    K = xb.shape[1]
    cuts = [0, K // 3, (2 * K) // 3, K]
    parts = [c_oracle.partial(np.ascontiguousarray(xb[:, a:b]), np.ascontiguousarray(wb[:, a:b]))
             for a, b in zip(cuts[:-1], cuts[1:])]
    return c_oracle.finalize(c_oracle.combine(parts))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gemm_any_k_past_one_call(dt):
    rng = np.random.default_rng(620 + (dt == "bf16"))
    for K, kind in ((det.K_MAX + 3000, "wide"), (2 * det.K_MAX + 1, "normal"), (det.K_MAX, "special")):
        announce(f"gemm_any_k {dt} {kind} 3 x 2 x {K}")
        xb, wb = random_operands(rng, 3, 2, K, dt, kind)
        got = f32_bits(det.gemm_any_k(to_device(xb, dt), to_device(wb, dt)))
        want = _oracle_gemm_long(xb, wb)
        assert np.array_equal(got, want), mismatch_report(got, want)


def test_detlinear_weight_and_bias_gradients_past_2e19_tokens():
    # T > 2^19 tokens: dW and db are K-slice compositions
    rng = np.random.default_rng(630)
    T, IN, OUT = det.K_MAX + 77, 4, 3
    announce(f"DetLinear bias f32 T={T} {IN}->{OUT}")
    xb, Wb = random_operands(rng, T, OUT, IN, "f32", "uniform")
    bb = random_operands(rng, 1, OUT, 1, "f32", "uniform")[1].reshape(OUT)
    layer = _layer("f32", IN, OUT, 1, Wb, bb)
    x = to_device(xb, "f32")
    y = layer(x)
    G = rng.standard_normal((T, OUT), dtype=np.float32)
    y.backward(torch.from_numpy(G).cuda())
    gb = G.view(np.uint32)
    dw = _oracle_gemm_long(np.ascontiguousarray(gb.T), np.ascontiguousarray(xb.T))
    db = _oracle_gemm_long(np.ascontiguousarray(gb.T), _ones((1, T), "f32")).reshape(OUT)
    assert np.array_equal(tensor_bits(layer.weight.grad), dw)
    assert np.array_equal(tensor_bits(layer.bias.grad), db)


def _oracle_digits(ab, bb):
    """The oracle's raw digits of sum_i a_i b_i (1-D bit arrays), over slices
    of 400000 when longer than its 2^19 limit (raw digits add, so the split
    does not change them)."""
    a, b = ab.reshape(1, -1), bb.reshape(1, -1)
    if a.shape[1] <= det.K_MAX:
        return c_oracle.partial(a, b).reshape(-1)
    K = a.shape[1]
    cuts = list(range(0, K, 400_000)) + [K]
    parts = [c_oracle.partial(np.ascontiguousarray(a[:, p:q]), np.ascontiguousarray(b[:, p:q]))
             for p, q in zip(cuts[:-1], cuts[1:])]
    return c_oracle.combine(parts).reshape(-1)


def _value(digits):
    return sum(int(d) << (32 * j) for j, d in enumerate(np.asarray(digits).tolist()))


DOT_CASES = [(0, "normal"), (1, "normal"), (3, "special"), (7, "wide"), (8, "normal"), (1000, "wide"),
             (4097, "special"), (det.K_MAX + 5, "normal"), (3_000_003, "wide")]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_exact_dot_digits_equal_the_oracles(dt):
    rng = np.random.default_rng(640 + (dt == "bf16"))
    for n, kind in DOT_CASES:
        announce(f"exact_dot {dt} {kind} n={n}")
        ab, bb = (v.reshape(n) for v in random_operands(rng, 1, 1, n, dt, kind))
        a, b = to_device(ab, dt), to_device(bb, dt)
        want = _oracle_digits(ab, bb)
        got = det.exact_dot_digits(a, b).cpu().numpy()
        assert np.array_equal(got, want), (got, want)
        assert f32_bits(det.exact_dot(a, b).reshape(1))[0] == c_oracle.finalize(want.reshape(1, 18))[0]
        if 0 < n <= det.K_MAX:       # the same raw digits as the 1 x 1 GEMM partial
            assert torch.equal(det.det_gemm_partial(a.reshape(1, n), b.reshape(1, n)).reshape(-1),
                               det.exact_dot_digits(a, b))
        # sum of squares: the digits' value is the exact sum of a_i^2
        got = det.exact_sqdiff_digits(a).cpu().numpy()
        assert _value(got) == _value(_oracle_digits(ab, ab))
        assert f32_bits(det.exact_sum_squares(a).reshape(1))[0] == \
            c_oracle.finalize(_oracle_digits(ab, ab).reshape(1, 18))[0]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_exact_dot_strided_unaligned_and_broadcast(dt):
    rng = np.random.default_rng(660 + (dt == "bf16"))
    M, K = 300, 257
    xb, wb = random_operands(rng, M, 2, K, dt, "normal")
    x, w = to_device(xb, dt), to_device(wb, dt)
    cases = [
        ("column", x[:, 5], xb[:, 5], x[:, 9], xb[:, 9]),                 # increment K
        ("unaligned", x[3, 1:], xb[3, 1:], x[4, 1:], xb[4, 1:]),          # 1 element off 16 B
        ("matrix", x[:, :64], xb[:, :64], x[:, 64:128], xb[:, 64:128]),   # 2-D, flattened
        ("broadcast", w[0], wb[0], w[1, :1].expand(K), np.repeat(wb[1, :1], K)),   # increment 0
    ]
    for name, a, ab, b, bbits in cases:
        announce(f"exact_dot {dt} {name}")
        ab, bbits = np.ascontiguousarray(ab).reshape(-1), np.ascontiguousarray(bbits).reshape(-1)
        got = det.exact_dot_digits(a, b).cpu().numpy()
        assert np.array_equal(got, _oracle_digits(ab, bbits)), name


def test_dot_digits_accumulate_across_calls():
    # accumulate = 1 adds into the digits of an earlier call: the digits of
    # both halves equal the digits of the whole
    rng = np.random.default_rng(670)
    ab, bb = (v.reshape(-1) for v in random_operands(rng, 1, 1, 10001, "f32", "wide"))
    a, b = to_device(ab, "f32"), to_device(bb, "f32")
    lib = det._lib.load()
    acc = torch.empty(18, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for lo, hi, accumulate in ((0, 4000, 0), (4000, 10001, 1)):
        det._lib.check(lib.det_dot_partial(0, a[lo:].data_ptr(), 1, b[lo:].data_ptr(), 1, hi - lo,
                                           acc.data_ptr(), accumulate, stream))
    assert np.array_equal(acc.cpu().numpy(), _oracle_digits(ab, bb))


def _loss_oracle(yb, tb, dt):
    neg = tb ^ NEG[dt]
    s = c_oracle.gemm(np.hstack([yb, tb, yb, yb]).reshape(1, -1),
                      np.hstack([yb, tb, neg, neg]).reshape(1, -1))[0, 0]
    return np.float32(np.array([s], dtype=np.uint32).view(np.float32)[0] / np.float32(yb.size))


def _mse_grad_reference(yb, tb, n, dt, gscale=1.0, negate=False):
    """The exact-MSE gradient's bits as the loss defines them:
    RNE_dt(RNE32(RNE32(RNE32(y - t) * RNE32(2 / fp32(n))) * g)), negated for the
    target's gradient, from exact rationals: the difference and the scale
    rounded to fp32 by pins.rne_fraction, each product formed exactly in fp64
    (two 24-bit significands, or one and a small integer g), one IEEE cast to
    fp32, and for bf16 rne_fraction to 8 bits."""
    as_f32 = lambda b: float(np.array([b], dtype=np.uint32).view(np.float32)[0])
    val = (lambda b: Fraction(as_f32(int(b)))) if dt == "f32" else (lambda b: Fraction(as_f32(int(b) << 16)))
    c = pins.rne_fraction(Fraction(2) / Fraction(float(np.float32(n))), 24)
    out = []
    for yv, tv in zip(yb.tolist(), tb.tolist()):
        d = pins.rne_fraction(val(yv) - val(tv), 24)
        if d == 0:                                    # an exact zero keeps IEEE's sign: (-0) - (+0) = -0
            d = (as_f32(int(yv)) if dt == "f32" else as_f32(int(yv) << 16)) - \
                (as_f32(int(tv)) if dt == "f32" else as_f32(int(tv) << 16))
        g = np.float32(np.float64(float(d)) * np.float64(float(c)))      # exact product, one rounding
        if gscale != 1.0:
            g = np.float32(np.float64(g) * np.float64(gscale))
        if negate:
            g = -g
        if dt == "bf16":
            gb = g if np.isinf(g) else np.float32(float(pins.rne_fraction(Fraction(float(g)), 8)))
            bits = int(np.array([gb], dtype=np.float32).view(np.uint32)[0]) >> 16
            if gb == 0 and np.signbit(g):             # a negative value rounded to zero is -0
                bits = 0x8000
            out.append(bits)
        else:
            out.append(int(np.array([g], dtype=np.float32).view(np.uint32)[0]))
    return np.array(out, dtype=np.uint16 if dt == "bf16" else np.uint32)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_exact_mse_loss(dt):
    rng = np.random.default_rng(650 + (dt == "bf16"))
    for n, kind in ((64, "normal"), (1000, "uniform"), (3 * 4096 + 5, "wide")):
        announce(f"exact_mse_loss {dt} {kind} n={n}")
        yb, tb = random_operands(rng, 1, 1, n, dt, kind)
        yb, tb = yb.reshape(n), tb.reshape(n)
        y = to_device(yb, dt).requires_grad_(True)
        t = to_device(tb, dt)
        loss = det.exact_mse_loss(y, t)
        want = _loss_oracle(yb, tb, dt)
        assert loss.dtype == torch.float32 and loss.dim() == 0
        assert f32_bits(loss.reshape(1))[0] == want.view(np.uint32)
        # the same elements in another order: the same bits
        perm = torch.from_numpy(rng.permutation(n)).cuda()
        assert torch.equal(det.exact_mse_loss(y.detach()[perm], t[perm]).view(torch.int32),
                           loss.detach().view(torch.int32))
        # the gradient, elementwise: RNE_dt(RNE32(RNE32(y - t) * RNE32(2 / fp32(n)))),
        # computed here from exact rationals and one IEEE cast
        loss.backward()
        want_g = _mse_grad_reference(yb, tb, n, dt)
        got_g = tensor_bits(y.grad)
        assert np.array_equal(got_g, want_g), mismatch_report(got_g, want_g)
    # a target that needs its gradient too, and an incoming gradient of 3
    yb, tb = random_operands(rng, 1, 1, 777, dt, "wide")
    yb, tb = yb.reshape(777), tb.reshape(777)
    y = to_device(yb, dt).requires_grad_(True)
    t = to_device(tb, dt).requires_grad_(True)
    (det.exact_mse_loss(y, t) * 3.0).backward()
    for got, neg in ((y.grad, False), (t.grad, True)):
        want_g = _mse_grad_reference(yb, tb, 777, dt, gscale=3.0, negate=neg)
        assert np.array_equal(tensor_bits(got), want_g), mismatch_report(tensor_bits(got), want_g)
    # operands one element past a 16-byte boundary: the one-at-a-time form
    yv = to_device(np.concatenate([yb[:1], yb]), dt)[1:].detach().requires_grad_(True)
    tv = to_device(np.concatenate([tb[:1], tb]), dt)[1:]
    assert yv.data_ptr() % 16 != 0
    det.exact_mse_loss(yv, tv).backward()
    want_g = _mse_grad_reference(yb, tb, 777, dt)
    assert np.array_equal(tensor_bits(yv.grad), want_g), mismatch_report(tensor_bits(yv.grad), want_g)
    # without a target: the gradient of sum y^2 / n
    y = to_device(yb, dt).requires_grad_(True)
    det.exact_mse_loss(y).backward()
    zero = np.zeros_like(yb)
    want_g = _mse_grad_reference(yb, zero, 777, dt)
    assert np.array_equal(tensor_bits(y.grad), want_g), mismatch_report(tensor_bits(y.grad), want_g)
    # the fp32 division of the rounded sum by n is correctly rounded
    s32 = rng.standard_normal(4096).astype(np.float32) * np.float32(1e3)
    for n in (3, 7, 1000, 12293, 8191, 1 << 20):
        want = (s32 / np.float32(n)).astype(np.float32)
        got = (torch.from_numpy(s32).cuda() / torch.tensor(float(n), device="cuda")).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), n
    # no target: sum y^2 / n
    yb = random_operands(rng, 1, 1, 256, dt, "normal")[0].reshape(256)
    y = to_device(yb, dt)
    s = c_oracle.gemm(yb.reshape(1, -1), yb.reshape(1, -1))[0, 0]
    want = np.float32(np.array([s], dtype=np.uint32).view(np.float32)[0] / np.float32(256))
    assert f32_bits(det.exact_mse_loss(y).reshape(1))[0] == want.view(np.uint32)
