"""A 160-step training run, unsharded against 4-way K-sharded forward GEMMs.

The det-train page's introduction describes the experiment: the same model
trained for 160 steps once with unsharded layers and once with 4-way K-sharded
ones.  With fp32 accumulation the per-step losses and final weights drift
apart (summation order differs); with the exact accumulator they are the same
bytes at every step.  This test runs that comparison on synthetic data: a
two-layer DetLinear MLP (f32 parameters) with k_shards=1 and k_shards=4
(forward GEMMs as det_gemm_partial over 4 K-slices, det_combine,
det_finalize), plain SGD; and, as the control, the same model with torch's
fp32 matmul, the sharded variant summing four K-slice products.
"""
import numpy as np
import pytest
import torch

import bitwise_deterministic_exact_amd as det
from oracle import c_oracle
from tests.gpu_util import announce, mismatch_report

pytestmark = pytest.mark.gpu

STEPS = 160
IN, HID, OUT, BATCH = 192, 256, 32, 128
LR = 0.05


def _data(seed=7):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((BATCH, IN), dtype=np.float32)
    teacher = rng.standard_normal((IN, OUT), dtype=np.float32) / np.sqrt(IN)
    y = np.tanh(x @ teacher).astype(np.float32)
    w1 = (rng.standard_normal((HID, IN), dtype=np.float32) / np.sqrt(IN)).astype(np.float32)
    w2 = (rng.standard_normal((OUT, HID), dtype=np.float32) / np.sqrt(HID)).astype(np.float32)
    return [torch.from_numpy(a).cuda() for a in (x, y, w1, w2)]


RECORD = (0, 80, STEPS - 1)       # steps whose GEMMs are checked against the oracle


def _train_det(k_shards, record=()):
    """Train; for the steps in `record` also keep what each layer's GEMMs
    read and wrote: the layer inputs and weights of the step, the forward
    outputs, the gradients arriving at the outputs (dY), the layer-2 input
    gradient (dX) and the weight gradients."""
    x, y, w1, w2 = _data()
    l1 = det.DetLinear(IN, HID, device="cuda", k_shards=k_shards)
    l2 = det.DetLinear(HID, OUT, device="cuda", k_shards=k_shards)
    with torch.no_grad():
        l1.weight.copy_(w1)
        l2.weight.copy_(w2)
    losses, kept = [], {}
    for step in range(STEPS):
        y1 = l1(x)
        h = torch.relu(y1)
        h.retain_grad()
        y2 = l2(h)
        loss = (y2 - y).square().mean()
        grads = {}
        if step in record:
            y1.register_hook(lambda g: grads.__setitem__("dy1", g.detach().clone()))
            y2.register_hook(lambda g: grads.__setitem__("dy2", g.detach().clone()))
            kept[step] = {"x": x, "w1": l1.weight.detach().clone(), "w2": l2.weight.detach().clone(),
                          "y1": y1.detach().clone(), "h": h.detach().clone(), "y2": y2.detach().clone()}
        l1.weight.grad = l2.weight.grad = None
        loss.backward()
        if step in record:
            kept[step].update(grads, dh=h.grad.detach().clone(), dw1=l1.weight.grad.detach().clone(),
                              dw2=l2.weight.grad.detach().clone())
        with torch.no_grad():
            l1.weight -= LR * l1.weight.grad
            l2.weight -= LR * l2.weight.grad
        losses.append(loss.detach())
    out = (torch.stack(losses), l1.weight.detach().clone(), l2.weight.detach().clone())
    return out + (kept,) if record else out


def _np_bits(t):
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


def _check_step_against_oracle(rec):
    """Each of the step's five GEMMs, every output, against the oracle (f32
    parameters: the results are the oracle's fp32 bits): y1 = x W1^T, y2 =
    h W2^T, dh = dY2 W2 (K = 32), dW2 = dY2^T h and dW1 = dY1^T x (K =
    the batch, 128)."""
    b = {k: _np_bits(v) for k, v in rec.items()}
    T = lambda a: np.ascontiguousarray(a.T)
    cases = [("y1", b["x"], b["w1"]), ("y2", b["h"], b["w2"]), ("dh", b["dy2"], T(b["w2"])),
             ("dw2", T(b["dy2"]), T(b["h"])), ("dw1", T(b["dy1"]), T(b["x"]))]
    for name, xa, wa in cases:
        want = c_oracle.gemm(xa, wa)
        assert np.array_equal(b[name], want), f"{name}: " + mismatch_report(b[name].ravel(), want.ravel())


def _linear_fp32(x, w, k_shards):
    if k_shards == 1:
        return x @ w.t()
    out = None
    for a, b in det.linear.shard_bounds(x.shape[1], k_shards):
        part = x[:, a:b] @ w[:, a:b].t()
        out = part if out is None else out + part
    return out


def _train_fp32(k_shards):
    x, y, w1, w2 = _data()
    w1 = w1.clone().requires_grad_(True)
    w2 = w2.clone().requires_grad_(True)
    losses = []
    for _ in range(STEPS):
        h = torch.relu(_linear_fp32(x, w1, k_shards))
        loss = (_linear_fp32(h, w2, k_shards) - y).square().mean()
        w1.grad = w2.grad = None
        loss.backward()
        with torch.no_grad():
            w1 -= LR * w1.grad
            w2 -= LR * w2.grad
        losses.append(loss.detach())
    return torch.stack(losses), w1.detach().clone(), w2.detach().clone()


def _bits(t):
    return t.contiguous().view(torch.int32)


def test_160_steps_unsharded_vs_4way_ksharded_identical_bytes():
    announce(f"training {STEPS} steps, DetLinear MLP {IN}-{HID}-{OUT}, k_shards 1 and 4")
    loss1, a1, b1, kept1 = _train_det(1, RECORD)
    loss4, a4, b4, kept4 = _train_det(4, RECORD)
    # at steps 0, 80 and 159 every GEMM of both runs equals the oracle's
    for step in RECORD:
        announce(f"training step {step}: the five GEMMs of each run against the oracle")
        _check_step_against_oracle(kept1[step])
        _check_step_against_oracle(kept4[step])
    # it trains: the loss falls
    assert loss1[-1].item() < 0.5 * loss1[0].item()
    # exact accumulation: identical losses at every step and identical weights
    assert torch.equal(_bits(loss1), _bits(loss4))
    assert torch.equal(_bits(a1), _bits(a4))
    assert torch.equal(_bits(b1), _bits(b4))
    # and a repeat of the unsharded run gives the same bytes again
    loss1b, a1b, _ = _train_det(1)
    assert torch.equal(_bits(loss1), _bits(loss1b)) and torch.equal(_bits(a1), _bits(a1b))


def test_fp32_control_drifts_under_ksharding():
    announce(f"fp32 control: {STEPS} steps, torch matmul unsharded vs 4 K-slices")
    loss1, a1, _ = _train_fp32(1)
    loss4, a4, _ = _train_fp32(4)
    assert loss1[-1].item() < 0.5 * loss1[0].item()
    dl = (loss1 - loss4).abs().max().item()
    dw = ((a1 - a4).abs().max() / a1.abs().max()).item()
    announce(f"fp32 control: max |loss difference| {dl:.3g}, max relative weight difference {dw:.3g}")
    # the summation order changes the bits: the runs are not identical
    assert not torch.equal(_bits(a1), _bits(a4))
