"""Exact loss reductions: the sum over a whole tensor formed in the long
accumulator, so the loss value does not depend on how the elements are split
or ordered (det-train page, "Method": an exact sum is independent of its
order; "Usage": the partials of K-slices compose into the whole sum).

exact_mse_loss(y, t) = RNE32( sum_i (y_i - t_i)^2 ) / n

The squared error is never rounded per element: with every product exact,
sum (y - t)^2 = sum y*y + sum t*t - sum 2*y*t, three exact products per
element added into one accumulator (det_sqdiff_partial), rounded once to
fp32 (det_finalize).  The division by n is one more IEEE fp32 division,
correctly rounded, by n as an fp32 value (n itself rounded to fp32 above
2^24; the quotient is exact when n is a power of two and stays normal).
Without a target the loss is sum y^2 / n.

The gradient 2 (y - t) / n is elementwise (no reduction, so no order to fix)
and is formed by the library's det_mse_grad kernel, one correctly rounded fp32
operation at a time:
  dy = RNE_dtype( RNE32( RNE32(y - t) * c ) * g ),  c = RNE32(2 / fp32(n)),
with g the incoming gradient (1 when the loss is the output) and the last
rounding only for bfloat16 y; the target's gradient is the negation.  c is one
IEEE fp32 division on the host.  When n is a power of two (and nothing
underflows) c is exact and the scaling adds no rounding.
"""
from __future__ import annotations

from typing import Optional

import torch

from .api import det_finalize, exact_sqdiff_digits, mse_grad


class _ExactMSE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, y: torch.Tensor, t: Optional[torch.Tensor]) -> torch.Tensor:
        s = det_finalize(exact_sqdiff_digits(y, t, check_finite=False)).reshape(())
        ctx.save_for_backward(y, t if t is not None else y)
        ctx.has_target = t is not None
        # a true fp32 division by a device tensor: torch turns a division by
        # a host scalar into a product with its rounded reciprocal
        n = torch.full((), float(max(y.numel(), 1)), dtype=torch.float32, device=s.device)
        return s / n

    @staticmethod
    def backward(ctx, g: torch.Tensor):
        y, t = ctx.saved_tensors
        need_dt = ctx.has_target and ctx.needs_input_grad[1]
        dy, dt = mse_grad(y, t if ctx.has_target else None, g, ctx.needs_input_grad[0], need_dt)
        return dy, dt


def exact_mse_loss(y: torch.Tensor, target: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mean squared error with the sum formed exactly; a 0-d float32 tensor.

    y (and target, if given): float32 or bfloat16 GPU tensors of one shape
    and dtype, finite; at most 2^30 / 3 elements with a target, 2^30
    without."""
    if target is not None:
        if target.shape != y.shape or target.dtype != y.dtype:
            raise ValueError("exact_mse_loss needs y and target of one shape and dtype")
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("exact_mse_loss takes float32 or bfloat16 tensors")
    return _ExactMSE.apply(y, target)
