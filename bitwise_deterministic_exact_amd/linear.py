"""DetLinear: a linear layer whose forward and backward GEMMs are exact
long-accumulator GEMMs (det-train page, "Usage" section: DetLinear(4096,
4096) with a deterministic forward and backward).

forward : y  = x W^T                     (K = in_features), fp32 out
          with bias=True: y = x W^T + b, the bias one more exact term of the
          same sum ([x | 1] [W | b]^T, K = in_features + 1), rounded once
backward: dY rounded to the parameter dtype (nearest-even) when it is bf16,
          dX = dY W                      (K = out_features)
          dW = dY^T x                    (K = tokens)
          db = sum over tokens of dY     (K = tokens, exact, bias=True only)
Each product is exact and each result is rounded once to fp32; dX, dW and db
are then rounded (nearest-even) to the dtypes of x and the parameters.  K
beyond 2^19 (tokens) runs as exact K-slices composed by det_combine.  Every step runs in the
library's kernels; the transposed operands are strided views, not copies.

With k_shards > 1 the forward is computed the way a row-parallel
(K-sharded) layer computes it: in_features is cut into k_shards contiguous
slices, each slice's raw digits come from det_gemm_partial, the digit arrays
are added with det_combine (where a multi-GPU layer would all-reduce them) and
det_finalize rounds once.  The page's "Method" section makes this bit-for-bit
the unsharded result, so a model trains to the same bytes either way.
"""
from __future__ import annotations

import math

import torch

from .api import det_combine, det_finalize, det_gemm, det_gemm_partial, gemm_any_k, round_f32_to_bf16


def _to_dtype(t32: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    if dtype == torch.float32:
        return t32
    if dtype == torch.bfloat16:
        return round_f32_to_bf16(t32)
    raise ValueError(f"unsupported dtype {dtype}")


def shard_bounds(k: int, shards: int):
    """Contiguous [a, b) slices of range(k), as equal as possible."""
    cuts = [k * i // shards for i in range(shards + 1)]
    return [(cuts[i], cuts[i + 1]) for i in range(shards) if cuts[i] < cuts[i + 1]]


def _forward_gemm(x2: torch.Tensor, weight: torch.Tensor, k_shards: int) -> torch.Tensor:
    if k_shards <= 1:
        return gemm_any_k(x2, weight, check_finite=False)
    parts = [det_gemm_partial(x2[:, a:b], weight[:, a:b], check_finite=False)
             for a, b in shard_bounds(x2.shape[1], k_shards)]
    return det_finalize(det_combine(parts))


def _with_bias(x2: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor):
    """[x | 1] and [W | b]: the bias as the K-term 1 * b_n of the same sum."""
    ones = torch.ones((x2.shape[0], 1), dtype=x2.dtype, device=x2.device)
    return torch.cat([x2, ones], dim=1), torch.cat([weight, bias.reshape(-1, 1)], dim=1)


class _DetLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x: torch.Tensor, weight: torch.Tensor, bias, k_shards: int) -> torch.Tensor:
        x2 = x.reshape(-1, x.shape[-1])
        if bias is None:
            y = _forward_gemm(x2, weight, k_shards)
        else:
            y = _forward_gemm(*_with_bias(x2, weight, bias), k_shards)
        ctx.save_for_backward(x2, weight)
        ctx.x_shape = x.shape
        ctx.has_bias = bias is not None
        return y.reshape(*x.shape[:-1], weight.shape[0])

    @staticmethod
    def backward(ctx, gy: torch.Tensor):
        x2, weight = ctx.saved_tensors
        g32 = gy.reshape(-1, weight.shape[0]).to(torch.float32).contiguous()
        g = _to_dtype(g32, weight.dtype)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx32 = det_gemm(g, weight.t(), check_finite=False)        # [T, in], K = out
            dx = _to_dtype(dx32, x2.dtype).reshape(ctx.x_shape)
        if ctx.needs_input_grad[1]:
            dw32 = gemm_any_k(g.t(), x2.t(), check_finite=False)      # [out, in], K = T
            dw = _to_dtype(dw32, weight.dtype)
        db = None
        if ctx.has_bias and ctx.needs_input_grad[2]:
            ones = torch.ones((1, g.shape[0]), dtype=g.dtype, device=g.device)
            db32 = gemm_any_k(ones, g.t(), check_finite=False)        # [1, out], K = T
            db = _to_dtype(db32.reshape(-1), weight.dtype)
        return dx, dw, db, None


class DetLinear(torch.nn.Module):
    """y = x W^T with exact accumulation; W is [out_features, in_features]."""

    def __init__(self, in_features: int, out_features: int, bias: bool = False,
                 device=None, dtype=torch.float32, k_shards: int = 1):
        super().__init__()
        if k_shards < 1:
            raise ValueError("k_shards must be >= 1")
        self.k_shards = k_shards
        if dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("DetLinear supports float32 and bfloat16 parameters")
        self.in_features, self.out_features = in_features, out_features
        self.weight = torch.nn.Parameter(torch.empty(out_features, in_features, device=device,
                                                     dtype=dtype))
        with torch.no_grad():
            bound = 1.0 / math.sqrt(in_features)
            w = torch.empty(out_features, in_features, dtype=torch.float32).uniform_(-bound, bound)
            self.weight.copy_(w.to(dtype))
        if bias:
            self.bias = torch.nn.Parameter(torch.empty(out_features, device=device, dtype=dtype))
            with torch.no_grad():
                b = torch.empty(out_features, dtype=torch.float32).uniform_(-bound, bound)
                self.bias.copy_(b.to(dtype))
        else:
            self.register_parameter("bias", None)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.dtype != self.weight.dtype:
            raise ValueError(f"input dtype {x.dtype} differs from weight dtype {self.weight.dtype}")
        return _DetLinearFn.apply(x, self.weight, self.bias, self.k_shards)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}"
                + (f", k_shards={self.k_shards}" if self.k_shards > 1 else ""))
