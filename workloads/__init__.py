"""Seeded synthetic inputs for the exact GEMM, shared by the oracle tests, the
GPU parity tests and the benchmark.

This module holds none of the method's arithmetic: it only draws numbers
(numpy PCG64 via ``default_rng``, x before w) and rounds them to the operand
dtype with library routines (numpy's fp64->fp32 cast, torch's CPU fp32->bf16
cast, both round-to-nearest-even).

The det-train page measures on no public dataset; these configurations stand
for the shapes it names (the 4096x4096 DetLinear of its "Usage" section, K up
to 2^19 from "Requirements and limits", 2- to 16-way K-shards and arbitrary
fold groupings from "Correctness").

bf16 operands are returned as uint16 bit patterns (numpy has no bf16), f32
operands as float32 arrays.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

K_MAX = 1 << 19


def f32_bits(a: np.ndarray) -> np.ndarray:
    """uint32 view of a float32 array (no copy when contiguous)."""
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round a float32 array to bf16 (torch CPU cast, nearest-even); uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: bf16 is the top half of f32)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def wide_range_f32(rng: np.random.Generator, shape: Tuple[int, ...],
                   emin: int = -70, emax: int = 70, sub_frac: float = 0.01) -> np.ndarray:
    """Entries sign*m*2^e: m uniform in [1, 2), e uniform in [emin, emax];
    a fraction ``sub_frac`` of entries take e in [-149, -127] (subnormal).
    Formed in fp64 and rounded to fp32 by numpy (nearest-even)."""
    sign = np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    m = 1.0 + rng.random(size=shape)
    e = rng.integers(emin, emax + 1, size=shape)
    sub = rng.random(size=shape) < sub_frac
    e_sub = rng.integers(-149, -126, size=shape)
    e = np.where(sub, e_sub, e)
    fmax = float(np.finfo(np.float32).max)
    return np.clip(sign * np.ldexp(m, e), -fmax, fmax).astype(np.float32)


@dataclass
class Workload:
    """One configuration: operands plus the K-shard plan where one applies."""
    name: str
    dtype: str                     # "f32" or "bf16"
    x: np.ndarray                  # float32 [M, K] or uint16 bf16 bits
    w: np.ndarray                  # float32 [N, K] or uint16 bf16 bits
    cuts: List[int] = field(default_factory=list)       # K-shard boundaries
    fold: List[Tuple[int, int]] = field(default_factory=list)  # fold-tree picks
    note: str = ""

    @property
    def shape(self) -> Tuple[int, int, int]:
        return self.x.shape[0], self.w.shape[0], self.x.shape[1]

    def bits(self) -> Tuple[np.ndarray, np.ndarray]:
        if self.dtype == "f32":
            return f32_bits(self.x), f32_bits(self.w)
        return self.x, self.w


def c1_small_f32(seed: int = 0) -> Workload:
    """f32 64x64, K=256, x and w iid uniform[-1, 1); shards split at k=100."""
    rng = np.random.default_rng(seed)
    x = rng.random((64, 256), dtype=np.float32) * np.float32(2) - np.float32(1)
    w = rng.random((64, 256), dtype=np.float32) * np.float32(2) - np.float32(1)
    return Workload("f32 64x64x256 uniform[-1,1)", "f32", x, w, cuts=[100])


def c2_bf16_cancel(seed: int = 1, n: int = 1024) -> Workload:
    """bf16 n^3, N(0,1) drawn in fp32 then rounded; 10% of w's k-columns are the
    exact negation of another column (targets and sources from one permutation)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, n), dtype=np.float32)
    w = rng.standard_normal((n, n), dtype=np.float32)
    perm = rng.permutation(n)
    nt = n // 10
    targets, sources = perm[:nt], perm[nt:2 * nt]
    w[:, targets] = -w[:, sources]
    return Workload(f"bf16 {n}^3 N(0,1), 10% negated w columns", "bf16",
                    to_bf16_bits(x), to_bf16_bits(w),
                    note=f"targets={targets.tolist()} sources={sources.tolist()}")


def c3_wide_f32(seed: int = 2, n: int = 4096) -> Workload:
    """f32 n^3, entries sign*m*2^e, e in [-70, 70], 1% subnormal entries."""
    rng = np.random.default_rng(seed)
    x = wide_range_f32(rng, (n, n))
    w = wide_range_f32(rng, (n, n))
    return Workload(f"f32 {n}^3 wide range e in [-70,70], 1% subnormal", "f32", x, w)


def c4_ksharded_f32(seed: int = 3, m: int = 2048, k: int = K_MAX, nshards: int = 16) -> Workload:
    """f32 m x m, K = k, N(0,1); K cut into ``nshards`` at seeded random
    boundaries and a seeded random fold tree over the shard partials: at each
    step two list positions (i, j) are drawn and replaced by their combine."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    w = rng.standard_normal((m, k), dtype=np.float32)
    cuts = sorted(int(c) for c in rng.choice(np.arange(1, k), nshards - 1, replace=False))
    fold = []
    live = nshards
    while live > 1:
        i, j = (int(v) for v in rng.choice(live, 2, replace=False))
        fold.append((i, j))
        live -= 1
    return Workload(f"f32 {m}x{m}, K={k}, {nshards} K-shards, random fold tree", "f32",
                    x, w, cuts=cuts, fold=fold)


def c5_detlinear_bf16(seed: int = 4, tokens: int = 8192, d_in: int = 4096,
                      d_out: int = 4096) -> Workload:
    """DetLinear d_in -> d_out in bf16: x [tokens, d_in] ~ N(0,1),
    W [d_out, d_in] ~ N(0, 1/d_in) (N(0,1)/64 for 4096), both rounded to bf16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, d_in), dtype=np.float32)
    W = rng.standard_normal((d_out, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in))
    return Workload(f"DetLinear {d_in}->{d_out} bf16, {tokens} tokens", "bf16",
                    to_bf16_bits(x), to_bf16_bits(W))


def apply_fold(parts: list, fold: List[Tuple[int, int]], combine) -> object:
    """Replay a fold tree: each (i, j) replaces list entries i and j by
    combine([a_i, a_j]) appended at the end.  Returns the last remaining item."""
    live = list(parts)
    for i, j in fold:
        a, b = live[i], live[j]
        live = [p for t, p in enumerate(live) if t not in (i, j)]
        live.append(combine([a, b]))
    assert len(live) == 1
    return live[0]


def shard_bounds(k: int, cuts: List[int]) -> List[Tuple[int, int]]:
    edges = [0] + list(cuts) + [k]
    return [(edges[i], edges[i + 1]) for i in range(len(edges) - 1)]


def random_operands(rng: np.random.Generator, M: int, N: int, K: int, dtype: str,
                    kind: str = "normal") -> Tuple[np.ndarray, np.ndarray]:
    """Operands for tests, as bit patterns (uint32 for f32, uint16 for bf16).

    kinds: "normal" N(0,1); "uniform" [-1,1); "wide" sign*m*2^e over the whole
    finite exponent range with subnormals; "special" a mix of zeros, +-0,
    subnormals, the largest finite values and powers of two; "int" small
    integers in [-1024, 1024]."""
    def draw(shape):
        if kind == "normal":
            return rng.standard_normal(shape, dtype=np.float32)
        if kind == "uniform":
            return rng.random(shape, dtype=np.float32) * np.float32(2) - np.float32(1)
        if kind == "int":
            return rng.integers(-1024, 1025, size=shape).astype(np.float32)
        if kind == "wide":
            return wide_range_f32(rng, shape, emin=-126, emax=127, sub_frac=0.05)
        if kind == "special":
            pool = np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -149, -(2.0 ** -149), 2.0 ** -126,
                             3.0 * 2.0 ** -140, float(np.finfo(np.float32).max),
                             -float(np.finfo(np.float32).max), 2.0 ** 100, -(2.0 ** -100),
                             1.5, 0.75, 2.0 ** 64, 2.0 ** -64], dtype=np.float64)
            v = pool[rng.integers(0, pool.size, size=shape)].astype(np.float32)
            mix = rng.random(shape) < 0.5
            return np.where(mix, wide_range_f32(rng, shape, -126, 127, 0.1), v).astype(np.float32)
        raise ValueError(kind)
    x, w = draw((M, K)), draw((N, K))
    if dtype == "bf16":   # keep values below the bf16 overflow threshold
        bmax = np.float32(2.0 ** 128 - 2.0 ** 120)
        x, w = np.clip(x, -bmax, bmax), np.clip(w, -bmax, bmax)
    if dtype == "f32":
        return f32_bits(x), f32_bits(w)
    if dtype == "bf16":
        return to_bf16_bits(x), to_bf16_bits(w)
    raise ValueError(dtype)
