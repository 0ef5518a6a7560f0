"""Helpers for the GPU parity tests: moving bit patterns to and from torch
device tensors, and naming each case before it runs (so a run that dies
leaves the name of its last case in the log)."""
import hashlib
import sys

import numpy as np
import torch


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def device() -> torch.device:
    return torch.device("cuda:0")


def to_device(bits: np.ndarray, dtype: str) -> torch.Tensor:
    """uint32 fp32 bits or uint16 bf16 bits -> float32/bfloat16 device tensor."""
    bits = np.ascontiguousarray(bits)
    if dtype == "f32":
        return torch.from_numpy(bits.view(np.float32)).to(device())
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device())


def f32_bits(y: torch.Tensor) -> np.ndarray:
    return y.detach().cpu().contiguous().view(torch.int32).numpy().view(np.uint32)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return f32_bits(t)


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def mismatch_report(got: np.ndarray, want: np.ndarray, limit: int = 5) -> str:
    bad = np.argwhere(got != want)
    lines = [f"{len(bad)} of {got.size} differ"]
    for idx in bad[:limit]:
        t = tuple(int(i) for i in idx)
        lines.append(f"  at {t}: got {got[t]!r} want {want[t]!r}")
    return "\n".join(lines)
