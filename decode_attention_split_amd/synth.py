"""Seeded synthetic inputs for decode attention.

This module holds no attention arithmetic: it only draws seeded random numbers in a
fixed order and rounds them to bf16.  Both the GPU path and the fp64 oracle consume
exactly these tensors.

Recipe (one workload, one seed):
  * ``ctx_lens`` -- integers uniform on [lo, hi], both ends included;
  * ``q``        -- N(0,1) float32 samples rounded to bf16 (round to nearest even);
  * ``K`` then ``V`` caches -- N(0,1) float32 -> bf16, every physical slot filled.
The draws come from one ``torch.Generator`` in the order ctx_lens, q, K, V.
"""
from __future__ import annotations

import numpy as np
import torch


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def uniform_int(gen: torch.Generator, n: int, lo: int, hi: int, device="cpu") -> torch.Tensor:
    """n integers uniform on [lo, hi] inclusive, int32."""
    return torch.randint(int(lo), int(hi) + 1, (int(n),), generator=gen, device=device,
                         dtype=torch.int64).to(torch.int32)


def normal_bf16(gen: torch.Generator, shape, device="cpu") -> torch.Tensor:
    """N(0,1) float32 samples rounded to bf16 by round-to-nearest-even."""
    return torch.randn(tuple(shape), generator=gen, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 tensor, as a host numpy array."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bf16 tensor")
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, device="cpu") -> torch.Tensor:
    """bf16 tensor whose bits are the given uint16 array."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)


BF16_NAN = 0x7FC0  # quiet NaN bit pattern, used only to poison never-valid slots
