"""Seeded synthetic inputs.

Random numbers only: numpy ``Generator(PCG64(seed))`` draws fp32
``standard_normal`` values (or uniform integers for lengths); bf16 tensors are
the RNE rounding of those fp32 draws done by ``torch.Tensor.to``.  Both the
HIP path and the oracle receive exactly these values (the oracle upcasts them
to fp64 without rounding).  Nothing here computes any part of attention.
"""
from __future__ import annotations

import numpy as np
import torch

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def normal(shape, seed: int, dtype: str = "bf16", std: float = 1.0) -> torch.Tensor:
    """i.i.d. N(0, std^2) fp32 draws from PCG64(seed), cast to ``dtype``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        a = (a * np.float32(std)).astype(np.float32)
    return torch.from_numpy(a).to(_DTYPES[dtype]).contiguous()


def lengths(batch: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """int32 [batch], uniform on the integers lo..hi inclusive."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return torch.from_numpy(rng.integers(lo, hi + 1, size=batch).astype(np.int32))
