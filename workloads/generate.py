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


# Levels of the staircase below: (fraction of the key axis where the level
# starts, level; every level is exact in bf16).  The steps up are 5.25, 6,
# 20, 5.5 and 27.75; one step goes down.  With amplitude 8 at d = 64 a step of x raises the scaled logits of
# the keys after it by x, i.e. by x log2(e) in base-2 exponent units: the
# steps of 5.25 and 5.5 stay just under 8 such units, the others exceed it.
STAIRCASE_LEVELS = ((0.0, 0.0), (0.12, 5.25), (0.25, 11.25), (0.37, 1.25), (0.5, 31.25),
                    (0.62, 36.75), (0.75, 64.5))
STAIRCASE_AMPS = (0.0, 1.0, 4.0, 8.0)
# A staircase that climbs far higher: 130 scaled-logit units above its start
# at amplitude 8 (about 188 base-2 units), with steps of 30, 70 and 30.
STAIRCASE_HUGE_LEVELS = ((0.0, 0.0), (0.3, 30.0), (0.6, 100.0), (0.8, 130.0))


def staircase(q: torch.Tensor, k: torch.Tensor, levels=STAIRCASE_LEVELS,
              amps=STAIRCASE_AMPS) -> tuple:
    """Copies of q [B, Lq, h, d] and k [B, Lk, h, d] with channel 0 of
    every head overwritten: q[:, i, :, 0] = amps[i % len(amps)] and
    k[:, j, :, 0] = level(j) * sqrt(d) / 8, level(j) being the last entry
    of ``levels`` whose start fraction is at most j / Lk.

    Input construction only (nothing of attention is computed): keys
    further along the axis carry larger first components, so a query's
    logits rise in steps along the key axis, by amounts that depend on the
    query's amplitude (0 leaves its logits i.i.d.)."""
    q = q.clone()
    k = k.clone()
    Lq, Lk, d = q.shape[1], k.shape[1], q.shape[3]
    a = torch.tensor([amps[i % len(amps)] for i in range(Lq)], dtype=torch.float32)
    lv = torch.from_numpy(staircase_levels(Lk, levels) * np.float32(np.sqrt(d) / 8.0))
    q[:, :, :, 0] = a.to(q.dtype)[None, :, None]
    k[:, :, :, 0] = lv.to(k.dtype)[None, :, None]
    return q.contiguous(), k.contiguous()


def staircase_levels(L: int, levels=STAIRCASE_LEVELS) -> np.ndarray:
    """fp32 [L]: level(j) of the staircase for positions j = 0 .. L-1."""
    lv = np.zeros(L, dtype=np.float32)
    for start, level in levels:
        lv[int(np.ceil(start * L)):] = level
    return lv


def staircase_block(x: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor,
                    h: int, levels=STAIRCASE_LEVELS, amps=STAIRCASE_AMPS) -> tuple:
    """The staircase of ``staircase`` carried through the projections of a
    self-attention block: copies of x [B, L, d_model] and of the weights
    [d_model, h*64] in which column 0 of x holds amps[i % len(amps)],
    column 1 holds level(i), W^Q has a single 1 (row 0) in column 64t of
    every head t and W^K a single 1 (row 1) there, and rows 0 and 1 of
    every weight are zero elsewhere.  The projections then carry the two
    columns into channel 0 of every head's queries and keys exactly, with
    no rounding, and nowhere else."""
    x, w_q, w_k, w_v = (t.clone() for t in (x, w_q, w_k, w_v))
    L = x.shape[1]
    a = torch.tensor([amps[i % len(amps)] for i in range(L)], dtype=torch.float32)
    x[:, :, 0] = a.to(x.dtype)[None, :]
    x[:, :, 1] = torch.from_numpy(staircase_levels(L, levels)).to(x.dtype)[None, :]
    for w in (w_q, w_k, w_v):
        w[0:2, :] = 0
    for t in range(h):
        w_q[:, 64 * t] = 0
        w_k[:, 64 * t] = 0
        w_q[0, 64 * t] = 1
        w_k[1, 64 * t] = 1
    return x.contiguous(), w_q.contiguous(), w_k.contiguous(), w_v.contiguous()
