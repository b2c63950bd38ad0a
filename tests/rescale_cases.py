"""Inputs whose logits rise in steps along the key axis, and the cases that
route them through every attention launch variant.

The online softmax keeps a running row maximum and, when a 32-key tile's
maximum exceeds it by more than 8 base-2 exponent units, rescales the
partial output and row sum (the exact identity softmax(x) = softmax(x - c),
"Paper Deep Reading: Attention Is All You Need", section 04, on why the
logits are scaled: large logits saturate the softmax).  With i.i.d. N(0, 1)
inputs the maximum settles after the first tile and that branch never runs;
the staircase inputs (workloads.generate.staircase) make it run several
times per row, with steps just under the threshold too.

``growths`` measures, from the oracle's scaled logits, how far the true
running maximum grows at each tile after a row's first legal one; a growth
above 8 there means the kernel's (possibly stale) maximum is exceeded by
more than 8 as well, so the rescale runs.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from workloads import generate

NONE, PAD, CAUSAL = 0, 1, 2
LOG2E = 1.4426950408889634
KT = 32  # keys per tile in every bf16 attention kernel


@dataclasses.dataclass(frozen=True)
class Case:
    name: str          # the launch variant the shape selects
    B: int
    h: int
    Lq: int
    Lk: int
    d: int
    mask: int
    dtype: str = "bf16"
    window: Optional[int] = None
    sampled: bool = False   # compare sampled rows (the oracle's full run is slow)
    huge: bool = False      # the staircase that climbs ~188 base-2 units

    def label(self):
        w = "" if self.window is None else f" w={self.window}"
        hg = " huge" if self.huge else ""
        return (f"{self.name} B={self.B} h={self.h} Lq={self.Lq} Lk={self.Lk} d={self.d} "
                f"mask={self.mask}{w} {self.dtype}{hg}")


def tiles_name(name: str, mask: int, Lq: int) -> str:
    """The streaming kernel's query tile for a d = 64 shape without a
    window: 128 queries for causal rows up to 2048, 256 otherwise."""
    q = 128 if (mask & CAUSAL) and Lq <= 2048 else 256
    return f"{name}, {q}-query tiles"


def _cases():
    out = []
    for m in (NONE, PAD, CAUSAL, PAD | CAUSAL):
        # rows of at most 128 keys: whole row in LDS, four tiles
        out.append(Case("short rows NT=4", 3, 2, 128, 128, 64, m))
        # at most 256 keys: eight tiles
        out.append(Case("short rows NT=8", 3, 2, 256 if m & CAUSAL else 200, 256, 64, m))
    for m in (NONE, CAUSAL, PAD | CAUSAL):
        # the streaming kernel (rows above 256 keys): 256-query workgroups
        # without a mask, 128-query ones for causal rows up to 2048
        out.append(Case(tiles_name("long rows", m, 700), 2, 2, 700, 700, 64, m))
    out.append(Case(tiles_name("long rows causal", CAUSAL, 2200), 1, 2, 2200, 2200, 64, CAUSAL))
    out.append(Case("long rows, many heads", 2, 80, 768, 768, 64, NONE, sampled=True))
    out.append(Case("long rows, many heads, padded", 2, 80, 768, 768, 64, PAD, sampled=True))
    for d in (16, 32, 128):
        for m in (NONE, CAUSAL):
            out.append(Case(f"head size {d}", 2, 2, 600, 600, d, m))
    for d in (64, 128):
        for m in (NONE, CAUSAL):
            out.append(Case(f"restricted attention d={d}", 2, 2, 1024, 1024, d, m, window=200))
    for m in (NONE, CAUSAL, PAD):
        out.append(Case("fp32", 2, 2, 300, 300, 64, m, dtype="f32"))
    return out


def _huge_cases():
    """The huge staircase through the streaming kernels (rows longer than
    256 keys): its rows climb far enough above their first tiles that a
    reference fixed there would overflow."""
    out = []
    for m in (NONE, PAD, CAUSAL, PAD | CAUSAL):
        out.append(Case(tiles_name("long rows", m, 700), 2, 2, 700, 700, 64, m, huge=True))
    out.append(Case(tiles_name("long rows causal", CAUSAL, 2200), 1, 2, 2200, 2200, 64, CAUSAL,
                    huge=True))
    for m in (NONE, CAUSAL):
        out.append(Case("restricted attention", 2, 2, 1024, 1024, 64, m, window=300, huge=True))
    out.append(Case("restricted attention", 2, 2, 1024, 1024, 128, NONE, window=300, huge=True))
    for d in (16, 32, 128):
        out.append(Case(f"head size {d}", 2, 2, 600, 600, d, CAUSAL, huge=True))
    out.append(Case("head size 128", 2, 2, 600, 600, 128, PAD, huge=True))
    return out


HUGE_CASES = _huge_cases()


CASES = _cases()


def lengths(c: Case):
    """Key lengths of a case: full rows and a few ragged ones."""
    choices = [c.Lk, c.Lk - 7, max(c.Lk // 2 + 3, 1), c.Lk - 31]
    return torch.tensor([choices[i % len(choices)] for i in range(c.B)], dtype=torch.int32)


def inputs(c: Case, seed: int):
    q = generate.normal((c.B, c.Lq, c.h, c.d), seed, c.dtype)
    k = generate.normal((c.B, c.Lk, c.h, c.d), seed + 1, c.dtype)
    v = generate.normal((c.B, c.Lk, c.h, c.d), seed + 2, c.dtype)
    if c.huge:
        q, k = generate.staircase(q, k, levels=generate.STAIRCASE_HUGE_LEVELS)
    else:
        q, k = generate.staircase(q, k)
    return q, k, v, (lengths(c) if c.mask & PAD else None)


def growths(s: np.ndarray) -> np.ndarray:
    """s: scaled logits [..., Lq, Lk] with -inf at masked pairs.  Returns
    the growths (base-2 units) of every row's running maximum over 32-key
    tiles, at each tile after the row's first legal tile."""
    s = np.asarray(s, dtype=np.float64) * LOG2E
    Lk = s.shape[-1]
    nt = (Lk + KT - 1) // KT
    pad = nt * KT - Lk
    if pad:
        s = np.concatenate([s, np.full(s.shape[:-1] + (pad,), -np.inf)], axis=-1)
    tmax = s.reshape(s.shape[:-1] + (nt, KT)).max(axis=-1)     # [..., Lq, nt]
    run = np.maximum.accumulate(tmax, axis=-1)
    prev = run[..., :-1]
    with np.errstate(invalid="ignore"):  # -inf - -inf past a band's end
        g = tmax[..., 1:] - prev
    ok = np.isfinite(prev) & np.isfinite(g)
    return g[ok]


def climbs(s: np.ndarray, first_tiles: int = 1) -> np.ndarray:
    """s: scaled logits [..., Lq, Lk] (-inf at masked pairs).  For every
    row with a legal key, how far (base-2 units) its maximum rises above
    the maximum of its first `first_tiles` 32-key tiles that hold a legal
    key."""
    s = np.asarray(s, dtype=np.float64) * LOG2E
    Lk = s.shape[-1]
    nt = (Lk + KT - 1) // KT
    pad = nt * KT - Lk
    if pad:
        s = np.concatenate([s, np.full(s.shape[:-1] + (pad,), -np.inf)], axis=-1)
    tmax = s.reshape(-1, nt, KT).max(axis=-1)          # [rows, nt]
    out = []
    for row in tmax:
        legal = np.nonzero(np.isfinite(row))[0]
        if legal.size == 0:
            continue
        first = row[legal[0]:legal[0] + first_tiles].max()
        out.append(row.max() - first)
    return np.array(out)
