"""Seeded sweep of attention shapes across every launch variant.

Each case draws a head size, batch, head count, lengths (straddling the
launch boundaries: rows of at most 128 and 256 keys, the streaming kernel's
32-key tiles and 128/256-query workgroups, causal rows up to and past 2048
queries), a mask and, for self-attention, possibly a restricted-attention
window, then compares sampled output rows (plus every batch row's first and
last query) with the fp64 oracle (oracle_attention_rows), bf16 to
1e-2 + 1e-2|o|.  A few fp32 cases compare the whole output to 1e-5.  The
cases are fixed by their seed, so a failure names a reproducible shape.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_scaled_dot_fwd_amd as mha
from gpu_util import check, device, say
from workloads import generate

pytestmark = pytest.mark.gpu

NONE, PAD, CAUSAL = mha.MASK_NONE, mha.MASK_KEY_PADDING, mha.MASK_CAUSAL

# length bands: tiny, around the 128-key and 256-key short-row limits, and
# streaming lengths around the 2048-query causal switch
BANDS = [(1, 40), (96, 160), (200, 300), (300, 1100), (1900, 2200)]


def draw_case(i):
    rng = np.random.Generator(np.random.PCG64(71000 + i))
    d = int(rng.choice([16, 32, 64, 64, 128]))
    lo, hi = BANDS[int(rng.integers(0, len(BANDS)))]
    L = int(rng.integers(lo, hi + 1))
    big = L > 1000
    B = int(rng.integers(1, 3 if big else 4))
    h = int(rng.integers(1, 3 if big else 7))
    cross = bool(rng.random() < 0.3)
    if cross:
        lo2, hi2 = BANDS[int(rng.integers(0, len(BANDS) - 1))]
        Lk = int(rng.integers(lo2, hi2 + 1))
        mask = int(rng.choice([NONE, PAD]))
        window = None
    else:
        Lk = L
        mask = int(rng.choice([NONE, PAD, CAUSAL, PAD | CAUSAL]))
        window = int(rng.integers(0, 300)) if rng.random() < 0.3 else None
    lens = [int(x) for x in rng.integers(0, Lk + 6, B)]
    if B > 1:
        lens[0] = Lk  # at least one full row
    return dict(d=d, B=B, h=h, Lq=L, Lk=Lk, mask=mask, window=window, lens=lens, seed=71000 + i)


N_BF16 = 40
# and the launch boundaries themselves (d = 64): causal rows at and just past
# 2048 queries, rows of 128/129 and 256/257 keys, a window on a short row
EDGES = [dict(d=64, B=1, h=2, Lq=2049, Lk=2049, mask=CAUSAL, window=None, lens=[2049]),
         dict(d=64, B=2, h=2, Lq=2048, Lk=2048, mask=PAD | CAUSAL, window=None, lens=[2048, 1000]),
         dict(d=64, B=2, h=3, Lq=129, Lk=129, mask=NONE, window=None, lens=[129, 129]),
         dict(d=64, B=2, h=3, Lq=128, Lk=128, mask=PAD, window=None, lens=[128, 31]),
         dict(d=64, B=1, h=2, Lq=257, Lk=257, mask=CAUSAL, window=None, lens=[257]),
         dict(d=64, B=2, h=2, Lq=256, Lk=256, mask=PAD, window=1, lens=[256, 100])]
CASES = [draw_case(i) for i in range(N_BF16)] + [dict(c, seed=71900 + n) for n, c in enumerate(EDGES)]


def label(c):
    w = "" if c["window"] is None else f"_w{c['window']}"
    return f"d{c['d']}_B{c['B']}_h{c['h']}_Lq{c['Lq']}_Lk{c['Lk']}_m{c['mask']}{w}"


def sample_rows(B, h, Lq, n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = np.stack([rng.integers(0, B, n), rng.integers(0, h, n), rng.integers(0, Lq, n)], 1)
    edges = [(b, t, i) for b in range(B) for t in (0, h - 1) for i in (0, Lq - 1)]
    return np.concatenate([rows, np.array(edges)]).astype(np.int64)


@pytest.mark.parametrize("case", CASES, ids=label)
def test_shape_sweep_bf16(case):
    dev = device()
    c = case
    say(f"case shape sweep {label(c)} seed={c['seed']}")
    q = generate.normal((c["B"], c["Lq"], c["h"], c["d"]), c["seed"] * 10 + 1, "bf16")
    k = generate.normal((c["B"], c["Lk"], c["h"], c["d"]), c["seed"] * 10 + 2, "bf16")
    v = generate.normal((c["B"], c["Lk"], c["h"], c["d"]), c["seed"] * 10 + 3, "bf16")
    lens = torch.tensor(c["lens"], dtype=torch.int32)
    use_lens = bool(c["mask"] & PAD)
    o = mha.mha_forward(q.to(dev), k.to(dev), v.to(dev), mask=c["mask"],
                        kv_lens=lens.to(dev) if use_lens else None, window=c["window"])
    torch.cuda.synchronize()
    rows = sample_rows(c["B"], c["h"], c["Lq"], 64, c["seed"] * 10 + 4)
    ref = oracle.attention_rows(q, k, v, rows, mask=c["mask"],
                                kv_lens=lens if use_lens else None, window=c["window"])
    got = o.cpu()[rows[:, 0], rows[:, 2], rows[:, 1]]
    check(got, ref, "bf16", label(c))
    if use_lens:
        # a batch row with no legal key outputs exact zeros
        for b in range(c["B"]):
            if min(c["lens"][b], c["Lk"]) <= 0:
                assert torch.equal(o[b].cpu(), torch.zeros_like(o[b].cpu()))


F32_CASES = [dict(d=d, B=2, h=3, Lq=Lq, Lk=Lk, mask=m, window=w, lens=[Lk, max(Lk // 3, 0)],
                  seed=72000 + n)
             for n, (d, Lq, Lk, m, w) in enumerate([(8, 17, 17, CAUSAL, None), (16, 70, 33, PAD, None),
                                                      (32, 130, 130, PAD | CAUSAL, 9),
                                                      (64, 65, 65, NONE, 20), (64, 100, 190, PAD, None),
                                                      (64, 300, 300, CAUSAL, None),
                                                      (16, 257, 257, PAD | CAUSAL, 40),
                                                      (8, 129, 300, PAD, None)])]


@pytest.mark.parametrize("case", F32_CASES, ids=label)
def test_shape_sweep_f32(case):
    dev = device()
    c = case
    say(f"case shape sweep fp32 {label(c)} seed={c['seed']}")
    q = generate.normal((c["B"], c["Lq"], c["h"], c["d"]), c["seed"] * 10 + 1, "f32")
    k = generate.normal((c["B"], c["Lk"], c["h"], c["d"]), c["seed"] * 10 + 2, "f32")
    v = generate.normal((c["B"], c["Lk"], c["h"], c["d"]), c["seed"] * 10 + 3, "f32")
    lens = torch.tensor(c["lens"], dtype=torch.int32)
    use_lens = bool(c["mask"] & PAD)
    o = mha.mha_forward(q.to(dev), k.to(dev), v.to(dev), mask=c["mask"],
                        kv_lens=lens.to(dev) if use_lens else None, window=c["window"])
    torch.cuda.synchronize()
    ref = oracle.attention(q, k, v, mask=c["mask"], kv_lens=lens if use_lens else None,
                           window=c["window"])
    check(o.cpu(), ref, "f32", label(c))
