"""GPU parity on inputs that make the online softmax rescale mid-row.

The staircase inputs (tests/rescale_cases.py) raise a row's logits in
steps along the key axis, so its running maximum grows by up to ~40
base-2 units several times per row, and by 6-8 units (just under the
rescale threshold) elsewhere.  Every launch variant is driven through the
C ABI (short rows with 4 and 8 tiles, the streaming kernel with 32 and 64
queries per wave, head sizes 16/32/128, restricted attention, fp32, the
fused projection kernel and the decoding step's split over the cache) and
compared element by element with the fp64 oracle at the bf16 bound
1e-2 + 1e-2 |o| (fp32: 1e-5).  Section 04 of "Paper Deep Reading:
Attention Is All You Need" explains why large logits are the softmax's
hard case.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_scaled_dot_fwd_amd as mha
from gpu_util import check, device, say, to_np
from rescale_cases import CASES, HUGE_CASES, climbs, growths, inputs
from workloads import generate

pytestmark = pytest.mark.gpu


def _rows(c, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 3, 31, 32, 255, 256, 257, c.Lq // 2, c.Lq - 2, c.Lq - 1]
    rows = []
    for b in range(c.B):
        for t in sorted({0, 1, c.h // 2, c.h - 1, int(rng.integers(0, c.h))}):
            idx = [i for i in fixed if 0 <= i < c.Lq] + list(rng.integers(0, c.Lq, n))
            rows += [(b, t, int(i)) for i in idx]
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.label())
def test_rescale_mid_row(case):
    dev = device()
    say(f"case rescale {case.label()}")
    q, k, v, lens = inputs(case, 7000)
    o = mha.mha_forward(q.to(dev), k.to(dev), v.to(dev), mask=case.mask,
                        kv_lens=None if lens is None else lens.to(dev), window=case.window)
    torch.cuda.synchronize()
    if case.sampled:
        rows = _rows(case, 24, 17)
        ref = oracle.attention_rows(q, k, v, rows, mask=case.mask, kv_lens=lens,
                                    window=case.window)
        o_np = to_np(o)
        check(np.stack([o_np[b, i, t] for (b, t, i) in rows]), ref, case.dtype,
              f"{case.label()} ({len(rows)} rows)")
    else:
        ref, s = oracle.attention(q, k, v, mask=case.mask, kv_lens=lens, window=case.window,
                                  return_s=True)
        g = growths(s)
        assert (g > 8).sum() > 0, "the inputs must make the running maximum jump"
        check(o, ref, case.dtype, case.label(), f32_atol=f32_bound(q, k, v, s))


def f32_bound(q, k, v, s):
    """The fp32 bound for staircase inputs.  The 1e-5 of the fp32 runs is
    stated for N(0, 1) inputs, whose raw dot products q.k stay near 8; here
    they reach ~520.  Rounding the dot product's running sum in fp32
    (unit roundoff u = 2^-24, about sqrt(d) = 8 roundings of a sum of that
    size) moves a scaled logit by up to 8 u max|q.k| / sqrt(d), and a
    logit error e moves a softmax average of V by at most 2 e max|v|."""
    d = q.shape[-1]
    u = 2.0 ** -24
    raw_max = float(np.nanmax(np.abs(np.where(np.isfinite(s), s, 0.0)))) * np.sqrt(d)
    vmax = float(v.abs().max())
    return 1e-5 + 2.0 * (8 * u * raw_max / np.sqrt(d)) * vmax


@pytest.mark.parametrize("mask", [0, 1, 2, 3])
@pytest.mark.parametrize("shape", [(4, 128, 512, 8), (3, 100, 1024, 16)])
def test_rescale_mid_row_fused_projection(shape, mask):
    """The fused projection + attention kernel on a block whose projected
    queries and keys carry the staircase in channel 0 of every head."""
    dev = device()
    B, L, dm, h = shape
    say(f"case rescale fused {shape} mask={mask}")
    x = generate.normal((B, L, dm), 7200 + dm, "bf16")
    ws = [generate.normal((dm, h * 64), 7201 + dm + i, "bf16", std=dm ** -0.5) for i in range(3)]
    x, wq, wk, wv = generate.staircase_block(x, *ws, h=h)
    lens = torch.tensor([[L, L - 9, L // 2 + 5][i % 3] for i in range(B)], dtype=torch.int32)
    xd, wd = x.to(dev), [w.to(dev) for w in (wq, wk, wv)]
    o = mha.mha_self_attention_fused(xd, *wd, h=h, mask=mask, kv_lens=lens.to(dev))
    assert o is not None
    qd, kd, vd = mha.mha_project_qkv(xd, xd, *wd, h=h)
    two_call = mha.mha_forward(qd, kd, vd, mask=mask, kv_lens=lens.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), two_call.cpu())
    # The fused kernel reproduces the two calls, whose Q, K and V are bf16
    # tensors: the oracle composes its fp64 projection, the same rounding
    # to bf16 (nearest even) and its fp64 attention.  With the staircase's
    # sharply peaked rows, comparing against unrounded fp64 projections
    # would charge the bf16 storage of Q/K/V to the attention.
    rq, rk, rv = (torch.from_numpy(t).to(torch.bfloat16)
                  for t in oracle.project_qkv(x, x, wq, wk, wv, h=h))
    ref, s = oracle.attention(rq, rk, rv, mask=mask, kv_lens=lens, return_s=True)
    assert (growths(s) > 8).sum() > 0
    check(o, ref, "bf16", f"fused {shape} m={mask}")


@pytest.mark.parametrize("d", [64, 128])
def test_rescale_across_decode_chunks(d):
    """The decoding step: keys rising across the 1024-key chunks of the
    split, so later chunks' maxima dominate the merge."""
    dev = device()
    B, h, L = 4, 8, 3100
    say(f"case rescale decode d={d}")
    q = generate.normal((B, 1, h, d), 7300 + d, "bf16")
    k = generate.normal((B, L, h, d), 7301 + d, "bf16")
    v = generate.normal((B, L, h, d), 7302 + d, "bf16")
    qs = torch.cat([q] * 4, dim=1)          # amplitudes 0, 1, 4, 8 in rows 0..3
    qs, k = generate.staircase(qs, k)
    lens = torch.tensor([L, 2900, 2049, 1500], dtype=torch.int32)
    for row in range(4):
        qr = qs[:, row:row + 1].contiguous()
        o = mha.mha_decode(qr.to(dev), k.to(dev), v.to(dev), lens.to(dev))
        torch.cuda.synchronize()
        check(o, oracle.attention(qr, k, v, mask=1, kv_lens=lens), "bf16",
              f"decode d={d} amplitude {generate.STAIRCASE_AMPS[row]}")


@pytest.mark.parametrize("case", HUGE_CASES, ids=lambda c: c.label())
def test_rows_climbing_past_the_fp32_range(case):
    """Rows whose maximum climbs ~188 base-2 units above their first tiles:
    the streaming kernel's reference, fixed at the first tiles, would
    overflow for them, so they take the recomputation with a moving
    reference; their neighbours in the same waves keep their results."""
    dev = device()
    say(f"case climb {case.label()}")
    q, k, v, lens = inputs(case, 7400)
    o = mha.mha_forward(q.to(dev), k.to(dev), v.to(dev), mask=case.mask,
                        kv_lens=None if lens is None else lens.to(dev), window=case.window)
    torch.cuda.synchronize()
    ref, s = oracle.attention(q, k, v, mask=case.mask, kv_lens=lens, window=case.window,
                              return_s=True)
    assert (climbs(s, 2 if case.window is not None else 1) > 130).sum() > 0
    check(o, ref, case.dtype, case.label())
