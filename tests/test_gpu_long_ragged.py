"""Long rows with ragged tails in the streaming kernel (rows above 256 keys).

The sweep shapes are multiples of 256 (the streaming kernel's queries per
workgroup) and of its 32-key tiles, so these cases put ragged query and key
tails, and cross-attention (Lq != Lk), through it.  The oracle evaluates
sampled rows one by one (oracle_attention_rows) on the full-size inputs,
including each sequence's last query row.
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

# (B, h, Lq, Lk, masks): long cross-attention and self-attention with ragged
# query and key tails; 256-query workgroups except causal rows up to 2048
# queries (the last case), which take 128-query ones.
CASES = [(7, 8, 2100, 3000, (NONE, PAD)), (2, 4, 2300, 2300, (CAUSAL, PAD | CAUSAL)),
         (3, 4, 700, 1900, (NONE, PAD)), (3, 4, 1500, 1500, (CAUSAL, PAD | CAUSAL))]


def sample_rows(B, h, Lq, n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = np.stack([rng.integers(0, B, n), rng.integers(0, h, n), rng.integers(0, Lq, n)], 1)
    edges = [(b, t, i) for b in (0, B - 1) for t in (0, h - 1) for i in (0, Lq - 1, Lq - 2)]
    return np.concatenate([rows, np.array(edges)]).astype(np.int64)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_h{}_Lq{}_Lk{}".format(*c[:4]))
def test_long_ragged_rows(case):
    dev = device()
    B, h, Lq, Lk, masks = case
    q = generate.normal((B, Lq, h, 64), 9300 + Lq, "bf16")
    k = generate.normal((B, Lk, h, 64), 9301 + Lk, "bf16")
    v = generate.normal((B, Lk, h, 64), 9302 + Lk, "bf16")
    choices = [Lk, 1, Lk - 1, 0, Lk + 9, Lk // 2 + 3, 257]
    lens = torch.tensor([choices[i % len(choices)] for i in range(B)], dtype=torch.int32)
    rows = sample_rows(B, h, Lq, 96, 9303 + Lq)
    for mask in masks:
        say(f"case long ragged B={B} h={h} Lq={Lq} Lk={Lk} mask={mask}")
        o = mha.mha_forward(q.to(dev), k.to(dev), v.to(dev), mask=mask,
                            kv_lens=lens.to(dev) if mask & PAD else None)
        torch.cuda.synchronize()
        ref = oracle.attention_rows(q, k, v, rows, mask=mask,
                                    kv_lens=lens if mask & PAD else None)
        got = o.cpu()[rows[:, 0], rows[:, 2], rows[:, 1]]
        check(got, ref, "bf16", f"long ragged {case[:4]} mask={mask}")
        if mask & PAD:
            for b in range(B):
                if int(lens[b]) <= 0:
                    assert torch.equal(o[b].cpu(), torch.zeros_like(o[b].cpu()))


def test_long_causal_first_row_and_prefix():
    """Causal rows past 2048 queries (256-query workgroups, two query blocks
    per wave): output row 0 is value row 0 bit-exactly (one legal key), and
    rows up to t stay bit-identical when every key and value after t is
    replaced (by values 50 times larger, so that the later rows of those
    waves overflow their first reference and take the recomputation)."""
    dev = device()
    B, h, L, d = 1, 2, 2304, 64
    q = generate.normal((B, L, h, d), 9400, "bf16")
    k = generate.normal((B, L, h, d), 9401, "bf16")
    v = generate.normal((B, L, h, d), 9402, "bf16")
    say(f"case long causal prefix B={B} h={h} L={L}")
    base = mha.mha_forward(q.to(dev), k.to(dev), v.to(dev), mask=CAUSAL).cpu()
    assert torch.equal(base[:, 0], v[:, 0])
    for t in (31, 255, 256, 1000, 2100):
        k2, v2 = k.clone(), v.clone()
        k2[:, t + 1:] = generate.normal(k2[:, t + 1:].shape, 9410 + t, "bf16") * 50
        v2[:, t + 1:] = generate.normal(v2[:, t + 1:].shape, 9420 + t, "bf16") * 50
        o2 = mha.mha_forward(q.to(dev), k2.to(dev), v2.to(dev), mask=CAUSAL).cpu()
        assert torch.equal(o2[:, :t + 1], base[:, :t + 1]), t
        assert torch.isfinite(o2.float()).all(), t
