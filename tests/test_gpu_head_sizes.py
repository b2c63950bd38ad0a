"""GPU parity of mha_forward at the other head sizes of the base width
(d_model 512: h=32 d=16, h=16 d=32, h=4 d=128; "Paper Deep Reading",
section 08, Table 3, rows (A)), bf16, against the fp64 oracle: ragged
multi-tile shapes with every mask, the properties that fix bits, the
Table 3 shapes at L = 1024 and 4096 on sampled rows, and the block with
those heads end to end.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_scaled_dot_fwd_amd as mha
from gpu_util import check, device, say, to_np
from workloads import configs, generate

pytestmark = pytest.mark.gpu

NONE, PAD, CAUSAL = 0, 1, 2
HEAD_SIZES = [16, 32, 128]


def make(B, h, Lq, Lk, d, seed):
    return (generate.normal((B, Lq, h, d), seed, "bf16"),
            generate.normal((B, Lk, h, d), seed + 1, "bf16"),
            generate.normal((B, Lk, h, d), seed + 2, "bf16"))


def run(q, k, v, mask, lens, dev):
    o = mha.mha_forward(q.to(dev), k.to(dev), v.to(dev), mask=mask,
                        kv_lens=lens.to(dev) if lens is not None else None)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("d", HEAD_SIZES)
@pytest.mark.parametrize("mask", [NONE, PAD, CAUSAL, PAD | CAUSAL])
@pytest.mark.parametrize("shape", [(3, 2, 200, 177), (1, 2, 257, 257), (2, 2, 5, 300),
                                   (1, 1, 1, 1), (2, 3, 130, 64), (1, 2, 600, 600)])
def test_head_size_ragged(d, shape, mask):
    dev = device()
    B, h, Lq, Lk = shape
    if mask & CAUSAL:
        Lk = Lq
    say(f"case bf16 d={d} B={B} h={h} Lq={Lq} Lk={Lk} mask={mask}")
    q, k, v = make(B, h, Lq, Lk, d, 3000 + d + Lq + 3 * Lk + mask)
    choices = [Lk, 1, max(Lk - 1, 0), 0, Lk + 50, -5, Lk // 2, 65]
    lens = torch.tensor([choices[i % len(choices)] for i in range(B)], dtype=torch.int32)
    o = run(q, k, v, mask, lens, dev)
    check(o, oracle.attention(q, k, v, mask=mask, kv_lens=lens), "bf16",
          f"bf16 d={d} {shape} m={mask}")


@pytest.mark.parametrize("d", HEAD_SIZES)
def test_head_size_padding_garbage_and_single_key(d):
    """NaN/Inf/1e30 in K/V rows at or past the length leave O bit-identical
    to zeros there; one legal key gives that V row bit-exactly; none gives 0."""
    dev = device()
    B, h, L = 4, 2, 300
    q, k, v = make(B, h, L, L, d, 3100 + d)
    lens = torch.tensor([L, 1, 0, L - 50], dtype=torch.int32)
    k0, v0 = k.clone(), v.clone()
    for b in range(B):
        k0[b, lens[b]:] = 0
        v0[b, lens[b]:] = 0
    for mask in (PAD, PAD | CAUSAL):
        base = run(q, k0, v0, mask, lens, dev)
        for junk in (float("nan"), float("inf"), 1e30):
            k2, v2 = k.clone(), v.clone()
            for b in range(B):
                k2[b, lens[b]:] = junk
                v2[b, lens[b]:] = junk
            assert torch.equal(run(q, k2, v2, mask, lens, dev), base), (d, mask, junk)
    o = run(q, k, v, PAD, lens, dev).cpu()
    assert torch.equal(o[1], v[1, 0:1].expand(L, h, d))
    assert torch.equal(o[2], torch.zeros(L, h, d, dtype=o.dtype))


@pytest.mark.parametrize("d", HEAD_SIZES)
def test_head_size_causal_prefix(d):
    dev = device()
    B, h, L = 2, 2, 300
    q, k, v = make(B, h, L, L, d, 3200 + d)
    base = run(q, k, v, CAUSAL, None, dev)
    for t in (0, 63, 130, L - 20):
        k2, v2 = k.clone(), v.clone()
        k2[:, t + 1:] = generate.normal(k2[:, t + 1:].shape, 3300 + t, "bf16") * 50
        v2[:, t + 1:] = generate.normal(v2[:, t + 1:].shape, 3400 + t, "bf16") * 50
        o2 = run(q, k2, v2, CAUSAL, None, dev)
        assert torch.equal(o2[:, :t + 1], base[:, :t + 1]), (d, t)


def sample_rows(B, h, L, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 127, 128, 255, 256, L // 2, L - 1]
    return np.array([(b, t, int(i)) for b in range(B) for t in range(h)
                     for i in [f for f in fixed if f < L] + list(rng.integers(0, L, n))],
                    dtype=np.int64)


@pytest.mark.parametrize("name", [w.name for w in configs.head_sizes()])
def test_table3_head_shapes_sampled(name):
    """The Table 3 (A) shapes at full size, in the benchmark's launch
    configuration, on sampled rows the oracle computes one by one."""
    dev = device()
    w = configs.get(name)
    say(f"case {w.name} (sampled rows)")
    inp = configs.make_inputs(w)
    o = run(inp["q"], inp["k"], inp["v"], w.mask, None, dev)
    rows = sample_rows(w.B, w.h, w.Lq, 2, 77)
    ref = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, mask=w.mask)
    o_np = to_np(o)
    got = np.stack([o_np[b, i, t] for (b, t, i) in rows])
    check(got, ref, "bf16", f"{w.name} ({len(rows)} rows)")


@pytest.mark.parametrize("h,d", [(32, 16), (16, 32), (4, 128)])
def test_block_with_other_head_shapes(h, d):
    """X [8,128,512] through projection, attention (causal + padding) and
    W^O with the Table 3 (A) heads, end to end against the fp64 block."""
    dev = device()
    B, L, dm = 8, 128, 512
    say(f"case block h={h} d={d}")
    x = generate.normal((B, L, dm), 3500 + d, "bf16")
    ws = [generate.normal((dm, h * d), 3501 + d + i, "bf16", std=dm ** -0.5) for i in range(3)]
    wo = generate.normal((h * d, dm), 3510 + d, "bf16", std=(h * d) ** -0.5)
    lens = generate.lengths(B, 32, 128, 3520 + d)
    y = mha.mha_block(x.to(dev), x.to(dev), *(w.to(dev) for w in ws), wo.to(dev), h=h,
                      mask=3, kv_lens=lens.to(dev))
    torch.cuda.synchronize()
    ref = oracle.mha_block(x, x, *ws, wo, h=h, mask=3, kv_lens=lens)
    check(y, ref, "bf16", f"block h={h} d={d}")
