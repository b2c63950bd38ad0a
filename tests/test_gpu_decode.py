"""GPU parity of mha_decode, one decoding step against a K/V cache: the
newest position's query over cache_lens[b] cached keys, which is attention
with Lq = 1 and the cache length as key padding ("Paper Deep Reading",
section 04 attention equation; section 03 decoder, one position per step).
Compared with the fp64 oracle's attention on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_scaled_dot_fwd_amd as mha
from gpu_util import check, device, say, to_np
from workloads import configs, generate

pytestmark = pytest.mark.gpu

PAD = 1


def make(B, h, L, d, seed):
    q = generate.normal((B, 1, h, d), seed, "bf16")
    k = generate.normal((B, L, h, d), seed + 1, "bf16")
    v = generate.normal((B, L, h, d), seed + 2, "bf16")
    return q, k, v


def decode(q, k, v, lens, dev, **kw):
    o = mha.mha_decode(q.to(dev), k.to(dev), v.to(dev), lens.to(dev), **kw)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("d", [64, 128])
# h up to 8, 16 and 32 select 1, 2 and 4 heads per lane group; above 32,
# further workgroups take the next 32 heads (a partial last group at 40 and
# 70).
@pytest.mark.parametrize("B,h,L", [(5, 3, 1), (4, 8, 300), (3, 2, 1000), (9, 8, 4097),
                                   (2, 16, 257), (3, 24, 700), (4, 32, 2100),
                                   (3, 40, 1500), (2, 64, 2100), (2, 70, 300)])
def test_decode_against_oracle(B, h, L, d):
    dev = device()
    say(f"case decode d={d} B={B} h={h} L={L}")
    q, k, v = make(B, h, L, d, 5000 + L + d)
    choices = [L, 1, 0, L + 5, -3, 255, 256, 257, 513, L // 2]
    lens = torch.tensor([min(choices[i % len(choices)], L + 5) for i in range(B)],
                        dtype=torch.int32)
    o = decode(q, k, v, lens, dev)
    ref = oracle.attention(q, k, v, mask=PAD, kv_lens=lens)
    check(o, ref, "bf16", f"decode d={d} B={B} h={h} L={L}")
    for b in range(B):
        if int(lens[b]) <= 0:
            assert torch.equal(o[b].cpu(), torch.zeros_like(o[b].cpu()))


@pytest.mark.parametrize("d", [64, 128])
def test_decode_chunk_boundaries(d):
    """Cache lengths on and next to multiples of 512 and 1024 keys, where a
    sequence's split over the cache gains or loses a (partial) chunk."""
    dev = device()
    lens = torch.tensor([511, 512, 513, 1023, 1024, 1025, 2047, 2048, 2049, 3071, 3072, 3073],
                        dtype=torch.int32)
    B, h, L = len(lens), 8, 3073
    say(f"case decode chunk boundaries d={d} L={L}")
    q, k, v = make(B, h, L, d, 5400 + d)
    o = decode(q, k, v, lens, dev)
    check(o, oracle.attention(q, k, v, mask=PAD, kv_lens=lens), "bf16",
          f"decode chunk boundaries d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_decode_never_reads_past_the_length_and_is_deterministic(d):
    dev = device()
    B, h, L = 4, 4, 700
    q, k, v = make(B, h, L, d, 5100 + d)
    lens = torch.tensor([700, 1, 300, 512], dtype=torch.int32)
    base = decode(q, k, v, lens, dev)
    again = decode(q, k, v, lens, dev)
    assert torch.equal(base, again)
    for junk in (float("nan"), float("inf"), 1e30):
        k2, v2 = k.clone(), v.clone()
        for b in range(B):
            k2[b, lens[b]:] = junk
            v2[b, lens[b]:] = junk
        assert torch.equal(decode(q, k2, v2, lens, dev), base), junk
    # one valid key: o is that V row (the weight is exactly 1)
    assert torch.equal(base[1, 0].cpu(), v[1, 0])


def test_decode_workspace_reuse_and_errors():
    """A caller workspace serves calls of different sizes (nothing in it
    carries over); a workspace that is too small is refused."""
    dev = device()
    ws = torch.empty(int(mha.lib().mha_decode_workspace_bytes(8, 8, 4096, 64)), dtype=torch.uint8,
                     device=dev)
    for (B, h, L) in ((8, 8, 4096), (3, 2, 100), (8, 8, 2000)):
        say(f"case decode workspace B={B} h={h} L={L}")
        q, k, v = make(B, h, L, 64, 5200 + L)
        lens = generate.lengths(B, 1, L, 5210 + L)
        o = decode(q, k, v, lens, dev, workspace=ws)
        check(o, oracle.attention(q, k, v, mask=PAD, kv_lens=lens), "bf16",
              f"decode reuse B={B} L={L}")
    q, k, v = make(2, 2, 600, 64, 5300)
    small = torch.empty(64, dtype=torch.uint8, device=dev)
    with pytest.raises(mha.MHAError):
        decode(q, k, v, torch.tensor([600, 3], dtype=torch.int32), dev, workspace=small)
    q48, k48, v48 = make(2, 2, 10, 48, 5310)
    with pytest.raises(mha.MHAError):
        decode(q48, k48, v48, torch.tensor([10, 3], dtype=torch.int32), dev)


@pytest.mark.parametrize("name", [w.name for w in configs.decodes()])
def test_decode_workloads_sampled(name):
    """The benchmark's decode workloads at full size, on sampled (sequence,
    head) rows the oracle computes one by one."""
    dev = device()
    w = configs.get(name)
    say(f"case {w.name} (sampled rows)")
    inp = configs.make_inputs(w)
    o = decode(inp["q"], inp["k"], inp["v"], inp["kv_lens"], dev)
    rng = np.random.default_rng(9)
    rows = np.array([(int(b), int(t), 0) for b, t in zip(rng.integers(0, w.B, 48),
                                                          rng.integers(0, w.h, 48))] +
                    [(0, 0, 0), (w.B - 1, w.h - 1, 0)], dtype=np.int64)
    ref = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, mask=PAD,
                                kv_lens=inp["kv_lens"])
    o_np = to_np(o)
    check(np.stack([o_np[b, 0, t] for (b, t, _) in rows]), ref, "bf16",
          f"{w.name} ({len(rows)} rows)")
