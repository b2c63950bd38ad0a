"""GPU parity of restricted (windowed) self-attention, mha_forward_windowed:
query i sees keys within w positions ("Paper Deep Reading", section 05,
complexity table, "Restricted self-attention").  Ragged shapes against the
fp64 oracle for every mask, window and head size; bit-exact properties of
the band; the benchmark's windowed workloads on sampled rows.
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


def make(B, h, L, d, dtype, seed):
    return tuple(generate.normal((B, L, h, d), seed + n, dtype) for n in range(3))


def run(q, k, v, mask, lens, window, dev):
    o = mha.mha_forward(q.to(dev), k.to(dev), v.to(dev), mask=mask,
                        kv_lens=lens.to(dev) if lens is not None else None, window=window)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (16, "bf16"), (128, "bf16"), (64, "f32"),
                                     (8, "f32")])
@pytest.mark.parametrize("mask", [NONE, PAD, CAUSAL, PAD | CAUSAL])
@pytest.mark.parametrize("B,h,L", [(2, 2, 300), (1, 3, 77), (2, 1, 1000)])
def test_window_ragged(B, h, L, d, dtype, mask):
    dev = device()
    q, k, v = make(B, h, L, d, dtype, 4000 + L + d + 7 * mask)
    lens = torch.tensor([L - 13, 40][:B], dtype=torch.int32)
    for w in (0, 1, 31, 32, 100, 257, L):
        say(f"case window {dtype} d={d} B={B} h={h} L={L} mask={mask} w={w}")
        o = run(q, k, v, mask, lens, w, dev)
        check(o, oracle.attention(q, k, v, mask=mask, kv_lens=lens, window=w), dtype,
              f"window {dtype} d={d} L={L} m={mask} w={w}")


@pytest.mark.parametrize("d", [16, 64, 128])
def test_window_zero_is_v_and_full_window_is_attention(d):
    """w = 0: each query sees only its own position, O_i = V_i bit for bit
    (rows at or past the length see nothing: 0).  w >= L - 1: ordinary
    attention."""
    dev = device()
    B, h, L = 2, 2, 300
    q, k, v = make(B, h, L, d, "bf16", 4100 + d)
    lens = torch.tensor([L, 120], dtype=torch.int32)
    o = run(q, k, v, NONE, None, 0, dev).cpu()
    assert torch.equal(o, v)
    o = run(q, k, v, PAD, lens, 0, dev).cpu()
    assert torch.equal(o[1, :120], v[1, :120])
    assert torch.equal(o[1, 120:], torch.zeros_like(o[1, 120:]))
    for mask in (NONE, CAUSAL, PAD | CAUSAL):
        full = run(q, k, v, mask, lens, None, dev)
        check(run(q, k, v, mask, lens, L - 1, dev), full.cpu().double().numpy(), "bf16",
              f"full window d={d} m={mask}")


@pytest.mark.parametrize("w", [5, 64, 200])
def test_keys_outside_the_band_do_not_reach_the_output(w):
    """Rewriting K/V at positions >= t (with any finite values: rows below
    the length are data, as for causal) leaves O rows i < t - w
    bit-identical; rewriting positions <= t leaves rows i > t + w
    bit-identical."""
    dev = device()
    B, h, L, d = 2, 2, 600, 64
    q, k, v = make(B, h, L, d, "bf16", 4200 + w)
    base = run(q, k, v, NONE, None, w, dev)
    for t in (100, 333):
        k2, v2 = k.clone(), v.clone()
        k2[:, t:] = generate.normal(k2[:, t:].shape, 4250 + t, "bf16") * 50
        v2[:, t:] = 1e30
        o2 = run(q, k2, v2, NONE, None, w, dev)
        if t - w > 0:
            assert torch.equal(o2[:, :t - w], base[:, :t - w]), (w, t)
        k3, v3 = k.clone(), v.clone()
        k3[:, :t + 1] = 1e30
        v3[:, :t + 1] = generate.normal(v3[:, :t + 1].shape, 4260 + t, "bf16") * 50
        o3 = run(q, k3, v3, NONE, None, w, dev)
        if t + w + 1 < L:
            assert torch.equal(o3[:, t + w + 1:], base[:, t + w + 1:]), (w, t)


@pytest.mark.parametrize("name", [w.name for w in configs.windows()])
def test_window_workloads_sampled(name):
    dev = device()
    w = configs.get(name)
    say(f"case {w.name} (sampled rows)")
    inp = configs.make_inputs(w)
    o = run(inp["q"], inp["k"], inp["v"], w.mask, None, w.window, dev)
    rng = np.random.default_rng(5)
    fixed = [0, 1, 255, 256, 257, 511, 2048, 4095 - 256, 4094, 4095]
    rows = np.array([(b, t, int(i)) for b in range(w.B) for t in range(w.h)
                     for i in fixed + list(rng.integers(0, w.Lq, 2))], dtype=np.int64)
    ref = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, mask=w.mask,
                                window=w.window)
    o_np = to_np(o)
    check(np.stack([o_np[b, i, t] for (b, t, i) in rows]), ref, "bf16",
          f"{w.name} ({len(rows)} rows)")


def test_window_rejected_arguments():
    dev = device()
    q, k, v = make(1, 1, 8, 64, "bf16", 4300)
    with pytest.raises(mha.MHAError):
        run(q, k, v, NONE, None, -1, dev)
    with pytest.raises(mha.MHAError):
        mha.mha_forward(q.to(dev), k[:, :7].contiguous().to(dev), v[:, :7].contiguous().to(dev),
                        window=2)
