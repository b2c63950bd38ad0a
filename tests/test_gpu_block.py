"""GPU parity of the projections and of the full multi-head block.

mha_project_qkv and mha_out_proj are compared with the oracle's fp64 matmul
on the generator's inputs; the block (projection -> attention -> W^O) is
compared end to end with the oracle's fp64 block on the same X and weights.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_scaled_dot_fwd_amd as mha
from gpu_util import check, device, say
from workloads import configs, generate

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(2, 100, 77, 512, 8, 64), (1, 3, 130, 256, 4, 64),
                                   (3, 129, 129, 1024, 16, 64),
                                   # many tiles: the launch with the 2-stage LDS ring
                                   (64, 128, 128, 512, 8, 64), (40, 200, 150, 512, 8, 64)])
def test_project_qkv(dtype, shape):
    dev = device()
    B, Lq, Lk, dm, h, d = shape
    say(f"case project_qkv {dtype} {shape}")
    s = 1200 + Lq + Lk + dm
    xq = generate.normal((B, Lq, dm), s, dtype)
    xkv = generate.normal((B, Lk, dm), s + 1, dtype)
    ws = [generate.normal((dm, h * d), s + 2 + i, dtype, std=dm ** -0.5) for i in range(3)]
    q, k, v = mha.mha_project_qkv(xq.to(dev), xkv.to(dev), *(w.to(dev) for w in ws), h=h)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.project_qkv(xq, xkv, *ws, h=h)
    for name, g, r in (("Q", q, rq), ("K", k, rk), ("V", v, rv)):
        check(g, r, dtype, f"{name} {dtype} {shape}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(2, 100, 8, 64, 512), (1, 257, 16, 64, 1024),
                                   (3, 5, 4, 64, 192)])
def test_out_proj(dtype, shape):
    dev = device()
    B, Lq, h, d, dm = shape
    say(f"case out_proj {dtype} {shape}")
    s = 1300 + Lq + dm
    o = generate.normal((B, Lq, h, d), s, dtype)
    wo = generate.normal((h * d, dm), s + 1, dtype, std=(h * d) ** -0.5)
    y = mha.mha_out_proj(o.to(dev), wo.to(dev))
    torch.cuda.synchronize()
    check(y, oracle.out_proj(o, wo), dtype, f"out_proj {dtype} {shape}")


def test_base_decoder_block_end_to_end():
    """The base decoder block: X [64,128,512], causal + key padding."""
    dev = device()
    w = configs.get("c3")
    say(f"case {w.name}")
    inp = configs.make_inputs(w)
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    y = mha.mha_block(d["x"], d["x"], d["w_q"], d["w_k"], d["w_v"], d["w_o"], h=w.h,
                      mask=w.mask, kv_lens=d["kv_lens"])
    torch.cuda.synchronize()
    ref = oracle.mha_block(inp["x"], inp["x"], inp["w_q"], inp["w_k"], inp["w_v"], inp["w_o"],
                           h=w.h, mask=w.mask, kv_lens=inp["kv_lens"])
    check(y, ref, "bf16", f"{w.name} end to end")
    # the stages one by one, each on oracle-side inputs from the generator
    q, k, v = mha.mha_project_qkv(d["x"], d["x"], d["w_q"], d["w_k"], d["w_v"], h=w.h)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.project_qkv(inp["x"], inp["x"], inp["w_q"], inp["w_k"], inp["w_v"],
                                    h=w.h)
    check(q, rq, "bf16", "block stage Q")
    check(v, rv, "bf16", "block stage V")


def test_cross_attention_block():
    """Decoder queries over encoder memory of a different length."""
    dev = device()
    B, Lq, Lk, dm, h = 4, 96, 128, 1024, 16
    say("case cross-attention block")
    x = generate.normal((B, Lq, dm), 1400, "bf16")
    z = generate.normal((B, Lk, dm), 1401, "bf16")
    ws = [generate.normal((dm, dm), 1402 + i, "bf16", std=dm ** -0.5) for i in range(4)]
    lens = generate.lengths(B, 48, 128, 1406)
    y = mha.mha_block(x.to(dev), z.to(dev), *(w.to(dev) for w in ws), h=h, mask=1,
                      kv_lens=lens.to(dev))
    torch.cuda.synchronize()
    ref = oracle.mha_block(x, z, *ws, h=h, mask=1, kv_lens=lens)
    check(y, ref, "bf16", "cross-attention block")


# ---------------------------------------------------------------------------
# Self-attention with the projections fused in (rows of at most 128 tokens).
# ---------------------------------------------------------------------------

def _fused_inputs(B, L, dm, h, seed):
    x = generate.normal((B, L, dm), seed, "bf16")
    ws = [generate.normal((dm, h * 64), seed + 1 + i, "bf16", std=dm ** -0.5) for i in range(3)]
    choices = [L, 1, 0, L + 7, max(L // 2, 1), -3, L - 1]
    lens = torch.tensor([choices[i % len(choices)] for i in range(B)], dtype=torch.int32)
    return x, ws, lens


@pytest.mark.parametrize("mask", [0, 1, 2, 3])
@pytest.mark.parametrize("shape", [(64, 128, 512, 8), (3, 77, 512, 8), (2, 1, 256, 4),
                                   (5, 100, 1024, 16), (2, 128, 64, 1), (9, 33, 128, 2)])
def test_fused_self_attention_equals_two_call_path(shape, mask):
    """The fused kernel does the projection GEMM's and the short-row
    attention's arithmetic in the same order: identical bits."""
    dev = device()
    B, L, dm, h = shape
    say(f"case fused {shape} mask={mask}")
    x, ws, lens = _fused_inputs(B, L, dm, h, 1500 + L + dm + h + mask)
    x, ws, lens = x.to(dev), [w.to(dev) for w in ws], lens.to(dev)
    fused = mha.mha_self_attention_fused(x, *ws, h=h, mask=mask, kv_lens=lens)
    assert fused is not None
    q, k, v = mha.mha_project_qkv(x, x, *ws, h=h)
    ref = mha.mha_forward(q, k, v, mask=mask, kv_lens=lens)
    torch.cuda.synchronize()
    assert torch.equal(fused.cpu(), ref.cpu())


@pytest.mark.parametrize("mask", [1, 3])
def test_fused_self_attention_against_oracle(mask):
    dev = device()
    B, L, dm, h = 6, 120, 512, 8
    say(f"case fused vs oracle mask={mask}")
    x, ws, lens = _fused_inputs(B, L, dm, h, 1600 + mask)
    o = mha.mha_self_attention_fused(x.to(dev), *(w.to(dev) for w in ws), h=h, mask=mask,
                                     kv_lens=lens.to(dev))
    torch.cuda.synchronize()
    rq, rk, rv = oracle.project_qkv(x, x, *ws, h=h)
    ref = oracle.attention(rq, rk, rv, mask=mask, kv_lens=lens)
    check(o, ref, "bf16", f"fused self-attention m={mask}")


def test_fused_padding_rows_of_x_are_not_read_as_keys():
    """NaN/Inf in X at positions >= len_b: the K/V rows they project to are
    masked and never reach the other rows' outputs."""
    dev = device()
    B, L, dm, h = 4, 96, 256, 4
    x, ws, _ = _fused_inputs(B, L, dm, h, 1700)
    lens = torch.tensor([96, 40, 1, 0], dtype=torch.int32)
    wd = [w.to(dev) for w in ws]
    base = mha.mha_self_attention_fused(x.to(dev), *wd, h=h, mask=1, kv_lens=lens.to(dev))
    for junk in (float("nan"), float("inf")):
        x2 = x.clone()
        for b in range(B):
            x2[b, lens[b]:] = junk
        o2 = mha.mha_self_attention_fused(x2.to(dev), *wd, h=h, mask=1, kv_lens=lens.to(dev))
        torch.cuda.synchronize()
        for b in range(B):
            n = int(lens[b])
            assert torch.equal(o2[b, :n].cpu(), base[b, :n].cpu()), (junk, b)


def test_fused_self_attention_unsupported_shapes():
    dev = device()
    x = generate.normal((2, 129, 256), 1800, "bf16").to(dev)
    ws = [generate.normal((256, 4 * 64), 1801 + i, "bf16").to(dev) for i in range(3)]
    assert mha.mha_self_attention_fused(x, *ws, h=4) is None           # L > 128
    ws32 = [generate.normal((256, 8 * 32), 1811 + i, "bf16").to(dev) for i in range(3)]
    assert mha.mha_self_attention_fused(x[:, :64].contiguous(), *ws32, h=8) is None  # d_k = 32
