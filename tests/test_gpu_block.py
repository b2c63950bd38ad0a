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
