"""GPU parity of mha_out_proj_post_norm, the attention sub-layer's output
with its residual connection and post-norm, LayerNorm(x + Concat(heads) W^O)
("Paper Deep Reading", section 03 residual + LayerNorm, section 04 MultiHead
equation).  Compared with the fp64 oracle on the same bf16 (or fp32) inputs.

Inputs: o ~ N(0, 1) (attention outputs are convex combinations of V rows,
of unit scale), W^O ~ N(0, 1/(h d_v)) so that the product has unit variance,
x ~ N(0, 1), gamma = 1 + 0.1 N(0, 1), beta = 0.1 N(0, 1).
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_scaled_dot_fwd_amd as mha
from gpu_util import check, device, say
from workloads import configs, generate

pytestmark = pytest.mark.gpu


def make(B, Lq, h, dv, dm, seed):
    K = h * dv
    o = generate.normal((B, Lq, h, dv), seed, "bf16")
    w_o = generate.normal((K, dm), seed + 1, "bf16", std=float(1.0 / np.sqrt(K)))
    x = generate.normal((B, Lq, dm), seed + 2, "bf16")
    gamma = (1.0 + 0.1 * generate.normal((dm,), seed + 3, "f32")).to(torch.bfloat16)
    beta = generate.normal((dm,), seed + 4, "bf16", std=0.1)
    return o, w_o, x, gamma, beta


def run(o, w_o, x, gamma, beta, dev, eps=1e-6, out=None):
    y = mha.mha_out_proj_post_norm(o.to(dev), w_o.to(dev), x.to(dev), gamma.to(dev),
                                   beta.to(dev), eps=eps, out=out)
    torch.cuda.synchronize()
    return y


# (B, Lq, h, d_v, d_model): one row; ragged tails over several 32-row tiles;
# the three widths; the smallest inner size (32) and one that is not a
# multiple of 64 (9 k steps of 32); big-model heads.
SHAPES = [(1, 1, 8, 64, 512), (2, 37, 8, 64, 512), (3, 50, 4, 64, 256), (2, 45, 16, 64, 1024),
          (1, 33, 2, 16, 256), (1, 70, 6, 48, 512), (4, 128, 8, 64, 512), (3, 31, 16, 64, 1024),
          (2, 96, 4, 128, 512)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_L{}_h{}_dv{}_dm{}".format(*s))
def test_post_norm_against_oracle(shape):
    dev = device()
    B, Lq, h, dv, dm = shape
    say(f"case post_norm {shape}")
    o, w_o, x, gamma, beta = make(B, Lq, h, dv, dm, 7000 + sum(shape))
    y = run(o, w_o, x, gamma, beta, dev)
    ref = oracle.out_proj_post_norm(o, w_o, x, gamma, beta, eps=1e-6)
    check(y, ref, "bf16", f"post_norm {shape}")


def test_base_block_size_sampled_rows():
    """The base decoder block's sub-layer output at full size (B=64, Lq=128,
    h=8, d_v=64, d_model=512: 8192 rows, 256 workgroups), in the launch
    configuration the bench times; 512 sampled rows against the oracle
    (rows are independent), every row checked for unit-free properties."""
    dev = device()
    w = configs.get("c3")
    B, Lq, h, dv, dm = w.B, w.Lq, w.h, w.d, w.d_model
    say(f"case post_norm base block {B}x{Lq} h={h} d_v={dv} d_model={dm}")
    o, w_o, x, gamma, beta = make(B, Lq, h, dv, dm, 7100)
    y = run(o, w_o, x, gamma, beta, dev)
    M = B * Lq
    rows = np.sort(np.random.Generator(np.random.PCG64(7101)).choice(M, 512, replace=False))
    rows = np.union1d(rows, [0, 31, 32, M - 1])
    o_rows = o.reshape(1, M, h, dv)[:, rows]
    x_rows = x.reshape(1, M, dm)[:, rows]
    ref = oracle.out_proj_post_norm(o_rows, w_o, x_rows, gamma, beta, eps=1e-6)
    check(y.reshape(M, dm)[rows].reshape(1, len(rows), dm), ref, "bf16", "base block rows")
    # every row: (y - beta) / gamma has mean ~0 and population variance ~1
    yn = (y.float() - beta.to(dev).float()) / gamma.to(dev).float()
    assert float(yn.mean(dim=-1).abs().max()) < 0.02
    assert float((yn.var(dim=-1, unbiased=False) - 1).abs().max()) < 0.03


def test_tail_rows_untouched_deterministic_and_in_place():
    dev = device()
    B, Lq, h, dv, dm = 3, 41, 8, 64, 512
    M = B * Lq
    o, w_o, x, gamma, beta = make(B, Lq, h, dv, dm, 7200)
    big = torch.full((M + 40, dm), 7.0, dtype=torch.bfloat16, device=dev)
    out = big[:M].view(B, Lq, dm)
    y = run(o, w_o, x, gamma, beta, dev, out=out)
    assert torch.equal(big[M:].cpu(), torch.full((40, dm), 7.0, dtype=torch.bfloat16))
    again = run(o, w_o, x, gamma, beta, dev)
    assert torch.equal(y.cpu(), again.cpu())
    # in place: the residual stream overwritten by the sub-layer output
    xs = x.to(dev).clone()
    mha.mha_out_proj_post_norm(o.to(dev), w_o.to(dev), xs, gamma.to(dev), beta.to(dev),
                               eps=1e-6, out=xs)
    torch.cuda.synchronize()
    assert torch.equal(xs.cpu(), again.cpu())


def test_constant_rows_give_beta_and_scaling_is_exact():
    """z = x + o W^O constant along a row has var = 0: y is beta exactly
    (z - mu = 0 in fp32).  Scaling o and x by 2 (exact in bf16) scales z, mu
    and sigma by 2 exactly, so with eps = 0 the output is bit-identical."""
    dev = device()
    B, Lq, h, dv, dm = 2, 40, 8, 64, 256
    o, w_o, x, gamma, beta = make(B, Lq, h, dv, dm, 7300)
    const = generate.normal((B, Lq, 1), 7305, "bf16").expand(B, Lq, dm).contiguous()
    y = run(o, torch.zeros_like(w_o), const, gamma, beta, dev)
    assert torch.equal(y.cpu(), beta.expand(B, Lq, dm))
    base = run(o, w_o, x, gamma, beta, dev, eps=0.0)
    twice = run((2 * o.float()).to(torch.bfloat16), w_o, (2 * x.float()).to(torch.bfloat16),
                gamma, beta, dev, eps=0.0)
    assert torch.equal(base.cpu(), twice.cpu())
    check(base, oracle.out_proj_post_norm(o, w_o, x, gamma, beta, eps=0.0), "bf16", "eps=0")


def test_empty_batch_is_a_no_op():
    dev = device()
    o, w_o, x, gamma, beta = make(1, 1, 8, 64, 512, 7400)
    y = mha.mha_out_proj_post_norm(o[:0].to(dev), w_o.to(dev), x[:0].to(dev), gamma.to(dev),
                                   beta.to(dev))
    torch.cuda.synchronize()
    assert y.shape == (0, 1, 512)


# fp32 (the accuracy path, exact fp32 FMAs): any h*d_v, including inner
# sizes that are not multiples of 32 or of the 256-wide k chunk.
F32_SHAPES = [(1, 1, 8, 64, 512), (2, 37, 8, 64, 512), (3, 50, 4, 64, 256), (2, 45, 16, 64, 1024),
              (1, 33, 3, 16, 256), (1, 20, 5, 100, 512)]


@pytest.mark.parametrize("shape", F32_SHAPES, ids=lambda s: "B{}_L{}_h{}_dv{}_dm{}".format(*s))
def test_post_norm_fp32_against_oracle(shape):
    dev = device()
    B, Lq, h, dv, dm = shape
    say(f"case post_norm fp32 {shape}")
    o, w_o, x, gamma, beta = (t.float() for t in make(B, Lq, h, dv, dm, 7500 + sum(shape)))
    y = run(o, w_o, x, gamma, beta, dev)
    assert y.dtype == torch.float32
    check(y, oracle.out_proj_post_norm(o, w_o, x, gamma, beta, eps=1e-6), "f32",
          f"post_norm fp32 {shape}")
    xs = x.to(dev).clone()
    mha.mha_out_proj_post_norm(o.to(dev), w_o.to(dev), xs, gamma.to(dev), beta.to(dev),
                               eps=1e-6, out=xs)
    torch.cuda.synchronize()
    assert torch.equal(xs.cpu(), y.cpu())
