"""GPU parity at the largest sizes the entry points accept.

Each kernel addresses one batch row of Q, K or V, one K/V cache, or the
weight matrix W^O with 32-bit byte offsets, and the entry points accept
exactly the shapes whose byte extent stays below 2^31.  These tests run one
shape at (just under) each limit:

* mha_forward, bf16, d = 128 (h = 64) and d = 64 (h = 128): Lk = 131071
  keys of 16 KB each, K and V 2 GiB - 16 KB apiece;
* mha_decode, bf16, d = 128, h = 16: a cache of 524287 positions of 4 KB;
* mha_out_proj_post_norm, d_model 1024, h d_v = 1048544: W^O of 2 GiB - 64 KB.

Inputs stay seeded: a 4096-row block drawn from the seeded generator is
repeated along the long axis and the last rows (those at the highest byte
offsets) are drawn on their own; those keys are scaled by 3 so that they
dominate every softmax, and a read of the wrong rows would show.  The oracle
computes a subset of heads (the first and the last, whose slices sit at the
highest offsets) from the same values.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_scaled_dot_fwd_amd as mha
from gpu_util import check, device, say
from workloads import generate

pytestmark = pytest.mark.gpu

BLOCK = 4096


def long_rows(L, h, d, seed, tail_scale=1.0):
    """[1, L, h, d] bf16: a seeded block repeated, the last BLOCK rows drawn
    on their own (times tail_scale)."""
    base = generate.normal((1, BLOCK, h, d), seed, "bf16")
    reps = (L + BLOCK - 1) // BLOCK
    x = base.repeat(1, reps, 1, 1)[:, :L].contiguous()
    tail = generate.normal((1, BLOCK, h, d), seed + 1, "f32")
    x[:, L - BLOCK:] = (tail_scale * tail).to(torch.bfloat16)
    return x


@pytest.mark.parametrize("h,d", [(64, 128), (128, 64)])
def test_forward_at_the_key_slab_limit(h, d):
    dev = device()
    Lk = (1 << 31) // (h * d * 2) - 1       # Lk h d 2 < 2^31
    Lq = 65
    say(f"case max forward h={h} d={d} Lq={Lq} Lk={Lk}")
    assert Lk * h * d * 2 < (1 << 31) <= (Lk + 1) * h * d * 2
    q = generate.normal((1, Lq, h, d), 8000 + d, "bf16")
    k = long_rows(Lk, h, d, 8010 + d, tail_scale=3.0)
    v = long_rows(Lk, h, d, 8020 + d)
    lens = torch.tensor([Lk], dtype=torch.int32)
    o = mha.mha_forward(q.to(dev), k.to(dev), v.to(dev), mask=mha.MASK_KEY_PADDING,
                        kv_lens=lens.to(dev))
    torch.cuda.synchronize()
    heads = [0, h - 1]
    ref = oracle.attention(q[:, :, heads].contiguous(), k[:, :, heads].contiguous(),
                           v[:, :, heads].contiguous(), mask=mha.MASK_KEY_PADDING,
                           kv_lens=lens)
    check(o[:, :, heads], ref, "bf16", f"max forward h={h} d={d}")


def test_decode_at_the_cache_limit():
    dev = device()
    h, d = 16, 128
    L = (1 << 31) // (h * d * 2) - 1        # L h d 2 < 2^31
    say(f"case max decode h={h} d={d} L={L}")
    q = generate.normal((1, 1, h, d), 8100, "bf16")
    k = long_rows(L, h, d, 8110, tail_scale=3.0)
    v = long_rows(L, h, d, 8120)
    lens = torch.tensor([L], dtype=torch.int32)
    o = mha.mha_decode(q.to(dev), k.to(dev), v.to(dev), lens.to(dev))
    torch.cuda.synchronize()
    heads = [0, h - 1]
    ref = oracle.attention(q[:, :, heads].contiguous(), k[:, :, heads].contiguous(),
                           v[:, :, heads].contiguous(), mask=mha.MASK_KEY_PADDING,
                           kv_lens=lens)
    check(o[:, :, heads], ref, "bf16", "max decode")


def test_post_norm_at_the_weight_limit():
    """W^O of h d_v = 1048544 rows by d_model = 1024 (2 GiB - 64 KB).  O is
    zero except on a set S of columns that includes the first and the last
    ones, so y = LayerNorm(x + O_S W^O_S): the oracle multiplies only those
    rows of W^O, while the kernel streams all of it."""
    dev = device()
    dm, dv = 1024, 32
    K = ((1 << 31) // (dm * 2) - 1) // 32 * 32   # largest multiple of 32 with K dm 2 < 2^31
    h = K // dv
    M = 33
    say(f"case max post-norm K={K} d_model={dm} rows={M}")
    assert K * dm * 2 < (1 << 31) and K % 32 == 0 and h * dv == K
    w = long_rows(K, 1, dm, 8200).reshape(K, dm)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(K - 64, K),
                                     np.random.Generator(np.random.PCG64(8201)).choice(K, 128)]))
    o = torch.zeros((1, M, K), dtype=torch.bfloat16)
    o[:, :, torch.from_numpy(cols)] = generate.normal((1, M, len(cols)), 8202, "bf16")
    x = generate.normal((1, M, dm), 8203, "bf16")
    gamma = (1.0 + generate.normal((dm,), 8204, "f32", 0.1)).to(torch.bfloat16)
    beta = generate.normal((dm,), 8205, "bf16", 0.1)
    y = mha.mha_out_proj_post_norm(o.view(1, M, h, dv).to(dev), w.to(dev), x.to(dev),
                                   gamma.to(dev), beta.to(dev))
    torch.cuda.synchronize()
    o_s = o[:, :, torch.from_numpy(cols)].reshape(1, M, 1, len(cols)).contiguous()
    ref = oracle.out_proj_post_norm(o_s, w[torch.from_numpy(cols)].contiguous(), x, gamma, beta)
    check(y, ref, "bf16", "max post-norm")
