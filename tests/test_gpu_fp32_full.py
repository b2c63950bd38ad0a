"""GPU parity of the fp32 (accuracy) path at the sizes bench.py times it.

The fp32 kernels run on the matrix cores (fp32 MFMAs with fp32
accumulation); these cases take the bench's own seeded inputs: attention at
the base model's head shape (h = 8, d_k = 64; "Paper Deep Reading", section
08, Table 3) with L = 1024, B = 4, and the base decoder block's projections,
W^O and post-norm (X [64, 128, 512]; section 04, MultiHead equations;
section 03, residual and LayerNorm).  Sampled attention rows and the whole
projection outputs are compared with the fp64 oracle at the fp32 bound
max |gpu - oracle| <= 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_scaled_dot_fwd_amd as mha
from gpu_util import check, device, say
from workloads import generate

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mask", [mha.MASK_NONE, mha.MASK_CAUSAL])
def test_fp32_attention_base_head_shape(mask):
    dev = device()
    B, L, h, d = 4, 1024, 8, 64
    q = generate.normal((B, L, h, d), 9600, "f32")
    k = generate.normal((B, L, h, d), 9601, "f32")
    v = generate.normal((B, L, h, d), 9602, "f32")
    say(f"case fp32 attention B={B} L={L} h={h} d={d} mask={mask}")
    o = mha.mha_forward(q.to(dev), k.to(dev), v.to(dev), mask=mask).cpu()
    rng = np.random.Generator(np.random.PCG64(9603 + mask))
    n = 160
    rows = np.stack([rng.integers(0, B, n), rng.integers(0, h, n), rng.integers(0, L, n)], 1)
    edges = [(b, t, i) for b in (0, B - 1) for t in (0, h - 1) for i in (0, 127, 128, L - 1)]
    rows = np.concatenate([rows, np.array(edges)]).astype(np.int64)
    ref = oracle.attention_rows(q, k, v, rows, mask=mask)
    got = o[rows[:, 0], rows[:, 2], rows[:, 1]]
    check(got, ref, "f32", f"fp32 attention mask={mask} ({len(rows)} rows)")


def test_fp32_block_linear_maps_base_shape():
    dev = device()
    B, L, dm, h = 64, 128, 512, 8
    x = generate.normal((B, L, dm), 9700, "f32")
    ws = [generate.normal((dm, dm), 9701 + j, "f32", std=dm ** -0.5) for j in range(4)]
    say(f"case fp32 block maps X [{B}, {L}, {dm}], h={h}")
    xd, wd = x.to(dev), [w.to(dev) for w in ws]
    q, k, v = mha.mha_project_qkv(xd, xd, *wd[:3], h)
    rq, rk, rv = oracle.project_qkv(x, x, *ws[:3], h=h)
    for name, g, r in (("Q", q, rq), ("K", k, rk), ("V", v, rv)):
        check(g, r, "f32", f"fp32 projection {name}")
    y = mha.mha_out_proj(q, wd[3])
    check(y, oracle.out_proj(q.cpu(), ws[3]), "f32", "fp32 W^O")
    gamma = 1.0 + 0.1 * generate.normal((dm,), 9705, "f32")
    beta = 0.1 * generate.normal((dm,), 9706, "f32")
    z = mha.mha_out_proj_post_norm(q, wd[3], xd, gamma.to(dev), beta.to(dev), eps=1e-6)
    check(z, oracle.out_proj_post_norm(q.cpu(), ws[3], x, gamma, beta, eps=1e-6), "f32",
          "fp32 W^O + residual + post-norm")
