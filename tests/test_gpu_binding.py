"""The Python binding's argument checks.

The library writes each output by the shape its size arguments give, so the
binding must refuse, before any launch, an output buffer of another shape,
a tensor on another device, a non-contiguous view or a dtype that differs.
Every case here raises on the host, and the output buffer handed in keeps
its contents.
"""
import pytest
import torch

import transformer_scaled_dot_fwd_amd as mha
from gpu_util import device, say

pytestmark = pytest.mark.gpu


def bf16(*shape, dev):
    return torch.randn(shape, device=dev).to(torch.bfloat16)


def untouched(buf, before):
    torch.cuda.synchronize()
    return torch.equal(buf, before)


def test_output_shapes_are_checked():
    dev = device()
    B, L, h, d, dm = 2, 16, 4, 64, 256
    x = bf16(B, L, dm, dev=dev)
    w_q, w_k, w_v = (bf16(dm, h * d, dev=dev) for _ in range(3))
    w_o = bf16(h * d, dm, dev=dev)
    q, k, v = mha.mha_project_qkv(x, x, w_q, w_k, w_v, h)
    o = mha.mha_forward(q, k, v)
    torch.cuda.synchronize()

    small_y = torch.full((B, L - 1, dm), 3.0, dtype=torch.bfloat16, device=dev)
    before = small_y.clone()
    with pytest.raises(ValueError):
        mha.mha_out_proj(o, w_o, out=small_y)
    assert untouched(small_y, before)

    bad = torch.full((B, L, h, d // 2), 3.0, dtype=torch.bfloat16, device=dev)
    before = bad.clone()
    with pytest.raises(ValueError):
        mha.mha_project_qkv(x, x, w_q, w_k, w_v, h, out=(q, bad, v))
    with pytest.raises(ValueError):
        mha.mha_forward(q, k, v, out=bad)
    with pytest.raises(ValueError):
        mha.mha_self_attention_fused(x, w_q, w_k, w_v, h, out=bad)
    assert untouched(bad, before)

    gamma = torch.ones(dm, dtype=torch.bfloat16, device=dev)
    beta = torch.zeros(dm, dtype=torch.bfloat16, device=dev)
    before = small_y.clone()
    with pytest.raises(ValueError):
        mha.mha_out_proj_post_norm(o, w_o, x, gamma, beta, out=small_y)
    assert untouched(small_y, before)
    say("  every mis-shaped output refused, buffers untouched")


def test_lengths_devices_layouts_and_dtypes_are_checked():
    dev = device()
    B, L, h, d = 2, 16, 4, 64
    q, k, v = (bf16(B, L, h, d, dev=dev) for _ in range(3))
    with pytest.raises(ValueError):  # lengths of the wrong shape
        mha.mha_forward(q, k, v, mask=mha.MASK_KEY_PADDING,
                        kv_lens=torch.full((B + 1,), L, dtype=torch.int32, device=dev))
    with pytest.raises(TypeError):  # lengths of the wrong dtype
        mha.mha_forward(q, k, v, mask=mha.MASK_KEY_PADDING,
                        kv_lens=torch.full((B,), L, dtype=torch.int64, device=dev))
    with pytest.raises(ValueError):  # a host tensor
        mha.mha_forward(q, k.cpu(), v)
    with pytest.raises(ValueError):  # lengths on the host
        mha.mha_forward(q, k, v, mask=mha.MASK_KEY_PADDING,
                        kv_lens=torch.full((B,), L, dtype=torch.int32))
    with pytest.raises(ValueError):  # a strided view
        mha.mha_forward(q, k.transpose(1, 2).contiguous().transpose(1, 2), v)
    with pytest.raises(TypeError):  # mixed dtypes
        mha.mha_forward(q, k.float(), v)
    with pytest.raises(ValueError):  # mismatched key and value lengths
        mha.mha_forward(q, k, v[:, :L - 1].contiguous())
    say("  lengths, devices, layouts and dtypes refused")
