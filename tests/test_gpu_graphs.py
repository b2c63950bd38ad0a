"""HIP graph capture of every entry point.

bench.py times each kernel alone as replays of captured graphs (one launch
per buffer set) and reports graph replays of its step beside the direct
launches; callers may capture the entry points too.  Each test here runs a
call eagerly, captures the same call in a graph, and then replays the graph
several times.  Before every replay the outputs are
overwritten with NaN by eager work on the same stream, followed by a
synchronisation.  Every replay must reproduce the eager outputs bit for bit
(the kernels are deterministic, and no call records a memset or any other
node that depends on state left by an earlier replay).
"""
import pytest
import torch

import transformer_scaled_dot_fwd_amd as mha
from gpu_util import device, say
from workloads import configs, generate

pytestmark = pytest.mark.gpu

REPLAYS = 4


def replay_matches_eager(fn, outputs, what):
    torch.cuda.synchronize()
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(REPLAYS):
        for o in outputs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert torch.equal(o, r), f"{what}: replay {i} differs from the eager run"
    say(f"  {what}: {REPLAYS} replays bit-identical to the eager run")


def test_block_step_graph():
    """The benchmark's step: fused self-attention then W^O, on the base
    decoder block workload, and the two-call path beside it."""
    dev = device()
    w = configs.get("c3")
    inp = configs.make_inputs(w, dev)
    B, L, h, d, dm = w.B, w.Lq, w.h, w.d, w.d_model
    o = torch.empty((B, L, h, d), dtype=torch.bfloat16, device=dev)
    y = torch.empty((B, L, dm), dtype=torch.bfloat16, device=dev)

    def fused_step():
        mha.mha_self_attention_fused(inp["x"], inp["w_q"], inp["w_k"], inp["w_v"], h,
                                     mask=w.mask, kv_lens=inp["kv_lens"], out=o)
        mha.mha_out_proj(o, inp["w_o"], out=y)

    replay_matches_eager(fused_step, [o, y], "fused self-attention + W^O")

    q, k, v = (torch.empty_like(o) for _ in range(3))

    def two_call_step():
        mha.mha_project_qkv(inp["x"], inp["x"], inp["w_q"], inp["w_k"], inp["w_v"], h,
                            out=(q, k, v))
        mha.mha_forward(q, k, v, mask=w.mask, kv_lens=inp["kv_lens"], out=o)
        mha.mha_out_proj(o, inp["w_o"], out=y)

    replay_matches_eager(two_call_step, [q, k, v, o, y], "projection, attention, W^O")


def test_sub_layer_with_post_norm_graph():
    dev = device()
    w = configs.get("c3")
    inp = configs.make_inputs(w, dev)
    B, L, h, d, dm = w.B, w.Lq, w.h, w.d, w.d_model
    o = torch.empty((B, L, h, d), dtype=torch.bfloat16, device=dev)
    z = torch.empty((B, L, dm), dtype=torch.bfloat16, device=dev)

    def step():
        mha.mha_self_attention_fused(inp["x"], inp["w_q"], inp["w_k"], inp["w_v"], h,
                                     mask=w.mask, kv_lens=inp["kv_lens"], out=o)
        mha.mha_out_proj_post_norm(o, inp["w_o"], inp["x"], inp["gamma"], inp["beta"], out=z)

    replay_matches_eager(step, [o, z], "fused self-attention + post-norm")


@pytest.mark.parametrize("name", ["sweep_h8_L1024_causal", "heads_h4_d128_L1024_nomask",
                                  "window_h8_L4096_w256_causal"])
def test_long_attention_graph(name):
    dev = device()
    w = configs.get(name)
    inp = configs.make_inputs(w, dev)
    o = torch.empty_like(inp["q"])

    def step():
        mha.mha_forward(inp["q"], inp["k"], inp["v"], mask=w.mask, kv_lens=inp["kv_lens"],
                        out=o, window=w.window)

    replay_matches_eager(step, [o], name)


def test_decode_graph():
    """The decode step with its caller workspace (no clearing between calls)."""
    dev = device()
    w = configs.get("decode_h8_B64_L4096")
    inp = configs.make_inputs(w, dev)
    ws = torch.empty(int(mha.lib().mha_decode_workspace_bytes(w.B, w.h, w.Lk, w.d)),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(inp["q"])

    def step():
        mha.mha_decode(inp["q"], inp["k"], inp["v"], inp["kv_lens"], out=o, workspace=ws)

    replay_matches_eager(step, [o], "decode")


def test_fp32_attention_graph():
    dev = device()
    q = generate.normal((2, 40, 3, 32), 9100, "f32").to(dev)
    k = generate.normal((2, 40, 3, 32), 9101, "f32").to(dev)
    v = generate.normal((2, 40, 3, 32), 9102, "f32").to(dev)
    lens = torch.tensor([40, 17], dtype=torch.int32, device=dev)
    o = torch.empty_like(q)

    def step():
        mha.mha_forward(q, k, v, mask=mha.MASK_CAUSAL | mha.MASK_KEY_PADDING, kv_lens=lens,
                        out=o)

    replay_matches_eager(step, [o], "fp32 attention")
