"""Concurrent callers: the library keeps no per-call state (only a cached
device property), so host threads may call it at the same time on their
own streams.  Four threads, each with its own (default-priority) stream,
repeatedly run a different entry point; every result must equal the one a
single thread computes on its own.
"""
import threading

import pytest
import torch

import transformer_scaled_dot_fwd_amd as mha
from gpu_util import device, say
from workloads import configs

pytestmark = pytest.mark.gpu

ROUNDS = 5


def test_concurrent_callers_on_their_own_streams():
    dev = device()
    blk = configs.make_inputs(configs.get("c3"), dev)
    wb = configs.get("c3")
    att = configs.make_inputs(configs.get("sweep_h8_L1024_causal"), dev)
    wa = configs.get("sweep_h8_L1024_causal")
    dec = configs.make_inputs(configs.get("decode_h8_B64_L4096"), dev)
    wd = configs.get("decode_h8_B64_L4096")
    ws = torch.empty(int(mha.lib().mha_decode_workspace_bytes(wd.B, wd.h, wd.Lk, wd.d)),
                     dtype=torch.uint8, device=dev)

    jobs = {
        "block": lambda: mha.mha_block(blk["x"], blk["x"], blk["w_q"], blk["w_k"], blk["w_v"],
                                       blk["w_o"], wb.h, mask=wb.mask, kv_lens=blk["kv_lens"]),
        "attention": lambda: mha.mha_forward(att["q"], att["k"], att["v"], mask=wa.mask),
        "decode": lambda: mha.mha_decode(dec["q"], dec["k"], dec["v"], dec["kv_lens"],
                                         workspace=ws),
        "post-norm": lambda: mha.mha_out_proj_post_norm(
            torch.ones((wb.B, wb.Lq, wb.h, wb.d), dtype=torch.bfloat16, device=dev),
            blk["w_o"], blk["x"], blk["gamma"], blk["beta"]),
    }
    ref = {}
    for name, fn in jobs.items():
        ref[name] = fn()
        torch.cuda.synchronize()
    errors = []

    def worker(name, fn):
        try:
            stream = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(stream):
                for r in range(ROUNDS):
                    out = fn()
                    stream.synchronize()
                    if not torch.equal(out, ref[name]):
                        errors.append(f"{name}: round {r} differs")
        except Exception as e:  # reported below, on the main thread
            errors.append(f"{name}: {e!r}")

    threads = [threading.Thread(target=worker, args=item) for item in jobs.items()]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    say(f"  {len(jobs)} threads x {ROUNDS} rounds: every result equals the single-thread run")
