#!/usr/bin/env python3
"""Benchmark of the multi-head attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

The headline figure is the metric's own: attention-forward TFLOP/s at the
base model's head shape (h = 8, d_k = 64) with L >= 1024.  One step is one
mha_forward launch on each of the six rows of that sweep (L = 1024, 2048,
4096 with B = 24576 / L, no mask and causal, bf16, seeded N(0,1) inputs),
each on its own buffer set from a rotation of at least 1 GiB per row so the
256 MB Infinity Cache cannot serve a repeat.  K steps are launched back to
back on one stream, bracketed by torch.cuda.synchronize() and HIP events on
that stream; the value is the steps' algorithmic FLOPs (4 d per legal
(query, key) pair) over that time.

Printed beside it, in the same JSON line:
* every row of the sweep timed alone (h = 8 and h = 16, and the long
  causal workload), and the roofline of the dominant kernel: the streaming
  attention kernel on the step's longest row, its average launch duration
  timed with HIP events on the stream it runs on;
* the short-sequence workloads, HBM-bound: base encoder self-attention
  with key padding, big cross-attention over encoder memory, and the
  attention of the base decoder block, as algorithmic GB/s against the
  8 TB/s peak and against a measured device copy;
* the base decoder block step (projection, attention, W^O; fused
  projection + attention where rows are at most 128 tokens) with its
  per-kernel figures and the sub-layer with its residual and post-norm;
* the other head sizes, restricted attention and the decoding step;
* the fp64 CPU oracle timed on the host: on a sample of the headline rows
  (the reported baseline) and per configuration.

Counter runs: ``--kernel-only NAME`` runs just one kernel (or a plain
device copy of known size, ``copy``) so rocprofv3 can trace it or read its
FETCH_SIZE / WRITE_SIZE.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12       # MI355X HBM3E
PEAK_FP32_FLOPS = 157.3e12    # MI355X dense fp32 (vector and matrix)
ROTATE_BYTES = 1 << 30        # rotate buffers over >= 1 GiB (Infinity Cache is 256 MB)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "attention": os.path.join(ROOT, "transformer_scaled_dot_fwd_amd", "csrc", "attention.hip"),
    "attn_stream": os.path.join(ROOT, "transformer_scaled_dot_fwd_amd", "csrc", "attn_stream.hip"),
    "self_attention_fused": os.path.join(ROOT, "transformer_scaled_dot_fwd_amd", "csrc",
                                         "fused.hip"),
    "project_qkv": os.path.join(ROOT, "transformer_scaled_dot_fwd_amd", "csrc", "gemm.hip"),
    "out_proj": os.path.join(ROOT, "transformer_scaled_dot_fwd_amd", "csrc", "gemm.hip"),
    "out_proj_post_norm": os.path.join(ROOT, "transformer_scaled_dot_fwd_amd", "csrc",
                                       "norm.hip"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(name: str) -> str:
    """Hash of a kernel's source file and of every header beside it."""
    h = hashlib.sha256()
    src = KERNEL_SOURCES[name]
    d = os.path.dirname(src)
    for p in [src] + sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".h")):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3",
                    help="with --kernel-only: the workload the kernel runs on")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="rough CPU-time budget of the oracle sample")
    ap.add_argument("--kernel-only", choices=["project_qkv", "attention", "out_proj",
                                              "self_attention_fused", "out_proj_post_norm",
                                              "decode", "copy"])
    ap.add_argument("--warm-seconds", type=float, default=0.0,
                    help="with --kernel-only: launch the kernel for this long first, "
                    "untimed, so the traced --steps launches run at full clock")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step as three launches (projection, attention, W^O) even "
                         "where the fused self-attention kernel applies")
    return ap.parse_args()


class Block:
    """Device buffers of one step of the block workload, in n_sets copies."""

    def __init__(self, w, inputs, dev, n_sets):
        import torch
        import transformer_scaled_dot_fwd_amd as mha
        self.w, self.mha = w, mha
        B, L, h, d, dm = w.B, w.Lq, w.h, w.d, w.d_model
        self.sets = []
        for _ in range(n_sets):
            s = {k: v.to(dev) if v is not None else None for k, v in inputs.items()}
            s["q"] = torch.empty((B, L, h, d), dtype=torch.bfloat16, device=dev)
            s["k"] = torch.empty_like(s["q"])
            s["v"] = torch.empty_like(s["q"])
            s["o"] = torch.empty_like(s["q"])
            s["y"] = torch.empty((B, L, dm), dtype=torch.bfloat16, device=dev)
            s["z"] = torch.empty_like(s["y"])
            self.sets.append(s)
        self.fused = False

    def project_qkv(self, s):
        self.mha.mha_project_qkv(s["x"], s["x"], s["w_q"], s["w_k"], s["w_v"], self.w.h,
                                 out=(s["q"], s["k"], s["v"]))

    def attention(self, s):
        self.mha.mha_forward(s["q"], s["k"], s["v"], mask=self.w.mask, kv_lens=s["kv_lens"],
                             out=s["o"])

    def out_proj(self, s):
        self.mha.mha_out_proj(s["o"], s["w_o"], out=s["y"])

    def out_proj_post_norm(self, s):
        self.mha.mha_out_proj_post_norm(s["o"], s["w_o"], s["x"], s["gamma"], s["beta"],
                                        out=s["z"])

    def self_attention_fused(self, s):
        return self.mha.mha_self_attention_fused(s["x"], s["w_q"], s["w_k"], s["w_v"],
                                                 self.w.h, mask=self.w.mask,
                                                 kv_lens=s["kv_lens"], out=s["o"])

    def fused_supported(self):
        return self.self_attention_fused(self.sets[0]) is not None

    def step(self, s):
        if self.fused:
            self.self_attention_fused(s)
        else:
            self.project_qkv(s)
            self.attention(s)
        self.out_proj(s)

    def sublayer_step(self, s):
        """The attention sub-layer with its residual and post-norm:
        LayerNorm(x + MultiHead(x, x, x))."""
        if self.fused:
            self.self_attention_fused(s)
        else:
            self.project_qkv(s)
            self.attention(s)
        self.out_proj_post_norm(s)


def working_set_bytes(tensors) -> int:
    return sum(t.numel() * t.element_size() for t in tensors if t is not None)


def capture(fn_per_set, sets):
    """One HIP graph per buffer set, each holding fn(set)."""
    import torch
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the launch path outside capture
        for s in sets:
            fn_per_set(s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for s in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn_per_set(s)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_graphs(graphs, n, warmup):
    """Replay graphs[i % len] for i < n; return seconds per replay."""
    import torch
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        graphs[i % len(graphs)].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / n


def time_steps(step, sets, n, warmup):
    """Seconds per step over exactly n steps, step(sets[i % len(sets)]) for
    i < n, run as replays of one graph holding a pass over all sets plus one
    graph holding the remaining n % len(sets) steps."""
    import torch
    full = capture(lambda s0: [step(s) for s in sets], sets[:1])[0]
    rest = n % len(sets)
    tail = capture(lambda s0: [step(s) for s in sets[:rest]], sets[:1])[0] if rest else None
    for _ in range(max(1, warmup // len(sets))):
        full.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n // len(sets)):
        full.replay()
    if tail is not None:
        tail.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / n


def warm_gpu(step, sets, seconds):
    """Run the step for about `seconds` of wall time before anything is
    timed, so the first timed region does not pay for the GPU clocks
    ramping up."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(len(sets)):
            step(sets[i % len(sets)])
            i += 1
        torch.cuda.synchronize()


def time_eager(step, sets, n, warmup, host=None):
    """Seconds per step over exactly n steps launched directly on the stream
    (no graph), step(sets[i % len(sets)]) for i < n.  With a dict `host`,
    also stores the host's own seconds per step for issuing the launches
    (below the GPU time, the GPU never waited for the host)."""
    import torch
    for i in range(warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    t0 = time.perf_counter()
    for i in range(n):
        step(sets[i % len(sets)])
    t1 = time.perf_counter()
    e1.record(stream)
    torch.cuda.synchronize()
    if host is not None:
        host["s_per_step"] = (t1 - t0) / n
    return e0.elapsed_time(e1) * 1e-3 / n


def kernel_time(fn, sets, launches, warmup, repeats=5):
    """Average duration of one launch of fn, timed in graphs that each hold
    one launch per buffer set (so consecutive launches use different
    buffers): the median of `repeats` timed regions of at least `launches`
    launches each."""
    g = capture(lambda s0: [fn(s) for s in sets], sets[:1])
    reps = max(1, math.ceil(launches / len(sets)))
    time_graphs(g, reps, max(1, warmup // len(sets)))
    return statistics.median(time_graphs(g, reps, 0) / len(sets) for _ in range(repeats))


def time_median(fn, sets, warmup, host=None, min_calls=0, min_sec=0.02, repeats=5):
    """Seconds per call of fn(sets[i % len(sets)]) launched directly on the
    stream: after `warmup` untimed calls, `repeats` timed regions, each of at
    least min_calls calls and at least min_sec of GPU time (sized from a
    first timed pass over the sets); the median region.  With `host`, the
    median host issue time per call as well."""
    est = time_eager(fn, sets, len(sets), warmup)
    n = max(min_calls, len(sets), math.ceil(min_sec / max(est, 1e-9)))
    n = math.ceil(n / len(sets)) * len(sets)
    runs = []
    for _ in range(repeats):
        h = {}
        runs.append((time_eager(fn, sets, n, 0, h), h["s_per_step"]))
    runs.sort()
    sec, host_s = runs[len(runs) // 2]
    if host is not None:
        host["s_per_step"] = host_s
        host["calls"] = n
    return sec


def traffic_for(name, launches_key):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None
    when absent or taken on a different version of the kernel source.
    Entries are keyed "kernel@workload" (or, for the block's kernels,
    by kernel name with the workload recorded inside)."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get(f"{name}@{launches_key}") or t.get(name)
    if not e or e.get("source_sha") != source_sha(name) or e.get("workload") != launches_key:
        return None
    return e.get("bytes_per_launch")


def attention_sets(w, dev, n_max=16):
    """Rotating device copies of an attention workload's inputs (each with
    its own output), enough to cover ROTATE_BYTES."""
    import torch
    from workloads import configs
    inp = configs.make_inputs(w)
    one = working_set_bytes([inp["q"], inp["k"], inp["v"], inp["q"]])
    n_sets = max(2, min(n_max, math.ceil(ROTATE_BYTES / one)))
    sets = []
    for _ in range(n_sets):
        s = {k: v.to(dev) if v is not None else None for k, v in inp.items()}
        s["o"] = torch.empty_like(s["q"])
        sets.append(s)
    return inp, sets


def attention_call(w):
    import transformer_scaled_dot_fwd_amd as mha
    return lambda s: mha.mha_forward(s["q"], s["k"], s["v"], mask=w.mask, kv_lens=s["kv_lens"],
                                     out=s["o"], window=w.window)


def attention_sweep(dev, steps, warmup, workloads=None):
    """Attention alone at the base (h=8) and big (h=16) shapes, L >= 1024,
    plus the long causal workload (or the given workloads)."""
    import torch
    from workloads import accounting, configs
    out = []
    if workloads is None:
        workloads = [configs.get("c5")] + configs.sweep()
    for w in workloads:
        inp, sets = attention_sets(w, dev)
        fn = attention_call(w)
        host = {}
        sec = time_median(fn, sets, max(warmup, len(sets)), host,
                          min_calls=max(steps // 4, 2 * len(sets)))
        flops = accounting.attention_flops(w.B, w.h, w.Lq, w.Lk, w.d, w.mask, inp["kv_lens"],
                                           w.window)
        tf = flops / sec / 1e12
        exps = accounting.legal_pairs(w.B, w.h, w.Lq, w.Lk, w.mask, inp["kv_lens"], w.window)
        # The roofline of the row: Q, K, V and O cross HBM once, so FLOP per
        # byte is 4 d (legal pairs) / bytes.  Under the ridge point
        # (2.5e15 / 8e12 = 312) the attainable rate is that times 8 TB/s:
        # the causal L = 1024 rows and the restricted-attention band are
        # HBM-bound by it, the other rows MFMA-bound.
        nbytes = accounting.attention_bytes(w.B, w.h, w.Lq, w.Lk, w.d, w.mask, inp["kv_lens"],
                                            w.dtype)
        intensity = flops / nbytes
        attainable = min(PEAK_BF16_FLOPS, intensity * PEAK_HBM_BYTES)
        gbps = nbytes / sec / 1e9
        out.append({"workload": w.name, "B": w.B, "h": w.h, "d": w.d, "L": w.Lq,
                    "window": w.window, "exps": exps, "flops": flops,
                    "mask": "causal" if w.mask & 2 else "none", "us": round(sec * 1e6, 2),
                    "host_us": round(host["s_per_step"] * 1e6, 2), "calls": host["calls"],
                    "tflops": round(tf, 1), "frac_peak_bf16": round(tf * 1e12 / PEAK_BF16_FLOPS, 4),
                    "bytes": nbytes, "gbps": round(gbps, 1),
                    "frac_peak_hbm": round(gbps * 1e9 / PEAK_HBM_BYTES, 4),
                    "flop_per_byte": round(intensity, 1),
                    "roofline_bound": "mfma" if attainable >= PEAK_BF16_FLOPS else "hbm",
                    "attainable_tflops": round(attainable / 1e12, 1),
                    "frac_roofline": round(tf * 1e12 / attainable, 4)})
        log(f"  sweep {w.name}: {sec * 1e6:.1f} us, {tf:.1f} TFLOP/s "
            f"({100 * tf * 1e12 / PEAK_BF16_FLOPS:.1f}% of bf16 peak, "
            f"{100 * tf * 1e12 / attainable:.1f}% of its roofline)")
        del sets
        torch.cuda.empty_cache()
    return out


def metric_step(dev, steps, warmup):
    """The headline step: one mha_forward launch per row of metric_rows()
    (h = 8, d_k = 64, L >= 1024, no mask and causal), each row cycling over
    its own rotating buffer sets.  Returns seconds per step, FLOPs per step
    and the rows."""
    import torch
    from workloads import accounting, configs
    rows = []
    for w in configs.metric_rows():
        inp, sets = attention_sets(w, dev, n_max=12)
        rows.append({"w": w, "sets": sets, "fn": attention_call(w),
                     "flops": accounting.attention_flops(w.B, w.h, w.Lq, w.Lk, w.d, w.mask,
                                                         inp["kv_lens"])})
    counter = [0]

    def step(_):
        i = counter[0]
        for r in rows:
            r["fn"](r["sets"][i % len(r["sets"])])
        counter[0] = i + 1

    warm_gpu(step, [None], 0.3)
    host = {}
    sec = time_eager(step, [None], steps, warmup, host)
    flops = sum(r["flops"] for r in rows)
    desc = [f"{r['w'].name} ({len(r['sets'])} sets)" for r in rows]
    del rows
    torch.cuda.empty_cache()
    return sec, flops, host["s_per_step"], desc


def hbm_workloads(dev, steps, warmup, copy_gbps):
    """The short-sequence workloads, whose attention is HBM-bound (FLOP per
    byte far under the ridge point of 2.5e15 / 8e12 = 312): algorithmic
    bytes (Q and O once, the legal K/V rows, the lengths) per second."""
    import torch
    import transformer_scaled_dot_fwd_amd as mha
    from workloads import accounting, configs
    out = []
    for name in ("c2", "c4", "c3"):
        w = configs.get(name)
        if w.block:
            # the block's attention on its own projected Q, K, V
            inputs = configs.make_inputs(w)
            probe = Block(w, inputs, dev, 1)
            s0 = probe.sets[0]
            one = working_set_bytes([s0[k] for k in ("q", "k", "v", "o")])
            del probe
            blk = Block(w, inputs, dev, max(2, min(16, math.ceil(ROTATE_BYTES / one))))
            for s in blk.sets:
                blk.project_qkv(s)
            sets, fn, lens = blk.sets, blk.attention, inputs["kv_lens"]
            what = "attention of the base decoder block (causal + key padding)"
        else:
            inp, sets = attention_sets(w, dev)
            fn, lens = attention_call(w), inp["kv_lens"]
            what = w.description
        host = {}
        sec_eager = time_median(fn, sets, max(warmup, len(sets)), host,
                                min_calls=max(steps // 4, 2 * len(sets)))
        # A launch this short is shorter than one eager call's host issue
        # time, so the kernel's own time comes from graph replays.
        sec = kernel_time(fn, sets, max(steps, 4 * len(sets)), max(warmup, len(sets)))
        nbytes = accounting.attention_bytes(w.B, w.h, w.Lq, w.Lk, w.d, w.mask, lens, w.dtype)
        flops = accounting.attention_flops(w.B, w.h, w.Lq, w.Lk, w.d, w.mask, lens)
        gbps = nbytes / sec / 1e9
        out.append({"workload": w.name, "what": what, "bound": "hbm", "bytes": nbytes,
                    "us": round(sec * 1e6, 2), "timing": "graph replays, one launch per buffer set",
                    "us_eager": round(sec_eager * 1e6, 2),
                    "host_us": round(host["s_per_step"] * 1e6, 2),
                    "calls": host["calls"], "gbps": round(gbps, 1),
                    "frac_peak_hbm": round(gbps * 1e9 / PEAK_HBM_BYTES, 4),
                    "frac_of_copy": round(gbps / copy_gbps, 4) if copy_gbps else None,
                    "tflops": round(flops / sec / 1e12, 1)})
        log(f"  hbm {w.name}: {sec * 1e6:.2f} us ({sec_eager * 1e6:.2f} eager), {gbps:.0f} GB/s "
            f"({100 * gbps * 1e9 / PEAK_HBM_BYTES:.1f}% of HBM peak)")
        del sets
        torch.cuda.empty_cache()
    return out


def copy_bandwidth(dev, nbytes=512 << 20, reps=20):
    """A plain device-to-device copy of nbytes (torch's copy, a runtime blit
    kernel), timed with HIP events on the current stream after a few untimed
    copies: bytes read plus bytes written per second.  The practical HBM
    ceiling the HBM-bound kernels are set against, next to the 8 TB/s spec."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / reps
        best = sec if best is None else min(best, sec)
    del src, dst
    torch.cuda.empty_cache()
    gbps = 2 * nbytes / best / 1e9
    return {"bytes_per_copy": 2 * nbytes, "us": round(best * 1e6, 2), "gbps": round(gbps, 1),
            "frac_peak_hbm": round(gbps * 1e9 / PEAK_HBM_BYTES, 4)}


def decode_sweep(dev, steps, warmup, copy_gbps=None):
    """One decoding step against a K/V cache (mha_decode): HBM-bound, so
    reported as algorithmic GB/s (the valid K/V rows, q, o and the lengths)
    against the 8 TB/s peak, next to the TFLOP/s of its 4 d FLOPs per key."""
    import torch
    import transformer_scaled_dot_fwd_amd as mha
    from workloads import accounting, configs
    out = []
    for w in configs.decodes():
        inp = configs.make_inputs(w)
        one = working_set_bytes([inp["q"], inp["k"], inp["v"], inp["q"]])
        n_sets = max(2, min(16, math.ceil(ROTATE_BYTES / one)))
        ws = torch.empty(int(mha.lib().mha_decode_workspace_bytes(w.B, w.h, w.Lk, w.d)),
                         dtype=torch.uint8, device=dev)
        sets = []
        for _ in range(n_sets):
            s = {k: v.to(dev) if v is not None else None for k, v in inp.items()}
            s["o"] = torch.empty_like(s["q"])
            sets.append(s)
        fn = lambda s: mha.mha_decode(s["q"], s["k"], s["v"], s["kv_lens"], out=s["o"],
                                      workspace=ws)
        host = {}
        sec = time_median(fn, sets, max(warmup, n_sets), host, min_calls=max(steps // 4, 2 * n_sets))
        lens = inp["kv_lens"]
        nbytes = accounting.attention_bytes(w.B, w.h, 1, w.Lk, w.d, w.mask, lens, w.dtype)
        flops = accounting.attention_flops(w.B, w.h, 1, w.Lk, w.d, w.mask, lens)
        gbps = nbytes / sec / 1e9
        out.append({"workload": w.name, "B": w.B, "h": w.h, "d": w.d, "L_cache": w.Lk,
                    "us": round(sec * 1e6, 2), "host_us": round(host["s_per_step"] * 1e6, 2),
                    "calls": host["calls"], "gbps": round(gbps, 1),
                    "frac_peak_hbm": round(gbps * 1e9 / PEAK_HBM_BYTES, 4),
                    "frac_of_copy": round(gbps / copy_gbps, 4) if copy_gbps else None,
                    "tflops": round(flops / sec / 1e12, 2)})
        log(f"  decode {w.name}: {sec * 1e6:.1f} us, {gbps:.0f} GB/s "
            f"({100 * gbps * 1e9 / PEAK_HBM_BYTES:.1f}% of HBM peak)")
        del sets
        torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sample_rows(w, n, seed):
    """n random (b, head, i) rows of an attention workload."""
    import numpy as np
    rng = np.random.default_rng(seed)
    return np.stack([rng.integers(0, w.B, n), rng.integers(0, w.h, n),
                     rng.integers(0, w.Lq, n)], axis=1).astype(np.int64)


def row_flops(w, rows, kv_lens):
    """Algorithmic FLOPs of the given rows: 4 d per legal key."""
    import numpy as np
    b, i = rows[:, 0], rows[:, 2]
    n = np.full(len(rows), w.Lk, dtype=np.int64)
    if w.mask & 1:
        n = np.minimum(n, np.clip(np.asarray(kv_lens, dtype=np.int64)[b], 0, w.Lk))
    if w.mask & 2:
        n = np.minimum(n, i + 1)
    return int(4 * w.d * n.sum())


def oracle_rows_rate(w, budget_s, seed):
    """The oracle's attention over random rows of workload w, doubling the
    sample until it takes about budget_s: (seconds, rows, FLOPs)."""
    import oracle
    from workloads import configs
    inp = configs.make_inputs(w)
    n = 64
    while True:
        rows = sample_rows(w, n, seed)
        t0 = time.perf_counter()
        oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, mask=w.mask,
                              kv_lens=inp["kv_lens"], window=w.window)
        sec = time.perf_counter() - t0
        if sec >= budget_s / 2 or n >= 1 << 20:
            return sec, n, row_flops(w, rows, inp["kv_lens"])
        n *= 2


def cpu_baseline(budget_s):
    """The fp64 oracle (as it stands) on a bounded sample of the headline
    workload: random rows of each of the six rows of metric_rows(), about
    budget_s seconds in all."""
    import oracle
    from workloads import configs
    total_s, total_f, parts = 0.0, 0, []
    rows = configs.metric_rows()
    for n, w in enumerate(rows):
        sec, nr, f = oracle_rows_rate(w, budget_s / len(rows), 31 + n)
        total_s += sec
        total_f += f
        parts.append(f"{nr} rows of {w.name}")
    return {"value": round(total_f / total_s / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "random query rows (all heads, both masks) of the h=8 d_k=64 L>=1024 "
                      f"rows: {', '.join(parts)}; {total_s:.1f} s of oracle time, "
                      f"{total_f / 1e9:.2f} GFLOP"}


def oracle_per_config(budget_s):
    """The oracle's seconds for each configuration: c1 (best of 100), c2,
    c3 (the whole block) and c4 (best of 3) in full; c5 and the headline
    rows extrapolated from a timed sample of random rows by FLOPs (stated
    per entry)."""
    import oracle
    from workloads import accounting, configs
    out = {}

    def best(fn, n):
        t = []
        for _ in range(n):
            t0 = time.perf_counter()
            fn()
            t.append(time.perf_counter() - t0)
        return min(t)

    for name, reps in (("c1", 100), ("c2", 3), ("c3", 1), ("c4", 1)):
        w = configs.get(name)
        inp = configs.make_inputs(w)
        lens = inp["kv_lens"]
        if w.block:
            fn = lambda: oracle.mha_block(inp["x"], inp["x"], inp["w_q"], inp["w_k"],
                                          inp["w_v"], inp["w_o"], h=w.h, mask=w.mask,
                                          kv_lens=lens)
            flops = accounting.workload_work(w, lens.numpy())["total_flops"]
        else:
            fn = lambda: oracle.attention(inp["q"], inp["k"], inp["v"], mask=w.mask,
                                          kv_lens=lens)
            flops = accounting.attention_flops(w.B, w.h, w.Lq, w.Lk, w.d, w.mask, lens)
        sec = best(fn, reps)
        out[name] = {"workload": w.name, "seconds": round(sec, 4),
                     "gflops": round(flops / sec / 1e9, 3), "how": f"full, best of {reps}"}
    for w in [configs.get("c5")] + configs.metric_rows():
        sec, nr, f = oracle_rows_rate(w, budget_s / 7, 77)
        # these workloads have no key padding: no lengths
        full = accounting.attention_flops(w.B, w.h, w.Lq, w.Lk, w.d, w.mask)
        rate = f / sec
        key = "c5" if w.name == configs.get("c5").name else w.name
        out[key] = {"workload": w.name, "seconds": round(full / rate, 2),
                    "gflops": round(rate / 1e9, 3),
                    "how": f"extrapolated by FLOPs from {nr} random rows ({sec:.2f} s)"}
    return out


def kernel_only_block(w, dev, args):
    """One kernel of the block workload alone (or a device copy), for trace
    and counter runs."""
    import torch
    inputs = configs_make(w)
    blk = Block(w, inputs, dev, 4)
    for s in blk.sets:
        blk.project_qkv(s)
    if args.kernel_only == "copy":
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy: 256 MiB per launch")
        return
    if args.kernel_only == "decode":
        raise SystemExit("--kernel-only decode needs a decode workload")
    fn = getattr(blk, args.kernel_only)
    t0 = time.perf_counter()
    warm = 0
    while time.perf_counter() - t0 < args.warm_seconds:
        fn(blk.sets[warm % len(blk.sets)])
        warm += 1
        if warm % 50 == 0:
            torch.cuda.synchronize()
    for i in range(args.steps):
        fn(blk.sets[i % len(blk.sets)])
    torch.cuda.synchronize()
    log(f"{args.kernel_only} on {w.name}: {warm} warm-up launches, then {args.steps} launches")


def configs_make(w):
    from workloads import configs
    return configs.make_inputs(w)


def kernel_only_attention(w, dev, args):
    """mha_forward (or, for a decode workload, mha_decode) alone on an
    attention workload, for trace and counter runs."""
    import torch
    import transformer_scaled_dot_fwd_amd as mha
    from workloads import configs
    if args.kernel_only == "attention":
        # the rotating buffer sets the sweep times, so a trace's average
        # launch is the sweep's
        _, sets = attention_sets(w, dev)
        fn = attention_call(w)
        counter = [0]

        def call():
            fn(sets[counter[0] % len(sets)])
            counter[0] += 1
    elif args.kernel_only == "decode":
        if w.Lq != 1:
            raise SystemExit("--kernel-only decode needs a decode workload")
        inp = configs.make_inputs(w, dev)
        o = torch.empty_like(inp["q"])
        ws = torch.empty(int(mha.lib().mha_decode_workspace_bytes(w.B, w.h, w.Lk, w.d)),
                         dtype=torch.uint8, device=dev)
        call = lambda: mha.mha_decode(inp["q"], inp["k"], inp["v"], inp["kv_lens"], out=o,
                                      workspace=ws)
    else:
        raise SystemExit("attention workloads run the attention (or decode) kernels only")
    warm = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.warm_seconds:
        for _ in range(10):
            call()
        torch.cuda.synchronize()
        warm += 10
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    log(f"{args.kernel_only} on {w.name}: {warm} warm-up launches, then {args.steps} launches")


def block_step(dev, args, copy_gbps):
    """The base decoder block (c3): the step, every kernel of it timed alone
    in the same rotation, the dominant kernel's roofline, and the sub-layer
    with its residual and post-norm."""
    import torch
    from workloads import accounting, configs
    w = configs.get("c3")
    inputs = configs.make_inputs(w)
    work = accounting.workload_work(w, inputs["kv_lens"].numpy())
    probe = Block(w, inputs, dev, 1)
    s0 = probe.sets[0]
    one = working_set_bytes([s0[k] for k in ("x", "w_q", "w_k", "w_v", "w_o", "q", "k", "v",
                                             "o", "y", "z")])
    n_sets = max(1, min(64, math.ceil(ROTATE_BYTES / one)))
    del probe
    blk = Block(w, inputs, dev, n_sets)
    blk.fused = (not args.unfused) and blk.fused_supported()
    log(f"block {w.name}: working set {one / 1e6:.1f} MB x {n_sets} rotating sets; "
        f"{'fused self-attention + W^O' if blk.fused else 'projection + attention + W^O'}")
    warm_gpu(blk.step, blk.sets, 0.3)
    host = {}
    sec_step = time_eager(blk.step, blk.sets, args.steps, args.warmup, host)
    sec_graph = time_steps(blk.step, blk.sets, args.steps, args.warmup)
    sec_warm = time_eager(blk.step, blk.sets[:1], args.steps, args.warmup)
    flops_step = work["total_flops"]
    log(f"block step: {sec_step * 1e6:.2f} us, {flops_step / sec_step / 1e12:.1f} TFLOP/s")

    step_kernels = (["self_attention_fused", "out_proj"] if blk.fused
                    else ["project_qkv", "attention", "out_proj"])
    names = step_kernels + (["project_qkv", "attention"] if blk.fused else [])
    names.append("out_proj_post_norm")
    per = {}
    for name in names:
        per[name] = kernel_time(getattr(blk, name), blk.sets, max(args.steps, 2 * n_sets),
                                args.warmup)
        log(f"  {name}: {per[name] * 1e6:.2f} us"
            + ("" if name in step_kernels else " (not in the step)"))
    dom = max(step_kernels, key=per.get)
    if dom == "attention":
        bound, alg, unit, peak = "hbm", work["attention"]["bytes"], "GB/s", PEAK_HBM_BYTES
    else:
        bound, alg, unit, peak = "mfma", work[dom]["flops"], "TFLOP/s", PEAK_BF16_FLOPS
    scale = 1e9 if unit == "GB/s" else 1e12
    roofline = {"kernel": dom, "bound": bound, "achieved": round(alg / per[dom] / scale, 2),
                "peak": round(peak / scale, 1), "unit": unit,
                "frac": round(alg / per[dom] / peak, 4), "traffic": traffic_for(dom, w.name),
                "avg_launch_us": round(per[dom] * 1e6, 3)}
    kernels = {name: {"us": round(sec * 1e6, 3),
                      "tflops": round(work[name]["flops"] / sec / 1e12, 1),
                      "gbps": round(work[name]["bytes"] / sec / 1e9, 1),
                      "in_step": name in step_kernels} for name, sec in per.items()}
    pn = "out_proj_post_norm"
    pn_bytes = work[pn]["bytes"]
    sec_sub = time_eager(blk.sublayer_step, blk.sets, args.steps, args.warmup)
    post_norm = {
        "kernel": pn, "bound": "hbm", "us": round(per[pn] * 1e6, 3),
        "achieved": round(pn_bytes / per[pn] / 1e9, 1), "peak": PEAK_HBM_BYTES / 1e9,
        "unit": "GB/s", "frac": round(pn_bytes / per[pn] / PEAK_HBM_BYTES, 4),
        "frac_of_copy": round(pn_bytes / per[pn] / 1e9 / copy_gbps, 4),
        "tflops": round(work[pn]["flops"] / per[pn] / 1e12, 1),
        "intensity_flop_per_byte": round(work[pn]["flops"] / pn_bytes, 1),
        "traffic": traffic_for(pn, w.name),
        "vs_out_proj_gemm_us": round(per["out_proj"] * 1e6, 3),
        "sublayer_step_us": round(sec_sub * 1e6, 3),
        "sublayer_step": " -> ".join(step_kernels[:-1] + [pn]),
    }
    out = {"workload": w.name, "description": w.description,
           "step": " -> ".join(step_kernels) + f" (direct launches over {n_sets} buffer sets)",
           "us_per_step": round(sec_step * 1e6, 3),
           "us_per_step_host_issue": round(host["s_per_step"] * 1e6, 3),
           "us_per_step_graphs": round(sec_graph * 1e6, 3),
           "us_per_step_warm_cache": round(sec_warm * 1e6, 3),
           "flops_per_step": flops_step,
           "tflops": round(flops_step / sec_step / 1e12, 2),
           "frac_peak_bf16": round(flops_step / sec_step / PEAK_BF16_FLOPS, 4),
           "kernels": kernels, "roofline": roofline, "post_norm": post_norm}
    del blk
    torch.cuda.empty_cache()
    return out


def fp32_path(dev, steps, warmup):
    """The fp32 (accuracy) path, which runs on the matrix cores too: the tiny
    workload (c1, launch-bound) and fp32 inputs at the base shapes --
    attention at h = 8, d = 64, L = 1024, B = 4 without a mask, and the base
    block's projections, W^O and post-norm (X [64, 128, 512]).  Rotating
    input sets, direct launches, median of five timed regions."""
    import torch
    import transformer_scaled_dot_fwd_amd as mha
    from workloads import configs, generate
    out = []

    def entry(name, what, fn, sets, flops):
        sec = time_median(fn, sets, max(warmup, len(sets)), None,
                          min_calls=max(steps // 4, 2 * len(sets)))
        tf = flops / sec / 1e12
        out.append({"kernel": name, "what": what, "us": round(sec * 1e6, 2),
                    "tflops": round(tf, 2), "frac_peak_fp32": round(tf * 1e12 / PEAK_FP32_FLOPS, 4)})
        log(f"  fp32 {name}: {sec * 1e6:.1f} us, {tf:.2f} TFLOP/s")

    w = configs.get("c1")
    inp = configs.make_inputs(w)
    sets = [{k: v.to(dev) for k, v in inp.items() if v is not None} for _ in range(4)]
    entry("attention", w.description,
          lambda s: mha.mha_forward(s["q"], s["k"], s["v"]), sets,
          4.0 * w.d * w.B * w.h * w.Lq * w.Lk)
    B, L, h, d = 4, 1024, 8, 64
    sets = [{"q": generate.normal((B, L, h, d), 9600 + 3 * i, "f32").to(dev),
             "k": generate.normal((B, L, h, d), 9601 + 3 * i, "f32").to(dev),
             "v": generate.normal((B, L, h, d), 9602 + 3 * i, "f32").to(dev)} for i in range(4)]
    for s in sets:
        s["o"] = torch.empty_like(s["q"])
    entry("attention", f"B={B} h={h} L={L} d={d} fp32, no mask",
          lambda s: mha.mha_forward(s["q"], s["k"], s["v"], out=s["o"]), sets,
          4.0 * d * B * h * L * L)
    del sets
    B, L, dm, h = 64, 128, 512, 8
    M = B * L
    sets = []
    for i in range(4):
        s = {"x": generate.normal((B, L, dm), 9700 + 8 * i, "f32").to(dev),
             "w": [generate.normal((dm, dm), 9701 + 8 * i + j, "f32", std=dm ** -0.5).to(dev)
                   for j in range(4)],
             "g": torch.ones(dm, device=dev), "b": torch.zeros(dm, device=dev)}
        s["q"], s["k"], s["v"] = (torch.empty((B, L, h, dm // h), device=dev) for _ in range(3))
        s["y"] = torch.empty((B, L, dm), device=dev)
        sets.append(s)
    entry("project_qkv", "X [64, 128, 512] fp32 -> Q, K, V (h = 8)",
          lambda s: mha.mha_project_qkv(s["x"], s["x"], *s["w"][:3], h, out=(s["q"], s["k"], s["v"])),
          sets, 3 * 2.0 * M * dm * dm)
    entry("out_proj", "O [64, 128, 8, 64] fp32 -> Y [64, 128, 512]",
          lambda s: mha.mha_out_proj(s["q"], s["w"][3], out=s["y"]), sets, 2.0 * M * dm * dm)
    entry("out_proj_post_norm", "LayerNorm(x + O W^O), [64, 128, 512] fp32",
          lambda s: mha.mha_out_proj_post_norm(s["q"], s["w"][3], s["x"], s["g"], s["b"],
                                               out=s["y"]), sets, 2.0 * M * dm * dm)
    del sets
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_scaled_dot_fwd_amd as mha
    from workloads import accounting, configs

    mha.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    if args.kernel_only:
        w = configs.get(args.workload)
        if not w.block:
            return kernel_only_attention(w, dev, args)
        return kernel_only_block(w, dev, args)

    # ---- the headline step: the h = 8 rows of the L >= 1024 sweep ----
    sec_step, flops_step, host_s, desc = metric_step(dev, args.steps, args.warmup)
    value = flops_step / sec_step / 1e12
    log(f"step (h=8 L>=1024 rows): {sec_step * 1e6:.1f} us, {value:.1f} TFLOP/s "
        f"({100 * value * 1e12 / PEAK_BF16_FLOPS:.1f}% of bf16 peak)")

    # ---- every sweep row alone; the dominant kernel's roofline ----
    sweep = attention_sweep(dev, args.steps, args.warmup)
    rows8 = {r.name for r in configs.metric_rows()}
    dom = max((e for e in sweep if e["workload"] in rows8), key=lambda e: e["us"])
    roofline = {"kernel": "attn_stream_bf16 (streaming attention, d=64)",
                "workload": dom["workload"], "bound": "mfma",
                "achieved": round(dom["flops"] / (dom["us"] * 1e-6) / 1e12, 1),
                "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                "frac": dom["frac_peak_bf16"],
                "traffic": traffic_for("attn_stream", dom["workload"]),
                "avg_launch_us": dom["us"],
                "algorithmic_flops_per_launch": dom["flops"]}
    copy = copy_bandwidth(dev)
    log(f"device copy: {copy['gbps']:.0f} GB/s read + written "
        f"({100 * copy['frac_peak_hbm']:.1f}% of the HBM peak)")
    hbm = hbm_workloads(dev, args.steps, args.warmup, copy["gbps"])
    block = block_step(dev, args, copy["gbps"])
    heads = windowed = decoded = None
    if not args.no_sweep:
        heads = attention_sweep(dev, args.steps, args.warmup, configs.head_sizes())
        windowed = attention_sweep(dev, args.steps, args.warmup, configs.windows())
        decoded = decode_sweep(dev, args.steps, args.warmup, copy["gbps"])
    f32 = fp32_path(dev, args.steps, args.warmup)
    cpu = oracle_cfg = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds)
        log(f"cpu baseline: {cpu}")
        oracle_cfg = oracle_per_config(args.cpu_seconds)
        log(f"oracle per config: {oracle_cfg}")

    line = {
        "metric": "attention fwd TFLOP/s & % peak bf16 MFMA at h=8,d_k=64 (1 MI355X)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_step * 1e3, 5),
        "ms_per_step_host_issue": round(host_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1) Q/K/V, bf16)",
        "config": {"workload": "attention forward, h=8 d_k=64, L in {1024, 2048, 4096} with "
                               "B = 24576/L, no mask and causal (six mha_forward launches "
                               "per step)",
                   "rows": desc, "h": 8, "d_k": 64, "flops_per_step": flops_step,
                   "value_is": "sum of the six rows' algorithmic FLOPs / step time"},
        "frac_peak_bf16": round(value * 1e12 / PEAK_BF16_FLOPS, 4),
        "roofline": roofline,
        "attention_sweep": sweep,
        "hbm_workloads": hbm,
        "hbm_copy": copy,
        "block_step": block,
        "head_size_sweep": heads,
        "window_sweep": windowed,
        "decode_sweep": decoded,
        "fp32_path": f32,
        "cpu_baseline": cpu,
        "oracle_per_config": oracle_cfg,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
