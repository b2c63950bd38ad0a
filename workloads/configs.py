"""Named problem shapes.

Shapes follow the pages' models: base (d_model 512, h 8, d_k = d_v = 64) and
big (d_model 1024, h 16, d_k = d_v = 64) -- Deep-reading page section 08,
Table 3 rows "base" and "big" -- and their ~25k-token length-grouped batches
(slide "Training Details"; Deep-reading page section 06).  The pages'
WMT14 batches themselves are not used: i.i.d. N(0, 1) inputs of the same
geometry stand in for them (N(0, 1) components are the premise of the
1/sqrt(d_k) argument in Deep-reading page section 04).

Seeds: 1000 * config_number + tensor_number, tensor numbers q=0, k=1, v=2,
x_q=3, w_q=4, w_k=5, w_v=6, w_o=7, x_kv=8, lens=9, gamma=10,
beta=11.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import generate

MASK_NONE = 0
MASK_KEY_PADDING = 1
MASK_CAUSAL = 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    number: int              # seed base = 1000 * number
    B: int
    h: int
    Lq: int
    Lk: int
    d: int                   # d_k = d_v
    dtype: str               # "f32" | "bf16"
    mask: int
    lens: Optional[tuple] = None   # (lo, hi) of the key-padding lengths
    block: bool = False      # full block: projections + attention + W^O
    d_model: int = 0
    description: str = ""
    window: Optional[int] = None   # restricted attention half-width

    @property
    def seed(self) -> int:
        return 1000 * self.number

    def label(self) -> str:
        return self.name


C1 = Workload("tiny_selfattn_f32", 1, B=1, h=2, Lq=16, Lk=16, d=8, dtype="f32",
              mask=MASK_NONE,
              description="tiny self-attention, B=1 h=2 L=16 d=8 fp32, no mask")
C2 = Workload("base_encoder_selfattn_pad", 2, B=64, h=8, Lq=128, Lk=128, d=64,
              dtype="bf16", mask=MASK_KEY_PADDING, lens=(32, 128),
              description="base encoder self-attention, B=64 h=8 L=128 d=64 bf16, "
                          "key padding lens U{32..128}")
C3 = Workload("base_decoder_block_causal_pad", 3, B=64, h=8, Lq=128, Lk=128, d=64,
              dtype="bf16", mask=MASK_CAUSAL | MASK_KEY_PADDING, lens=(32, 128),
              block=True, d_model=512,
              description="base decoder multi-head block, X [64,128,512] bf16, "
                          "W 512x512 N(0,1/512), h=8 d=64, causal + key padding "
                          "lens U{32..128}: QKV projection, attention, W^O")
C4 = Workload("big_cross_attn_pad", 4, B=256, h=16, Lq=96, Lk=128, d=64, dtype="bf16",
              mask=MASK_KEY_PADDING, lens=(48, 128),
              description="big cross-attention, B=256 h=16 Lq=96 over Lk=128 encoder "
                          "memory, d=64 bf16, encoder padding lens U{48..128}")
C5 = Workload("long_causal", 5, B=4, h=16, Lq=4096, Lk=4096, d=64, dtype="bf16",
              mask=MASK_CAUSAL,
              description="long causal self-attention, B=4 h=16 L=4096 d=64 bf16")

CONFIGS = {w.name: w for w in (C1, C2, C3, C4, C5)}
# short aliases in configuration order
ALIASES = {"c1": C1.name, "c2": C2.name, "c3": C3.name, "c4": C4.name, "c5": C5.name}


def sweep():
    """The L >= 1024 sweep at the base (h=8) and big (h=16) head shapes:
    d=64, L in {1024, 2048, 4096}, B = 24576 / L (~25k tokens per batch),
    no mask and causal."""
    out = []
    n = 60
    for h in (8, 16):
        for L in (1024, 2048, 4096):
            for mask, tag in ((MASK_NONE, "nomask"), (MASK_CAUSAL, "causal")):
                n += 1
                out.append(Workload(f"sweep_h{h}_L{L}_{tag}", n, B=24576 // L, h=h,
                                    Lq=L, Lk=L, d=64, dtype="bf16", mask=mask,
                                    description=f"h={h} L={L} B={24576 // L} d=64 bf16 {tag}"))
    return out


def metric_rows():
    """The rows the headline figure aggregates: the L >= 1024 sweep at the
    base model's head shape (h = 8, d_k = 64), no mask and causal."""
    return [w for w in sweep() if w.h == 8]


def head_sizes():
    """The other head shapes of the base model's width (d_model 512; Deep-
    reading page section 08, Table 3, rows (A)): h=32 d=16, h=16 d=32, h=4
    d=128, at L in {1024, 4096} with B = 24576 / L, no mask and causal."""
    out = []
    n = 80
    for h, d in ((32, 16), (16, 32), (4, 128)):
        for L in (1024, 4096):
            for mask, tag in ((MASK_NONE, "nomask"), (MASK_CAUSAL, "causal")):
                n += 1
                out.append(Workload(f"heads_h{h}_d{d}_L{L}_{tag}", n, B=24576 // L, h=h,
                                    Lq=L, Lk=L, d=d, dtype="bf16", mask=mask,
                                    description=f"h={h} d={d} L={L} B={24576 // L} bf16 {tag}"))
    return out


def windows():
    """Restricted self-attention (Deep-reading page section 05, complexity
    table): the base and big head shapes at L = 4096 (B = 6), each query
    seeing the keys within w = 256 positions (r = 513), no mask and causal."""
    out = []
    n = 100
    for h in (8, 16):
        for mask, tag in ((MASK_NONE, "nomask"), (MASK_CAUSAL, "causal")):
            n += 1
            out.append(Workload(f"window_h{h}_L4096_w256_{tag}", n, B=6, h=h, Lq=4096, Lk=4096,
                                d=64, dtype="bf16", mask=mask, window=256,
                                description=f"h={h} L=4096 B=6 d=64 bf16 {tag}, window 256"))
    return out


def decodes():
    """One decoding step against a K/V cache (Deep-reading page section 03,
    one position per step; beam search with beam 4, section 06): 16
    sequences x 4 beams = 64 cache rows of up to 4096 positions, lengths
    U{2048..4096}, at the base (h=8) and big (h=16) head shapes, d=64.
    Lq = 1: the step's query per head."""
    out = []
    for n, h in ((121, 8), (122, 16)):
        out.append(Workload(f"decode_h{h}_B64_L4096", n, B=64, h=h, Lq=1, Lk=4096, d=64,
                            dtype="bf16", mask=MASK_KEY_PADDING, lens=(2048, 4096),
                            description=f"decode step: 64 caches (16 x beam 4), h={h}, "
                                        f"d=64, L_cache=4096, lens U{{2048..4096}}"))
    return out


def get(name: str) -> Workload:
    name = ALIASES.get(name, name)
    if name in CONFIGS:
        return CONFIGS[name]
    for w in sweep() + head_sizes() + windows() + decodes():
        if w.name == name:
            return w
    raise KeyError(name)


def make_inputs(w: Workload, device="cpu") -> dict:
    """Seeded inputs of a workload, as torch tensors on ``device``.

    Attention-only workloads: q, k, v (BLHD) and kv_lens.  Block workloads:
    x (the decoder input, used as both X_q and X_kv: self-attention),
    w_q, w_k, w_v, w_o, kv_lens, and gamma, beta of the post-norm.  Weights are N(0, 1/d_model): the second
    parameter of N(., .) is read as the variance.
    """
    s = w.seed
    out = {}
    if w.block:
        dm = w.d_model
        out["x"] = generate.normal((w.B, w.Lq, dm), s + 3, w.dtype)
        std = dm ** -0.5
        out["w_q"] = generate.normal((dm, w.h * w.d), s + 4, w.dtype, std)
        out["w_k"] = generate.normal((dm, w.h * w.d), s + 5, w.dtype, std)
        out["w_v"] = generate.normal((dm, w.h * w.d), s + 6, w.dtype, std)
        out["w_o"] = generate.normal((w.h * w.d, dm), s + 7, w.dtype, std)
        # gain and bias of the post-norm LayerNorm: 1 + 0.1 N(0, 1), 0.1 N(0, 1)
        out["gamma"] = (1.0 + generate.normal((dm,), s + 10, "f32", 0.1)).to(
            generate.torch_dtype(w.dtype))
        out["beta"] = generate.normal((dm,), s + 11, w.dtype, 0.1)
    else:
        out["q"] = generate.normal((w.B, w.Lq, w.h, w.d), s + 0, w.dtype)
        out["k"] = generate.normal((w.B, w.Lk, w.h, w.d), s + 1, w.dtype)
        out["v"] = generate.normal((w.B, w.Lk, w.h, w.d), s + 2, w.dtype)
    if w.mask & MASK_KEY_PADDING:
        out["kv_lens"] = generate.lengths(w.B, w.lens[0], w.lens[1], s + 9)
    else:
        out["kv_lens"] = None
    if device != "cpu":
        out = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in out.items()}
    return out
