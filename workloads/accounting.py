"""Algorithmic work of a workload: FLOPs and HBM bytes the method itself
needs, excluding padded or skipped work.

Attention: QK^T and PV each cost 2*d FLOPs per legal (query, key) pair, the
n^2 d term of the self-attention row of Table 1 (Deep-reading page section
05).  Bytes: Q and O once, and only the legal K/V rows (padding rows need
not be read), plus the int32 lengths.  GEMM: 2*M*N*K FLOPs and
(M*K + K*N + M*N) elements.
"""
from __future__ import annotations

import numpy as np

from .configs import MASK_CAUSAL, MASK_KEY_PADDING, Workload

ELEM_BYTES = {"f32": 4, "bf16": 2}


def legal_pairs(B, h, Lq, Lk, mask, kv_lens=None, window=None) -> int:
    """Number of (b, head, i, j) with M_ij = 0 (with a window w, only
    |i - j| <= w; restricted attention, Deep-reading page section 05)."""
    if window is not None:
        lens = (np.clip(np.asarray(kv_lens, dtype=np.int64), 0, Lk)
                if mask & MASK_KEY_PADDING else np.full(B, Lk, dtype=np.int64))
        i = np.arange(Lq, dtype=np.int64)
        lo = np.maximum(i - window, 0)
        total = 0
        for L in lens:
            hi = np.minimum(i + window, int(L) - 1)
            if mask & MASK_CAUSAL:
                hi = np.minimum(hi, i)
            total += int(np.maximum(hi - lo + 1, 0).sum())
        return total * h
    if mask & MASK_KEY_PADDING:
        lens = np.clip(np.asarray(kv_lens, dtype=np.int64), 0, Lk)
    else:
        lens = np.full(B, Lk, dtype=np.int64)
    total = 0
    for L in lens:
        L = int(L)
        if mask & MASK_CAUSAL:
            # query i sees keys 0..min(i, L-1): sum_i min(i+1, L)
            m = min(L, Lq)
            total += m * (m + 1) // 2 + (Lq - m) * L
        else:
            total += Lq * L
    return total * h


def attention_flops(B, h, Lq, Lk, d, mask, kv_lens=None, window=None) -> int:
    return 4 * d * legal_pairs(B, h, Lq, Lk, mask, kv_lens, window)


def attention_bytes(B, h, Lq, Lk, d, mask, kv_lens=None, dtype="bf16") -> int:
    e = ELEM_BYTES[dtype]
    if mask & MASK_KEY_PADDING:
        kv_rows = int(np.clip(np.asarray(kv_lens, dtype=np.int64), 0, Lk).sum())
    else:
        kv_rows = B * Lk
    qo = 2 * B * Lq * h * d
    kv = 2 * kv_rows * h * d
    lens = 4 * B if (mask & MASK_KEY_PADDING) else 0
    return e * (qo + kv) + lens


def gemm_flops(M, N, K) -> int:
    return 2 * M * N * K


def gemm_bytes(M, N, K, dtype="bf16") -> int:
    return ELEM_BYTES[dtype] * (M * K + K * N + M * N)


def workload_work(w: Workload, kv_lens=None) -> dict:
    """Per-step algorithmic FLOPs and bytes of each stage of a workload."""
    att_f = attention_flops(w.B, w.h, w.Lq, w.Lk, w.d, w.mask, kv_lens)
    att_b = attention_bytes(w.B, w.h, w.Lq, w.Lk, w.d, w.mask, kv_lens, w.dtype)
    out = {"attention": {"flops": att_f, "bytes": att_b,
                         "pairs": legal_pairs(w.B, w.h, w.Lq, w.Lk, w.mask, kv_lens)}}
    if w.block:
        M = w.B * w.Lq
        n = w.h * w.d
        qkv_f = 3 * gemm_flops(M, n, w.d_model)
        # X read once (self-attention: X_q is X_kv), three weights, three outputs
        qkv_b = ELEM_BYTES[w.dtype] * (M * w.d_model + 3 * w.d_model * n + 3 * M * n)
        out["project_qkv"] = {"flops": qkv_f, "bytes": qkv_b}
        out["out_proj"] = {"flops": gemm_flops(M, w.d_model, n),
                           "bytes": gemm_bytes(M, w.d_model, n, w.dtype)}
        # W^O with the residual add and the post-norm: the product's FLOPs
        # (the normalisation adds O(M d_model), under 1%); bytes: O, W^O, the
        # residual x, the output, gain and bias.
        e = ELEM_BYTES[w.dtype]
        out["out_proj_post_norm"] = {
            "flops": gemm_flops(M, w.d_model, n),
            "bytes": e * (M * n + n * w.d_model + 2 * M * w.d_model + 2 * w.d_model)}
    out["total_flops"] = sum(v["flops"] for k, v in out.items()
                             if isinstance(v, dict) and k != "out_proj_post_norm")
    if w.block:
        # The projections and the attention as one kernel: X and the weights
        # read once, O written once, Q/K/V never leave the chip.
        e = ELEM_BYTES[w.dtype]
        out["self_attention_fused"] = {
            "flops": out["project_qkv"]["flops"] + att_f,
            "bytes": e * (M * w.d_model + 3 * w.d_model * n + M * n)
                     + (4 * w.B if w.mask & 1 else 0)}
    return out
