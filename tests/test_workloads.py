"""Seeded generators, workload registry and FLOP/byte accounting (CPU)."""
import numpy as np
import torch

from workloads import accounting, configs, generate


def test_generator_is_deterministic_and_rne():
    a = generate.normal((3, 5, 7), 123, "bf16")
    b = generate.normal((3, 5, 7), 123, "bf16")
    assert torch.equal(a, b)
    f = generate.normal((3, 5, 7), 123, "f32")
    assert torch.equal(f.to(torch.bfloat16), a)           # bf16 = RNE of the fp32 draw
    assert not torch.equal(generate.normal((3, 5, 7), 124, "bf16"), a)


def test_generator_statistics():
    x = generate.normal((200000,), 7, "f32").double()
    assert abs(x.mean().item()) < 0.01 and abs(x.std().item() - 1) < 0.01
    w = generate.normal((512, 512), 8, "bf16", std=512 ** -0.5).double()
    assert abs(w.var().item() * 512 - 1) < 0.02              # N(0, 1/512): variance 1/512


def test_lengths_range():
    lens = generate.lengths(10000, 32, 128, 5)
    assert lens.dtype == torch.int32
    assert lens.min().item() == 32 and lens.max().item() == 128


def brute_pairs(B, h, Lq, Lk, mask, lens):
    n = 0
    for b in range(B):
        L = min(max(int(lens[b]), 0), Lk) if mask & 1 else Lk
        for i in range(Lq):
            for j in range(Lk):
                if j < L and (not (mask & 2) or j <= i):
                    n += 1
    return n * h


def test_pair_count_matches_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(30):
        B, h = rng.integers(1, 4), rng.integers(1, 3)
        Lq = rng.integers(1, 20)
        mask = int(rng.integers(0, 4))
        Lk = Lq if mask & 2 else rng.integers(1, 20)
        lens = rng.integers(-2, Lk + 3, size=B)
        assert accounting.legal_pairs(B, h, Lq, Lk, mask, lens) == brute_pairs(B, h, Lq, Lk,
                                                                                 mask, lens)


def test_config_shapes():
    for name in ("c1", "c2", "c3", "c4", "c5"):
        w = configs.get(name)
        inp = configs.make_inputs(w) if name != "c5" else None
        if inp is None:
            continue
        if w.block:
            assert inp["x"].shape == (w.B, w.Lq, w.d_model)
            assert inp["w_o"].shape == (w.h * w.d, w.d_model)
        else:
            assert inp["q"].shape == (w.B, w.Lq, w.h, w.d)
            assert inp["k"].shape == (w.B, w.Lk, w.h, w.d)
        if w.mask & 1:
            lo, hi = w.lens
            assert inp["kv_lens"].min() >= lo and inp["kv_lens"].max() <= hi
    sw = configs.sweep()
    assert len(sw) == 12 and all(w.B * w.Lq == 24576 for w in sw)


def test_long_causal_flops():
    w = configs.get("c5")
    # 4 * d * B * h * L (L + 1) / 2
    assert accounting.attention_flops(w.B, w.h, w.Lq, w.Lk, w.d, w.mask) == \
        4 * 64 * 4 * 16 * 4096 * 4097 // 2


def brute_window_pairs(B, h, Lq, Lk, mask, lens, w):
    n = 0
    for b in range(B):
        L = min(max(int(lens[b]), 0), Lk) if mask & 1 else Lk
        for i in range(Lq):
            for j in range(L):
                if abs(i - j) <= w and (not (mask & 2) or j <= i):
                    n += 1
    return n * h


def test_window_pair_count_matches_brute_force():
    """Restricted attention (Deep-reading page section 05): only |i - j| <= w
    is legal, on top of the padding and causal masks."""
    rng = np.random.default_rng(5)
    for _ in range(30):
        B, h = int(rng.integers(1, 4)), int(rng.integers(1, 3))
        Lq = int(rng.integers(1, 24))
        mask = int(rng.integers(0, 4))
        Lk = Lq if mask & 2 else int(rng.integers(1, 24))
        lens = rng.integers(-2, Lk + 3, size=B)
        w = int(rng.integers(0, 30))
        assert accounting.legal_pairs(B, h, Lq, Lk, mask, lens, w) == \
            brute_window_pairs(B, h, Lq, Lk, mask, lens, w)


def test_window_rows_are_under_the_ridge_point():
    """The band's closed forms at L = 4096, w = 256: causal rows see
    min(i, w) + 1 keys, unrestricted rows min(i, w) + min(L - 1 - i, w) + 1.
    Q, K, V and O cross HBM once (8 L d bytes per batch row and head in
    bf16), so the FLOP per byte is 124.48 causal and 248.47 without a mask,
    both under 2.5e15 / 8e12 = 312.5."""
    L, w = 4096, 256
    causal = w * (w + 1) // 2 + (L - w) * (w + 1)
    full = 2 * (w * (w - 1) // 2 + (L - w) * w) + L
    for wl in configs.windows():
        per_head = wl.B * wl.h
        pairs = accounting.legal_pairs(wl.B, wl.h, wl.Lq, wl.Lk, wl.mask, None, wl.window)
        expect = causal if wl.mask & 2 else full
        assert pairs == expect * per_head
        flops = accounting.attention_flops(wl.B, wl.h, wl.Lq, wl.Lk, wl.d, wl.mask, None,
                                           wl.window)
        nbytes = accounting.attention_bytes(wl.B, wl.h, wl.Lq, wl.Lk, wl.d, wl.mask)
        assert nbytes == 8 * L * 64 * per_head
        intensity = flops / nbytes
        assert intensity < 2.5e15 / 8e12
        assert abs(intensity - (124.48 if wl.mask & 2 else 248.47)) < 0.01
