"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each ``pin_*`` function checks the oracle against something the pages or the
mathematics fix: values printed on the pages (recomputed where the page is
wrong, see tests/golden/*.json), closed forms, invariants of softmax, special
cases that reduce to a library routine, and brute force on tiny inputs.  The
pytest tests run every pin on the real oracle; ``test_pins_catch_mutants``
compiles deliberately broken copies of oracle.c (a wrong scale, an
off-by-one mask, a dropped term, a swapped index ...) and checks that each
one fails at least one pin.
"""
import json
import math
import os
import tempfile

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE
from workloads import generate

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def sigma(x):
    return 1.0 / (1.0 + math.exp(-x))


def _as_blhd(m):
    """[L, d] -> [1, L, 1, d] fp64."""
    m = np.asarray(m, dtype=np.float64)
    return m.reshape(1, m.shape[0], 1, m.shape[1])


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------
# Pins.  Each takes an Oracle object and raises AssertionError on mismatch.
# --------------------------------------------------------------------------

def pin_worked_2x2_closed_form(O):
    """paperglide worked example, 2x2 scaled dot-product: with the 1/sqrt(2)
    scale applied the second weight row is (sigma(sqrt 2), sigma(-sqrt 2))
    (the printed 0.88/0.12 omit the scale; see the golden file)."""
    g = json.load(open(os.path.join(GOLDEN, "paperglide_scaled_dot_2x2.json")))
    Q, K, V = (np.array(g["inputs"][n], dtype=np.float64) for n in ("Q", "K", "V"))
    assert np.array_equal(Q @ K.T, np.array(g["printed"]["QKT"]))  # the reading of Q, K
    o, p, s = O.attention(_as_blhd(Q), _as_blhd(K), _as_blhd(V), return_p=True, return_s=True)
    r = math.sqrt(2.0)
    exp_s = np.array(g["printed"]["QKT"], dtype=np.float64) / r
    np.testing.assert_allclose(s[0, 0], exp_s, rtol=0, atol=1e-15)
    exp_p = np.array([[0.5, 0.5], [sigma(r), sigma(-r)]])
    np.testing.assert_allclose(p[0, 0], exp_p, rtol=0, atol=1e-15)
    exp_o = 5.0 * exp_p
    np.testing.assert_allclose(o[0, :, 0, :], exp_o, rtol=0, atol=1e-14)


def pin_worked_2x2_printed_digits(O):
    """The page's printed weights and outputs (2 decimals) are reproduced by
    the variant whose scale is cancelled, Q = sqrt(2) I."""
    g = json.load(open(os.path.join(GOLDEN, "paperglide_scaled_dot_2x2.json")))
    pr = g["printed"]
    Q = math.sqrt(2.0) * np.array(g["inputs"]["Q"], dtype=np.float64)
    K = np.array(g["inputs"]["K"], dtype=np.float64)
    V = np.array(g["inputs"]["V"], dtype=np.float64)
    o, p = O.attention(_as_blhd(Q), _as_blhd(K), _as_blhd(V), return_p=True)
    dec = pr["decimals"]
    assert np.array_equal(np.round(p[0, 0], dec), np.array(pr["weights"]))
    assert np.array_equal(np.round(o[0, :, 0, :], 1), np.array(pr["output"]))


def pin_two_head_toy(O):
    """paperglide two-head toy: column-selecting W_i, identity W^O.
    Q_i are the printed ones; the output has the printed concat's mirror
    structure and equals the recomputed [[a,b,b,a],[b,a,a,b]]."""
    g = json.load(open(os.path.join(GOLDEN, "paperglide_two_head_toy.json")))
    X = np.array(g["derived_inputs"]["X"], dtype=np.float64)
    sel = g["printed"]["head_column_selection"]
    W = np.zeros((4, 4))
    for head, cols in sel.items():
        for c_out, c_in in enumerate(cols):
            W[c_in, (int(head) - 1) * 2 + c_out] = 1.0
    x = X.reshape(1, 2, 4)
    q, k, v = O.project_qkv(x, x, W, W, W, h=2)
    assert np.array_equal(q[0, :, 0, :], np.array(g["printed"]["Q1"]))
    assert np.array_equal(q[0, :, 1, :], np.array(g["printed"]["Q2"]))
    y = O.mha_block(x, x, W, W, W, np.eye(4), h=2)[0]
    a, b = sigma(1 / math.sqrt(2)), sigma(-1 / math.sqrt(2))
    np.testing.assert_allclose(y, [[a, b, b, a], [b, a, a, b]], rtol=0, atol=1e-15)
    printed = np.array(g["printed"]["concat"])
    for M in (y, printed):  # the mirror structure of head_1 || head_2
        assert np.array_equal(M[:, 0], M[:, 3]) and np.array_equal(M[:, 1], M[:, 2])


def pin_head_owns_column_block(O):
    """Head t is column block t of X W: zero logits in block 0 give head 1
    uniform weights (the mean of its V block); block 1 built to pick key 2
    gives head 2 that key's V block."""
    L, dm, h, d = 3, 4, 2, 2
    X = np.eye(3, 4)
    Wq = np.zeros((dm, h * d))
    Wq[:, 2] = 40.0                        # head 2 query = 40 * e_0 in its block
    Wk = np.zeros((dm, h * d))
    Wk[2, 2] = 1.0                         # head 2 key of position 2 = e_0
    Wk[0, 0] = 1.0                         # head 1 keys nonzero, queries zero
    Wv = np.arange(dm * h * d, dtype=np.float64).reshape(dm, h * d) / 7.0
    x = X.reshape(1, L, dm)
    y = O.mha_block(x, x, Wq, Wk, Wv, np.eye(h * d), h=h)[0]
    Vf = X @ Wv
    np.testing.assert_allclose(y[:, 0:2], np.tile(Vf[:, 0:2].mean(axis=0), (L, 1)),
                               rtol=0, atol=1e-14)
    # weight on key 2 is 1/(1 + 2 e^{-40/sqrt 2}): Vf[2] up to ~1e-12
    np.testing.assert_allclose(y[:, 2:4], np.tile(Vf[2, 2:4], (L, 1)), rtol=0, atol=1e-10)


def pin_two_key_closed_form(O):
    """softmax([x, y]) = [sigma(x - y), sigma(y - x)] (d_k = 1, scale 1)."""
    rng = np.random.default_rng(11)
    for _ in range(50):
        x, y = rng.uniform(-30, 30, size=2)
        q = np.ones((1, 1, 1, 1))
        k = np.array([x, y]).reshape(1, 2, 1, 1)
        v = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 2, 1, 2)
        o, p = O.attention(q, k, v, return_p=True)
        np.testing.assert_allclose(p[0, 0, 0], [sigma(x - y), sigma(y - x)], rtol=1e-13,
                                   atol=1e-300)
        np.testing.assert_allclose(o[0, 0, 0], [sigma(x - y), sigma(y - x)], rtol=1e-13,
                                   atol=1e-300)


def _legal(mask, lens, Lq, Lk, b, window=None):
    L = Lk
    if mask & MASK_KEY_PADDING:
        L = min(max(int(lens[b]), 0), Lk)
    leg = np.zeros((Lq, Lk), dtype=bool)
    for i in range(Lq):
        for j in range(Lk):
            leg[i, j] = (j < L) and (not (mask & MASK_CAUSAL) or j <= i) and \
                (window is None or abs(i - j) <= window)
    return leg


def pin_convex_combination(O):
    """Weights of a row sum to 1; masked weights are exactly 0; every output
    element lies between the min and max of the legal V rows."""
    rng = np.random.default_rng(5)
    B, h, L, d = 3, 2, 19, 5
    q, k, v = (_rand(rng, B, L, h, d) for _ in range(3))
    lens = np.array([19, 7, 1], dtype=np.int32)
    for mask in (MASK_NONE, MASK_KEY_PADDING, MASK_CAUSAL, MASK_CAUSAL | MASK_KEY_PADDING):
        o, p = O.attention(q, k, v, mask=mask, kv_lens=lens, return_p=True)
        for b in range(B):
            leg = _legal(mask, lens, L, L, b)
            for t in range(h):
                P = p[b, t]
                assert np.all(P[~leg] == 0.0)
                assert np.all(P[leg] > 0.0)
                np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
                for i in range(L):
                    vv = v[b, leg[i], t, :]
                    assert np.all(o[b, i, t] <= vv.max(axis=0) + 1e-14)
                    assert np.all(o[b, i, t] >= vv.min(axis=0) - 1e-14)


def pin_masked_garbage_invariance(O):
    """Illegal keys contribute nothing whatever K and V hold there: NaN, Inf
    or huge values in padded rows leave O bit-identical; editing keys after
    position t leaves causal rows <= t bit-identical."""
    rng = np.random.default_rng(6)
    B, h, L, d = 2, 3, 21, 4
    q, k, v = (_rand(rng, B, L, h, d) for _ in range(3))
    lens = np.array([9, 14], dtype=np.int32)
    base = O.attention(q, k, v, mask=MASK_KEY_PADDING, kv_lens=lens)
    for junk in (np.nan, np.inf, -np.inf, 1e300):
        k2, v2 = k.copy(), v.copy()
        for b in range(B):
            k2[b, lens[b]:] = junk
            v2[b, lens[b]:] = junk
        o2 = O.attention(q, k2, v2, mask=MASK_KEY_PADDING, kv_lens=lens)
        assert np.array_equal(o2, base)
    basec = O.attention(q, k, v, mask=MASK_CAUSAL)
    for t in (0, 5, 20):
        k2, v2 = k.copy(), v.copy()
        k2[:, t + 1:] = _rand(rng, B, L - t - 1, h, d) * 100
        v2[:, t + 1:] = np.nan
        o2 = O.attention(q, k2, v2, mask=MASK_CAUSAL)
        assert np.array_equal(o2[:, :t + 1], basec[:, :t + 1])


def pin_shift_invariance(O):
    """Adding u to every key shifts each logit row by q_i.u/sqrt(d_k); the
    output is unchanged and stays finite for shifts of 1e3-1e4."""
    rng = np.random.default_rng(7)
    B, h, L, d = 2, 2, 17, 8
    q, k, v = (_rand(rng, B, L, h, d) for _ in range(3))
    lens = np.array([17, 6], dtype=np.int32)
    for mask in (MASK_NONE, MASK_CAUSAL | MASK_KEY_PADDING):
        o = O.attention(q, k, v, mask=mask, kv_lens=lens)
        for scale in (10.0, 1e3, 1e4):
            u = rng.standard_normal((1, 1, h, d)) * scale
            o2 = O.attention(q, k + u, v, mask=mask, kv_lens=lens)
            assert np.all(np.isfinite(o2))
            np.testing.assert_allclose(o2, o, rtol=0, atol=1e-8)


def pin_uniform_weights(O):
    """K = 0 makes every logit equal: O_i is the mean of the legal V rows
    (causal: of V_0..V_i)."""
    rng = np.random.default_rng(8)
    B, h, L, d = 2, 2, 13, 3
    q, v = _rand(rng, B, L, h, d), _rand(rng, B, L, h, d)
    k = np.zeros((B, L, h, d))
    lens = np.array([13, 4], dtype=np.int32)
    for mask in (MASK_NONE, MASK_KEY_PADDING, MASK_CAUSAL, MASK_CAUSAL | MASK_KEY_PADDING):
        o = O.attention(q, k, v, mask=mask, kv_lens=lens)
        for b in range(B):
            leg = _legal(mask, lens, L, L, b)
            for i in range(L):
                np.testing.assert_allclose(o[b, i], v[b, leg[i]].mean(axis=0), rtol=0,
                                           atol=1e-14)


def pin_single_key_and_empty(O):
    """One legal key gives that key's V row exactly; no legal key gives 0;
    lengths outside [0, Lk] are clamped."""
    rng = np.random.default_rng(9)
    B, h, L, d = 4, 2, 9, 6
    q, k, v = (_rand(rng, B, L, h, d) for _ in range(3))
    lens = np.array([1, 0, -3, 50], dtype=np.int32)
    o = O.attention(q, k, v, mask=MASK_KEY_PADDING, kv_lens=lens)
    assert np.array_equal(o[0], np.broadcast_to(v[0, 0], (L, h, d)))
    assert np.array_equal(o[1], np.zeros((L, h, d)))
    assert np.array_equal(o[2], np.zeros((L, h, d)))
    full = O.attention(q, k, v)
    assert np.array_equal(o[3], full[3])
    oc = O.attention(q, k, v, mask=MASK_CAUSAL)
    assert np.array_equal(oc[:, 0], v[:, 0])      # causal row 0 sees only key 0


def pin_permutation_equivariance(O):
    """Permuting keys together with values leaves O unchanged; permuting
    queries permutes the rows of O."""
    rng = np.random.default_rng(10)
    B, h, Lq, Lk, d = 2, 2, 7, 11, 4
    q = _rand(rng, B, Lq, h, d)
    k, v = _rand(rng, B, Lk, h, d), _rand(rng, B, Lk, h, d)
    o = O.attention(q, k, v)
    perm = rng.permutation(Lk)
    np.testing.assert_allclose(O.attention(q, k[:, perm], v[:, perm]), o, rtol=0, atol=1e-14)
    qp = rng.permutation(Lq)
    assert np.array_equal(O.attention(q[:, qp], k, v), o[:, qp])


def pin_scale_variance(O):
    """With q, k components i.i.d. N(0, 1) the dot product has variance d_k
    and the scaled logit variance 1 (Deep-reading page section 04, on the
    1/sqrt(d_k) factor), checked on the seeded generator's bf16 draws."""
    d = 64
    q = generate.normal((1, 256, 1, d), 424242, "bf16")
    k = generate.normal((1, 256, 1, d), 424243, "bf16")
    v = generate.normal((1, 256, 1, d), 424244, "bf16")
    _, s = O.attention(q, k, v, return_s=True)
    s = s.ravel()
    assert abs(s.mean()) < 0.02
    assert abs(s.var() - 1.0) < 0.05
    assert abs((s * math.sqrt(d)).var() / d - 1.0) < 0.05


def pin_projection_identity(O):
    """h = 1 and W = I: MultiHead reduces to Attention (X W = X exactly);
    the matmul equals numpy's on random shapes."""
    rng = np.random.default_rng(12)
    B, L, dm = 2, 6, 5
    x = _rand(rng, B, L, dm)
    y = O.mha_block(x, x, np.eye(dm), np.eye(dm), np.eye(dm), np.eye(dm), h=1)
    xa = x.reshape(B, L, 1, dm)
    assert np.array_equal(y, O.attention(xa, xa, xa).reshape(B, L, dm))
    for (M, K, N) in ((1, 1, 1), (7, 13, 5), (33, 64, 17)):
        a, w = _rand(rng, M, K), _rand(rng, K, N)
        np.testing.assert_allclose(O.matmul(a, w), a @ w, rtol=1e-13, atol=1e-13)


def _torch_reference(q, k, v, mask, lens):
    """softmax(q k^T / sqrt(d) + M) v with torch fp64 ops, M = -inf at
    illegal pairs; rows with no legal key are returned as NaN (excluded)."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a)).permute(0, 2, 1, 3) for a in (q, k, v))
    B, h, Lq, d = q.shape
    Lk = k.shape[2]
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) / math.sqrt(d)
    M = torch.zeros(B, 1, Lq, Lk, dtype=torch.float64)
    for b in range(B):
        M[b, 0][~torch.from_numpy(_legal(mask, lens, Lq, Lk, b))] = -math.inf
    p = torch.softmax(s + M, dim=-1)
    return torch.matmul(p, v).permute(0, 2, 1, 3).numpy()


def pin_torch_cross_check(O):
    """Library cross-check: torch.softmax / torch.matmul in fp64."""
    rng = np.random.default_rng(13)
    for (B, h, Lq, Lk, d) in ((2, 3, 10, 10, 8), (1, 2, 5, 23, 4), (3, 1, 31, 31, 16)):
        q = _rand(rng, B, Lq, h, d)
        k, v = _rand(rng, B, Lk, h, d), _rand(rng, B, Lk, h, d)
        lens = rng.integers(1, Lk + 1, size=B).astype(np.int32)
        masks = [MASK_NONE, MASK_KEY_PADDING]
        if Lq == Lk:
            masks += [MASK_CAUSAL, MASK_CAUSAL | MASK_KEY_PADDING]
        for mask in masks:
            o = O.attention(q, k, v, mask=mask, kv_lens=lens)
            ref = _torch_reference(q, k, v, mask, lens)
            np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def _brute(q, k, v, mask, lens, window=None):
    """Pure-Python loops, written from the attention equation."""
    B, Lq, h, d = q.shape
    Lk, dv = k.shape[1], v.shape[3]
    out = np.zeros((B, Lq, h, dv))
    for b in range(B):
        leg = _legal(mask, lens, Lq, Lk, b, window)
        for t in range(h):
            for i in range(Lq):
                js = [j for j in range(Lk) if leg[i, j]]
                if not js:
                    continue
                sc = [sum(q[b, i, t, c] * k[b, j, t, c] for c in range(d)) / math.sqrt(d)
                      for j in js]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                tot = sum(w)
                for e in range(dv):
                    out[b, i, t, e] = sum(w[n] / tot * v[b, js[n], t, e] for n in range(len(js)))
    return out


def pin_brute_force_tiny(O):
    rng = np.random.default_rng(14)
    for (B, h, Lq, Lk, d) in ((1, 1, 1, 1, 1), (2, 2, 5, 5, 2), (1, 3, 4, 9, 4), (2, 1, 8, 8, 8)):
        q = _rand(rng, B, Lq, h, d)
        k, v = _rand(rng, B, Lk, h, d), _rand(rng, B, Lk, h, d)
        lens = rng.integers(0, Lk + 1, size=B).astype(np.int32)
        masks = [MASK_NONE, MASK_KEY_PADDING] + ([MASK_CAUSAL, 3] if Lq == Lk else [])
        for mask in masks:
            np.testing.assert_allclose(O.attention(q, k, v, mask=mask, kv_lens=lens),
                                       _brute(q, k, v, mask, lens), rtol=1e-12, atol=1e-12)


def pin_rows_match_full(O):
    """attention_rows evaluates the same rows as attention."""
    rng = np.random.default_rng(15)
    B, h, L, d = 2, 3, 12, 4
    q, k, v = (_rand(rng, B, L, h, d) for _ in range(3))
    lens = np.array([12, 5], dtype=np.int32)
    full = O.attention(q, k, v, mask=3, kv_lens=lens)
    rows = np.array([[b, t, i] for b in range(B) for t in range(h) for i in range(L)])
    sel = O.attention_rows(q, k, v, rows, mask=3, kv_lens=lens)
    for n, (b, t, i) in enumerate(rows):
        assert np.array_equal(sel[n], full[b, i, t])


def pin_window_is_attention_over_the_neighbourhood(O):
    """Restricted self-attention (Deep-reading page section 05): each output
    row equals ordinary attention of that query over the keys within w
    positions of it -- the neighbourhood sliced out of K and V, with the
    padding length moved to the slice and causal cutting it at the query."""
    rng = np.random.default_rng(21)
    B, h, L, d = 2, 2, 17, 4
    q, k, v = (_rand(rng, B, L, h, d) for _ in range(3))
    lens = np.array([17, 9], dtype=np.int32)
    for w in (0, 1, 3, 7):
        for mask in (MASK_NONE, MASK_KEY_PADDING, MASK_CAUSAL, 3):
            o = O.attention(q, k, v, mask=mask, kv_lens=lens, window=w)
            for b in range(B):
                for i in range(L):
                    lo, hi = max(0, i - w), min(L, i + w + 1)
                    if mask & MASK_CAUSAL:
                        hi = min(hi, i + 1)
                    n = hi - lo
                    if mask & MASK_KEY_PADDING:
                        n = min(max(int(lens[b]) - lo, 0), hi - lo)
                    if n == 0:
                        assert np.all(o[b, i] == 0.0)
                        continue
                    ref = O.attention(q[b:b + 1, i:i + 1], k[b:b + 1, lo:lo + n],
                                      v[b:b + 1, lo:lo + n])
                    np.testing.assert_allclose(o[b, i], ref[0, 0], rtol=1e-13, atol=1e-13)


def pin_window_limits(O):
    """A window covering every position is ordinary attention (bit for
    bit); a window of 0 leaves each query its own position: O_i = V_i.  The
    legal pairs of a row number min(i, w) + min(L - 1 - i, w) + 1, so the
    work is O(r n d) with r = 2w + 1 (Deep-reading page section 05)."""
    rng = np.random.default_rng(22)
    B, h, L, d = 2, 3, 13, 4
    q, k, v = (_rand(rng, B, L, h, d) for _ in range(3))
    for mask in (MASK_NONE, MASK_CAUSAL):
        assert np.array_equal(O.attention(q, k, v, mask=mask, window=L - 1),
                              O.attention(q, k, v, mask=mask))
    assert np.array_equal(O.attention(q, k, v, window=0), v)
    for w in (1, 4):
        _, p = O.attention(q, k, v, window=w, return_p=True)
        for i in range(L):
            assert np.all((p[:, :, i] != 0).sum(axis=-1) == min(i, w) + min(L - 1 - i, w) + 1)


def pin_window_brute_force(O):
    rng = np.random.default_rng(23)
    for (B, h, L, d) in ((1, 1, 6, 2), (2, 2, 9, 4)):
        q, k, v = (_rand(rng, B, L, h, d) for _ in range(3))
        lens = rng.integers(0, L + 1, size=B).astype(np.int32)
        for w in (0, 2, 5):
            for mask in range(4):
                np.testing.assert_allclose(O.attention(q, k, v, mask=mask, kv_lens=lens, window=w),
                                           _brute(q, k, v, mask, lens, w), rtol=1e-12, atol=1e-12)


def pin_layer_norm_moments_and_invariance(O):
    """With unit gain and zero bias (eps = 0) every output row has mean 0
    and mean square 1; a positive scale and a shift of a row leave it
    unchanged; gain and bias act per feature afterwards."""
    rng = np.random.default_rng(31)
    z = _rand(rng, 5, 12)
    one, zero = np.ones(12), np.zeros(12)
    u = O.layer_norm(z, one, zero, eps=0.0)
    np.testing.assert_allclose(u.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose((u * u).mean(axis=1), 1.0, atol=1e-13)
    np.testing.assert_allclose(O.layer_norm(3.5 * z - 2.0, one, zero, eps=0.0), u, atol=1e-13)
    g, b = _rand(rng, 12), _rand(rng, 12)
    np.testing.assert_allclose(O.layer_norm(z, g, b, eps=0.0), g * u + b, atol=1e-13)


def pin_layer_norm_closed_forms(O):
    """Two features [a, c]: mean (a+c)/2, variance ((a-c)/2)^2, so the
    outputs are +-(a-c)/2 / sqrt(((a-c)/2)^2 + eps).  A constant row has
    variance 0 and gives the bias exactly."""
    for a, c, eps in ((1.0, -3.0, 1e-6), (0.25, 0.5, 0.5), (7.0, 7.5, 2.0)):
        h = (a - c) / 2.0
        r = h / math.sqrt(h * h + eps)
        out = O.layer_norm(np.array([[a, c]]), np.ones(2), np.zeros(2), eps=eps)
        np.testing.assert_allclose(out, [[r, -r]], rtol=0, atol=1e-15)
    beta = np.array([0.5, -1.25, 3.0])
    out = O.layer_norm(np.full((2, 3), 4.0), np.array([2.0, 3.0, 4.0]), beta, eps=1e-6)
    assert np.array_equal(out, np.stack([beta, beta]))


def pin_layer_norm_torch_cross_check(O):
    """Library cross-check: torch.nn.functional.layer_norm in fp64."""
    rng = np.random.default_rng(32)
    for (M, N, eps) in ((4, 16, 1e-6), (3, 512, 1e-5), (2, 7, 0.5)):
        z, g, b = _rand(rng, M, N), _rand(rng, N), _rand(rng, N)
        ref = torch.nn.functional.layer_norm(torch.from_numpy(z), (N,), torch.from_numpy(g),
                                             torch.from_numpy(b), eps).numpy()
        np.testing.assert_allclose(O.layer_norm(z, g, b, eps=eps), ref, rtol=1e-12, atol=1e-12)


def pin_post_norm_special_cases(O):
    """LayerNorm(x + Concat(heads) W^O): with W^O = 0 it is LayerNorm(x);
    with x = 0 it is LayerNorm of the projection alone; with W^O = I and
    heads = -x it is the bias (a zero row normalises to 0)."""
    rng = np.random.default_rng(33)
    B, L, h, d = 2, 3, 2, 4
    dm = h * d
    o, x = _rand(rng, B, L, h, d), _rand(rng, B, L, dm)
    g, b = _rand(rng, dm), _rand(rng, dm)
    np.testing.assert_allclose(O.out_proj_post_norm(o, np.zeros((dm, dm)), x, g, b),
                               O.layer_norm(x, g, b), atol=1e-13)
    w = _rand(rng, dm, dm)
    y = np.einsum("blk,kn->bln", o.reshape(B, L, dm), w)
    np.testing.assert_allclose(O.out_proj_post_norm(o, w, np.zeros((B, L, dm)), g, b),
                               O.layer_norm(y, g, b), atol=1e-12)
    out = O.out_proj_post_norm(-x.reshape(B, L, h, d), np.eye(dm), x, g, b)
    assert np.array_equal(out, np.broadcast_to(b, out.shape))


PINS = [pin_worked_2x2_closed_form, pin_worked_2x2_printed_digits, pin_two_head_toy,
        pin_head_owns_column_block, pin_two_key_closed_form, pin_convex_combination,
        pin_masked_garbage_invariance, pin_shift_invariance, pin_uniform_weights,
        pin_single_key_and_empty, pin_permutation_equivariance, pin_scale_variance,
        pin_projection_identity, pin_torch_cross_check, pin_brute_force_tiny,
        pin_rows_match_full, pin_window_is_attention_over_the_neighbourhood,
        pin_window_limits, pin_window_brute_force, pin_layer_norm_moments_and_invariance,
        pin_layer_norm_closed_forms, pin_layer_norm_torch_cross_check,
        pin_post_norm_special_cases]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.default())


@settings(max_examples=40, deadline=None)
@given(B=st.integers(1, 3), h=st.integers(1, 3), Lq=st.integers(1, 12),
       Lk=st.integers(1, 12), d=st.sampled_from([1, 2, 4, 8]), mask=st.integers(0, 3),
       seed=st.integers(0, 2**31 - 1))
def test_brute_force_hypothesis(B, h, Lq, Lk, d, mask, seed):
    if mask & MASK_CAUSAL:
        Lk = Lq
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Lq, h, d))
    k, v = rng.standard_normal((B, Lk, h, d)), rng.standard_normal((B, Lk, h, d))
    lens = rng.integers(-1, Lk + 2, size=B).astype(np.int32)
    np.testing.assert_allclose(oracle.attention(q, k, v, mask=mask, kv_lens=lens),
                               _brute(q, k, v, mask, lens), rtol=1e-12, atol=1e-12)


def test_rejects_bad_arguments():
    q = np.zeros((1, 4, 1, 2))
    k = np.zeros((1, 5, 1, 2))
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, window=2)                  # a window needs Lq == Lk
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, mask=MASK_CAUSAL)          # causal needs Lq == Lk
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, mask=MASK_KEY_PADDING)     # lengths missing


# --------------------------------------------------------------------------
# Mutation check: plausible mistakes planted in a copy of oracle.c, on the
# CPU, must each fail at least one pin.
# --------------------------------------------------------------------------

MUTANTS = {
    "scale_1_over_dk": ("1.0 / sqrt((double)d_k)", "1.0 / (double)d_k"),
    "no_scale": ("logits[j] = dot * scale;", "logits[j] = dot;"),
    "causal_excludes_diagonal": ("(mask_flags & ORACLE_MASK_CAUSAL) && j > i",
                                 "(mask_flags & ORACLE_MASK_CAUSAL) && j >= i"),
    "padding_off_by_one": ("(mask_flags & ORACLE_MASK_KEY_PADDING) && j >= len_b",
                           "(mask_flags & ORACLE_MASK_KEY_PADDING) && j > len_b"),
    "no_max_shift": ("exp(logits[j] - mx)", "exp(logits[j])"),
    "wrong_head_for_q": ("const double* qi = q + ((b * Lq + i) * h + t) * d_k;",
                         "const double* qi = q + ((b * Lq + i) * h + (h - 1 - t)) * d_k;"),
    "reversed_weights": ("o_row[e] += weights[j] * vj[e];",
                         "o_row[e] += weights[Lk - 1 - j] * vj[e];"),
    "dropped_last_d_term": ("for (long c = 0; c < d_k; ++c) dot += qi[c] * kj[c];",
                            "for (long c = 0; c + 1 < d_k; ++c) dot += qi[c] * kj[c];"),
    "matmul_dropped_term": ("for (long kk = 0; kk < K; ++kk) {",
                            "for (long kk = 0; kk + 1 < K; ++kk) {"),
    "padding_ignored": ("if ((mask_flags & ORACLE_MASK_KEY_PADDING) && j >= len_b) return 0;", ""),
    "window_off_by_one": ("j > i + window)", "j >= i + window)"),
    "window_one_sided": ("(j < i - window || j > i + window)", "(j > i + window)"),
    "ln_unbiased_variance": ("var /= (double)N;", "var /= (double)(N - 1);"),
    "ln_eps_outside_root": ("1.0 / sqrt(var + eps)", "1.0 / (sqrt(var) + eps)"),
    "ln_no_bias": (" * inv + beta[n];", " * inv;"),
    "ln_no_centering": ("var += (zm[n] - mu) * (zm[n] - mu);", "var += zm[n] * zm[n];"),
    "empty_row_not_zero": ("for (long e = 0; e < d_v; ++e) o_row[e] = 0.0;\n        if (p_row)",
                           "for (long e = 0; e < d_v; ++e) o_row[e] = 1.0;\n        if (p_row)"),
}


def test_pins_catch_mutants():
    src = open(oracle.SOURCE).read()
    escaped = {}
    with tempfile.TemporaryDirectory() as tmp:
        for name, (old, new) in MUTANTS.items():
            assert src.count(old) >= 1, f"mutation site for {name} not found"
            mutated = src.replace(old, new, 1)
            c_path = os.path.join(tmp, f"{name}.c")
            open(c_path, "w").write(mutated)
            so = oracle.compile_source(c_path, os.path.join(tmp, f"{name}.so"), quiet=True)
            mutant = oracle.Oracle(so)
            caught = []
            for pin in PINS:
                try:
                    pin(mutant)
                except (AssertionError, ValueError, FloatingPointError):
                    caught.append(pin.__name__)
            if not caught:
                escaped[name] = "no pin failed"
    assert not escaped, escaped
