"""The staircase inputs of the rescale parity tests do what those tests
need (CPU only): in every case, some row's running maximum grows by more
than 8 base-2 units at a tile after its first (the online softmax's
rescale branch runs) and some grows by 6 to 8 units (just under the
threshold: no rescale, exponentials up to 2^8)."""
import numpy as np
import pytest

import oracle
from rescale_cases import CASES, HUGE_CASES, climbs, growths, inputs
from workloads import generate


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.label())
def test_staircase_grows_the_running_max(case):
    q, k, v, lens = inputs(case, 7000)
    # one head of the first two batch rows is enough to show the growth
    sl = (slice(0, 2), slice(None), slice(0, 1))
    _, s = oracle.attention(q[sl], k[sl], v[sl], mask=case.mask,
                            kv_lens=None if lens is None else lens[:2],
                            return_s=True, window=case.window)
    g = growths(s)
    assert (g > 8).sum() >= 4, (case.label(), np.sort(g)[-5:])
    assert ((g > 6) & (g <= 8)).sum() >= 1, case.label()


def test_staircase_reaches_the_fused_kernel_exactly():
    """The block staircase puts the amplitudes and levels into channel 0 of
    every head's Q and K with no rounding, and nowhere else."""
    x = generate.normal((2, 100, 256), 7100, "bf16")
    ws = [generate.normal((256, 256), 7101 + i, "bf16", std=256 ** -0.5) for i in range(3)]
    x2, wq, wk, wv = generate.staircase_block(x, *ws, h=4)
    q, k, _ = oracle.project_qkv(x2, x2, wq, wk, wv, h=4)
    amps = np.array([generate.STAIRCASE_AMPS[i % 4] for i in range(100)])
    lv = generate.staircase_levels(100)
    assert np.array_equal(q[..., 0], np.broadcast_to(amps[None, :, None], q[..., 0].shape))
    assert np.array_equal(k[..., 0], np.broadcast_to(lv[None, :, None], k[..., 0].shape))
    x0 = x.clone()
    x0[:, :, :2] = 0
    q0, k0, _ = oracle.project_qkv(x0, x0, wq, wk, wv, h=4)
    assert np.array_equal(q0[..., 1:], q[..., 1:]) and np.array_equal(k0[..., 1:], k[..., 1:])


@pytest.mark.parametrize("case", HUGE_CASES, ids=lambda c: c.label())
def test_huge_staircase_climbs_past_the_fp32_range(case):
    """Some rows' maxima rise more than 127 base-2 units above their first
    tiles (2 under restricted attention), so a reference fixed there would
    give p = inf; other rows stay below that."""
    q, k, v, lens = inputs(case, 7400)
    sl = (slice(0, 2), slice(None), slice(0, 1))
    _, s = oracle.attention(q[sl], k[sl], v[sl], mask=case.mask,
                            kv_lens=None if lens is None else lens[:2],
                            return_s=True, window=case.window)
    c = climbs(s, 2 if case.window is not None else 1)
    assert (c > 130).sum() >= 4, (case.label(), np.sort(c)[-5:])
    assert (c < 120).sum() >= 4, case.label()
