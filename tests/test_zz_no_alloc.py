"""mha_decode_noalloc, the decode step for callers that cannot allocate,
through the C ABI: its output equals mha_decode's (the existing entry
point, with its own workspace) bit for bit, on calls in a row whose
second is smaller (the static scratch still holds the first call's
states), and inside a replayed HIP graph."""
import pytest
import torch

import oracle
import transformer_scaled_dot_fwd_amd as mha
from gpu_util import check, device, say
from workloads import generate

pytestmark = pytest.mark.gpu


def make(B, h, L, d, seed):
    q = generate.normal((B, 1, h, d), seed, "bf16")
    k = generate.normal((B, L, h, d), seed + 1, "bf16")
    v = generate.normal((B, L, h, d), seed + 2, "bf16")
    lens = generate.lengths(B, 0, L, seed + 3)
    return q, k, v, lens


@pytest.mark.parametrize("d", [64, 128])
def test_noalloc_equals_decode_on_calls_in_a_row(d):
    dev = device()
    # larger first, then smaller; then one with more heads than a workgroup
    # takes (two head groups) and one whose partial states fill most of the
    # 16 MiB scratch
    for n, (B, h, L) in enumerate(((16, 8, 4100), (3, 2, 700), (4, 40, 2100),
                                   (3900, 16, 16) if d == 64 else (2000, 16, 16))):
        say(f"case decode_noalloc d={d} B={B} h={h} L={L}")
        q, k, v, lens = (t.to(dev) for t in make(B, h, L, d, 8000 + 10 * n + d))
        assert mha.lib().mha_decode_workspace_bytes(B, h, L, d) <= 16 << 20
        ref = mha.mha_decode(q, k, v, lens)
        out = torch.empty_like(ref)
        mha.mha_decode_noalloc(q, k, v, lens, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (B, h, L, d)
        if n == 1:
            qc, kc, vc, lc = (t.cpu() for t in (q, k, v, lens))
            check(out, oracle.attention(qc, kc, vc, mask=1, kv_lens=lc), "bf16",
                  f"decode_noalloc d={d} B={B} h={h} L={L}")


def test_noalloc_refuses_more_than_its_scratch():
    dev = device()
    q, k, v, lens = (t.to(dev) for t in make(64, 16, 1, 64, 8100))
    need = mha.lib().mha_decode_workspace_bytes(64, 16, 65536, 64)
    assert need > 16 << 20
    # the shape is checked before anything touches the (tiny) cache tensors
    kk = k.expand(64, 65536, 16, 64)
    with pytest.raises(ValueError):      # the binding wants contiguous caches
        mha.mha_decode_noalloc(q, kk, kk, lens, torch.empty_like(q))
    rc = mha.lib().mha_decode_noalloc(1, 64, 16, 65536, 64, 64, q.data_ptr(), k.data_ptr(),
                                      v.data_ptr(), lens.data_ptr(), q.data_ptr(), None)
    assert rc == 4  # MHA_ERR_SCRATCH; nothing launched


def test_noalloc_in_a_replayed_graph():
    dev = device()
    q, k, v, lens = (t.to(dev) for t in make(8, 8, 3000, 64, 8200))
    ref = mha.mha_decode(q, k, v, lens)
    out = torch.zeros_like(ref)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mha.mha_decode_noalloc(q, k, v, lens, out)   # first call on this device, outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mha.mha_decode_noalloc(q, k, v, lens, out)
    for r in range(4):
        out.zero_()
        # eager work between replays, sharing the scratch
        q2, k2, v2, l2 = (t.to(dev) for t in make(2, 4, 900, 64, 8300 + r))
        mha.mha_decode_noalloc(q2, k2, v2, l2, torch.empty_like(q2))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
