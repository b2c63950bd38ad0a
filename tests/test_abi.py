"""The C ABI of libmha.so, checked without a GPU.

The library must load and export every function include/mha.h declares, and
its argument validation -- which runs before any HIP call -- must reject bad
calls with the documented status codes.  Nothing here launches a kernel.
"""
import ctypes
import os
import re

import pytest

import transformer_scaled_dot_fwd_amd as mha

OK, INVALID, UNSUPPORTED, LAUNCH, SCRATCH = 0, 1, 2, 3, 4
BF16, F32 = 1, 0
FAKE = 0x1000  # a 16-byte aligned non-NULL address; never dereferenced here


def declared_functions():
    text = open(mha.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mha_\w+)\s*\(", text, flags=re.M)


# The sanitizer leg (tests/test_sanitized_host.py) reruns this module on a
# host-only ASan/UBSan build of the same sources, named by this variable.
CHECKED = os.environ.get("MHA_HOST_CHECKED_LIBRARY")


@pytest.fixture(scope="module")
def L():
    if CHECKED:
        return mha.declare(ctypes.CDLL(CHECKED))
    if not os.path.exists(mha.LIBRARY):
        from transformer_scaled_dot_fwd_amd import build
        build.build()
    return mha.lib()


def test_header_declares_the_boundary():
    assert set(declared_functions()) == {"mha_forward", "mha_project_qkv", "mha_out_proj",
                                         "mha_self_attention_fused", "mha_forward_windowed",
                                         "mha_decode", "mha_decode_workspace_bytes",
                                         "mha_decode_noalloc",
                                         "mha_out_proj_post_norm", "mha_status_string"}


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for s in (OK, INVALID, UNSUPPORTED, LAUNCH, SCRATCH, 99):
        assert L.mha_status_string(s)
    assert L.mha_status_string(OK) == b"ok"


def fwd(L, dt=BF16, B=2, h=2, Lq=8, Lk=8, dk=64, dv=64, q=FAKE, k=FAKE, v=FAKE, mask=0,
        lens=None, o=FAKE):
    return L.mha_forward(dt, B, h, Lq, Lk, dk, dv, q, k, v, mask, lens, o, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(dt=7), INVALID),
    (dict(B=-1), INVALID),
    (dict(h=0), INVALID),
    (dict(Lq=-2), INVALID),
    (dict(dk=0), INVALID),
    (dict(mask=4), INVALID),
    (dict(mask=2, Lq=8, Lk=9), INVALID),          # causal needs Lq == Lk
    (dict(mask=1, lens=None), INVALID),           # key padding needs lengths
    (dict(q=None), INVALID),
    (dict(o=None), INVALID),
    (dict(k=None), INVALID),
    (dict(q=FAKE + 8), INVALID),                  # misaligned
    (dict(dk=64, dv=32), UNSUPPORTED),
    (dict(dk=48, dv=48), UNSUPPORTED),            # bf16 is built for d in {16, 32, 64, 128}
    (dict(dk=256, dv=256), UNSUPPORTED),
    (dict(dt=F32, dk=24, dv=24), UNSUPPORTED),
    (dict(B=0), OK),                              # empty: nothing launched
    (dict(Lq=0, Lk=0, mask=2), OK),
])
def test_forward_validation(L, kw, expect):
    assert fwd(L, **kw) == expect


def test_project_and_out_proj_validation(L):
    P = L.mha_project_qkv
    # (dt, B, Lq, Lk, d_model, h, dk, dv, x_q, x_kv, wq, wk, wv, q, k, v, stream)
    base = [BF16, 2, 8, 8, 512, 8, 64, 64] + [FAKE] * 8 + [None]
    def call(**over):
        a = list(base)
        keys = ["dt", "B", "Lq", "Lk", "dm", "h", "dk", "dv", "xq", "xkv", "wq", "wk", "wv",
                "q", "k", "v"]
        for name, val in over.items():
            a[keys.index(name)] = val
        return P(*a)
    assert call(dm=0) == INVALID
    assert call(xq=None) == INVALID
    assert call(wv=FAKE + 4) == INVALID
    assert call(dk=64, dv=32) == UNSUPPORTED
    assert call(dm=500) == UNSUPPORTED
    assert call(h=3, dk=20, dv=20) == UNSUPPORTED
    assert call(B=0) == OK
    O = L.mha_out_proj
    assert O(BF16, 2, 8, 8, 64, 512, None, FAKE, FAKE, None) == INVALID
    assert O(BF16, 2, 8, 8, 64, 500, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert O(BF16, 0, 8, 8, 64, 512, FAKE, FAKE, FAKE, None) == OK
    assert O(9, 2, 8, 8, 64, 512, FAKE, FAKE, FAKE, None) == INVALID


def test_fused_validation(L):
    F = L.mha_self_attention_fused
    # (dt, B, L, d_model, h, dk, x, wq, wk, wv, mask, lens, o, stream)
    base = [BF16, 2, 128, 512, 8, 64] + [FAKE] * 4 + [0, None, FAKE, None]
    keys = ["dt", "B", "L", "dm", "h", "dk", "x", "wq", "wk", "wv", "mask", "lens", "o"]
    def call(**over):
        a = list(base)
        for name, val in over.items():
            a[keys.index(name)] = val
        return F(*a)
    assert call(dt=5) == INVALID
    assert call(L=0) == INVALID
    assert call(h=0) == INVALID
    assert call(mask=8) == INVALID
    assert call(mask=1) == INVALID                  # key padding needs lengths
    assert call(x=None) == INVALID
    assert call(wk=FAKE + 2) == INVALID             # misaligned
    assert call(L=129) == UNSUPPORTED               # rows of at most 128 tokens
    assert call(dk=32) == UNSUPPORTED
    assert call(dt=F32) == UNSUPPORTED
    assert call(dm=96) == UNSUPPORTED
    assert call(B=0) == OK


@pytest.mark.skipif(bool(CHECKED), reason="binding test; the checked library is loaded apart")
def test_python_binding_checks_before_calling():
    import torch
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):          # host tensors are refused
        mha.mha_forward(q, q, q)


def test_projection_size_limits(L):
    """bf16 GEMMs address a weight matrix with 32-bit byte offsets: weights of
    2^30 elements or more are refused (nothing is launched)."""
    P = L.mha_project_qkv
    # (dt, B, Lq, Lk, d_model, h, d_k, d_v, x_q, x_kv, w_q, w_k, w_v, q, k, v, stream)
    assert P(BF16, 1, 8, 8, 32768, 512, 64, 64, *([FAKE] * 8), None) == UNSUPPORTED
    O = L.mha_out_proj
    assert O(BF16, 1, 8, 512, 64, 32768, FAKE, FAKE, FAKE, None) == UNSUPPORTED


def test_windowed_validation(L):
    import ctypes
    W = L.mha_forward_windowed
    i, p = ctypes.c_int, ctypes.c_void_p
    W.argtypes = [i, i, i, i, i, i, i, p, p, p, i, p, i, p, p]
    # (dt, B, h, Lq, Lk, dk, dv, q, k, v, mask, lens, window, o, stream)
    def call(**kw):
        a = dict(dt=BF16, B=2, h=2, Lq=8, Lk=8, dk=64, dv=64, q=FAKE, k=FAKE, v=FAKE, mask=0,
                 lens=None, window=3, o=FAKE)
        a.update(kw)
        return W(*a.values(), None)
    assert call(window=-1) == INVALID             # a window is >= 0
    assert call(Lk=9) == INVALID                  # queries and keys on one axis
    assert call(mask=1) == INVALID                # key padding needs lengths
    assert call(dk=48, dv=48) == UNSUPPORTED
    assert call(B=0) == OK


def test_decode_validation(L):
    import ctypes
    D = L.mha_decode
    i, p = ctypes.c_int, ctypes.c_void_p
    D.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p, ctypes.c_size_t, p]
    L.mha_decode_workspace_bytes.argtypes = [i, i, i, i]
    L.mha_decode_workspace_bytes.restype = ctypes.c_size_t
    need = L.mha_decode_workspace_bytes(4, 8, 2000, 64)
    assert need == 4 * 8 * 2 * (64 + 2) * 4            # 2 chunks of 1024 keys
    assert L.mha_decode_workspace_bytes(4, 8, 1024, 64) == 4 * 8 * 1 * 66 * 4
    assert L.mha_decode_workspace_bytes(4, 8, 1025, 128) == 4 * 8 * 2 * 130 * 4
    assert L.mha_decode_workspace_bytes(4, 8, 0, 64) == 4 * 8 * 1 * 66 * 4
    assert L.mha_decode_workspace_bytes(-1, 8, 10, 64) == 0
    # (dt, B, h, L, dk, dv, q, k, v, lens, o, ws, ws_bytes, stream)
    def call(**kw):
        a = dict(dt=BF16, B=4, h=8, L=2000, dk=64, dv=64, q=FAKE, k=FAKE, v=FAKE, lens=FAKE,
                 o=FAKE, ws=FAKE, nb=need)
        a.update(kw)
        return D(*a.values(), None)
    assert call(dt=9) == INVALID
    assert call(L=-1) == INVALID
    assert call(lens=None) == INVALID               # the cache lengths are required
    assert call(ws=None) == INVALID
    assert call(ws=FAKE + 4) == INVALID             # 16-byte alignment
    assert call(nb=need - 4) == INVALID             # too small
    assert call(dk=32, dv=32) == UNSUPPORTED
    assert call(dk=64, dv=128) == UNSUPPORTED
    assert call(dt=F32) == UNSUPPORTED
    assert call(B=0) == OK


def test_post_norm_validation(L):
    P = L.mha_out_proj_post_norm
    # (dt, B, Lq, h, dv, d_model, o, w_o, x_res, gamma, beta, eps, y, stream)
    def call(**kw):
        a = dict(dt=BF16, B=2, Lq=8, h=8, dv=64, dm=512, o=FAKE, w=FAKE, x=FAKE, g=FAKE,
                 b=FAKE, eps=1e-6, y=FAKE)
        a.update(kw)
        return P(*a.values(), None)
    assert call(dt=5) == INVALID
    assert call(B=-1) == INVALID
    assert call(h=0) == INVALID
    assert call(eps=-1e-3) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(eps=float("inf")) == INVALID
    assert call(g=None) == INVALID
    assert call(b=FAKE + 8) == INVALID                 # 16-byte alignment
    assert call(y=FAKE + 16) == INVALID                # partly over x_res
    assert call(dt=F32, dm=384) == UNSUPPORTED         # fp32 too: d_model in {256, 512, 1024}
    assert call(dt=F32, y=FAKE + 16) == INVALID        # overlap counted in 4-byte elements
    assert call(dm=384) == UNSUPPORTED                 # d_model in {256, 512, 1024}
    assert call(dm=2048) == UNSUPPORTED
    assert call(h=3, dv=16) == UNSUPPORTED             # h*d_v % 32
    assert call(h=1024, dv=1024, dm=1024) == UNSUPPORTED  # W^O of 2^30 elements
    assert call(B=0) == OK
    assert call(Lq=0, o=None) == OK


def test_decode_noalloc_validation(L):
    """The allocation-free decode step validates like mha_decode and refuses
    problems whose partial states exceed the static scratch (16 MiB) before
    any HIP call."""
    N = L.mha_decode_noalloc
    # (dt, B, h, L, dk, dv, q, k, v, lens, o, stream)
    def call(**kw):
        a = dict(dt=BF16, B=4, h=8, L=2000, dk=64, dv=64, q=FAKE, k=FAKE, v=FAKE, lens=FAKE,
                 o=FAKE)
        a.update(kw)
        return N(*a.values(), None)
    assert call(dt=9) == INVALID
    assert call(h=0) == INVALID
    assert call(lens=None) == INVALID
    assert call(o=FAKE + 4) == INVALID
    assert call(dk=32, dv=32) == UNSUPPORTED
    assert call(B=0) == OK
    # 64 x 16 heads x 64 chunks x 66 floats = 17.3 MB > 16 MiB
    assert L.mha_decode_workspace_bytes(64, 16, 65536, 64) > 16 << 20
    assert call(B=64, h=16, L=65536) == SCRATCH
    assert b"scratch" in L.mha_status_string(SCRATCH)
