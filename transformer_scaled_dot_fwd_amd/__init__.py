"""Multi-head scaled dot-product attention forward for AMD MI355X (gfx950).

A thin ctypes binding over ``libmha.so``, whose C ABI is ``include/mha.h``.
The functions carry the C names; they only check and marshal arguments
(torch tensors -> device pointers, torch's current HIP stream -> hipStream_t)
and raise on a non-zero status.  Every step of the computation runs in the
library's HIP kernels; there is no CPU or PyTorch fallback, and a missing
library raises at the first call.

    mha_forward(q, k, v, mask, kv_lens)          O = softmax(QK^T/sqrt(d_k) + M) V
    mha_forward(..., window=w)                    the same over keys |i - j| <= w only
    mha_decode(q, k_cache, v_cache, cache_lens)   one decoding step against a K/V cache
    mha_decode_noalloc(q, k, v, lens, out)        the same with no allocation at all
    mha_project_qkv(x_q, x_kv, w_q, w_k, w_v, h)  Q, K, V = X_q W^Q, X_kv W^K, X_kv W^V
    mha_out_proj(o, w_o)                          Y = Concat(heads) W^O
    mha_out_proj_post_norm(o, w_o, x, g, b)       LayerNorm(x + Concat(heads) W^O)
    mha_block(...)                                the three above in sequence

Tensors are CUDA (HIP) tensors, contiguous, all of one dtype (torch.bfloat16
or torch.float32); q/k/v/o use the BLHD layout [B, L, h, d].  ``kv_lens`` is
an int32 device tensor [B].
"""
from __future__ import annotations

import ctypes
import os

import torch

MASK_NONE = 0
MASK_KEY_PADDING = 1
MASK_CAUSAL = 2

MHA_F32 = 0
MHA_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libmha.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "mha.h")

_lib = None


def library_path() -> str:
    return LIBRARY


def lib() -> ctypes.CDLL:
    """The loaded libmha.so (ctypes), with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(
            f"{LIBRARY} is not built; run `python -m transformer_scaled_dot_fwd_amd.build` "
            "(or __graft_entry__.build())")
    _lib = declare(ctypes.CDLL(LIBRARY))
    return _lib


def declare(L: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the argument and return types of the C ABI on a loaded copy
    of the library (the in-tree libmha.so, or a host-only checking build of
    the same sources)."""
    i, p = ctypes.c_int, ctypes.c_void_p
    L.mha_forward.argtypes = [i, i, i, i, i, i, i, p, p, p, i, p, p, p]
    L.mha_forward.restype = i
    L.mha_forward_windowed.argtypes = [i, i, i, i, i, i, i, p, p, p, i, p, i, p, p]
    L.mha_forward_windowed.restype = i
    L.mha_decode.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p, ctypes.c_size_t, p]
    L.mha_decode.restype = i
    L.mha_decode_noalloc.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p]
    L.mha_decode_noalloc.restype = i
    L.mha_decode_workspace_bytes.argtypes = [i, i, i, i]
    L.mha_decode_workspace_bytes.restype = ctypes.c_size_t
    L.mha_project_qkv.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p, p, p, p]
    L.mha_project_qkv.restype = i
    L.mha_out_proj.argtypes = [i, i, i, i, i, i, p, p, p, p]
    L.mha_out_proj.restype = i
    L.mha_out_proj_post_norm.argtypes = [i, i, i, i, i, i, p, p, p, p, p, ctypes.c_float,
                                         p, p]
    L.mha_out_proj_post_norm.restype = i
    L.mha_self_attention_fused.argtypes = [i, i, i, i, i, i, p, p, p, p, i, p, p, p]
    L.mha_self_attention_fused.restype = i
    L.mha_status_string.argtypes = [i]
    L.mha_status_string.restype = ctypes.c_char_p
    return L


class MHAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().mha_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MHA_BF16
    if t.dtype == torch.float32:
        return MHA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _check(t: torch.Tensor, name: str, dtype=None, device=None, shape=None) -> None:
    """t is a contiguous device tensor; of `dtype`, on `device` and of
    `shape` where given (the library writes outputs by their shape, so a
    smaller buffer must never reach it)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def mha_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: int = MASK_NONE,
                kv_lens: torch.Tensor | None = None, out: torch.Tensor | None = None,
                window: int | None = None) -> torch.Tensor:
    """O = softmax(Q K^T / sqrt(d_k) + M) V; q [B,Lq,h,d_k], k [B,Lk,h,d_k],
    v [B,Lk,h,d_v] -> o [B,Lq,h,d_v].  window=w: restricted self-attention
    (keys within w positions of each query; mha_forward_windowed)."""
    _check(q, "q")
    _check(k, "k", q.dtype, q.device)
    _check(v, "v", q.dtype, q.device)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, L, h, d]")
    B, Lq, h, dk = q.shape
    Lk = k.shape[1]
    dv = v.shape[3]
    if k.shape != (B, Lk, h, dk) or v.shape[:3] != (B, Lk, h):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}")
    lens_ptr = None
    if mask & MASK_KEY_PADDING:
        if kv_lens is None:
            raise ValueError("key padding needs kv_lens")
        _check(kv_lens, "kv_lens", torch.int32, q.device, (B,))
        lens_ptr = kv_lens.data_ptr()
    if out is None:
        out = torch.empty((B, Lq, h, dv), dtype=q.dtype, device=q.device)
    else:
        _check(out, "out", q.dtype, q.device, (B, Lq, h, dv))
    if window is None:
        rc = lib().mha_forward(_dtype_code(q), B, h, Lq, Lk, dk, dv, q.data_ptr(),
                               k.data_ptr(), v.data_ptr(), int(mask), lens_ptr, out.data_ptr(),
                               _stream(q.device))
        name = "mha_forward"
    else:
        rc = lib().mha_forward_windowed(_dtype_code(q), B, h, Lq, Lk, dk, dv, q.data_ptr(),
                                        k.data_ptr(), v.data_ptr(), int(mask), lens_ptr,
                                        int(window), out.data_ptr(), _stream(q.device))
        name = "mha_forward_windowed"
    if rc != 0:
        raise MHAError(rc, name)
    return out


def mha_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               cache_lens: torch.Tensor, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decoding step: q [B,1,h,d] against the caches k_cache, v_cache
    [B,L_cache,h,d] with cache_lens (int32 [B]) valid keys -> o [B,1,h,d].
    `workspace` (bytes, mha_decode_workspace_bytes) is allocated per call
    from torch's caching allocator when not given."""
    _check(q, "q")
    _check(k_cache, "k_cache", q.dtype, q.device)
    _check(v_cache, "v_cache", q.dtype, q.device)
    _check(cache_lens, "cache_lens", torch.int32, q.device)
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be [B, 1, h, d]")
    B, _, h, dk = q.shape
    Lc = k_cache.shape[1]
    dv = v_cache.shape[3]
    if k_cache.shape != (B, Lc, h, dk) or v_cache.shape[:3] != (B, Lc, h):
        raise ValueError("cache shape mismatch")
    if cache_lens.shape != (B,):
        raise ValueError(f"cache_lens must have shape ({B},)")
    if out is None:
        out = torch.empty((B, 1, h, dv), dtype=q.dtype, device=q.device)
    else:
        _check(out, "out", q.dtype, q.device, (B, 1, h, dv))
    nbytes = int(lib().mha_decode_workspace_bytes(B, h, Lc, dk))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    else:
        _check(workspace, "workspace", device=q.device)
    rc = lib().mha_decode(_dtype_code(q), B, h, Lc, dk, dv, q.data_ptr(), k_cache.data_ptr(),
                          v_cache.data_ptr(), cache_lens.data_ptr(), out.data_ptr(),
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _stream(q.device))
    if rc != 0:
        raise MHAError(rc, "mha_decode")
    return out


def mha_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       cache_lens: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """mha_decode with the library's static scratch instead of a workspace:
    the call allocates nothing, so it may be captured in a HIP graph.  The
    output tensor must be given.  Calls that overlap in time on one GPU
    share the scratch and race."""
    _check(q, "q")
    _check(k_cache, "k_cache", q.dtype, q.device)
    _check(v_cache, "v_cache", q.dtype, q.device)
    _check(cache_lens, "cache_lens", torch.int32, q.device)
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be [B, 1, h, d]")
    B, _, h, dk = q.shape
    Lc = k_cache.shape[1]
    dv = v_cache.shape[3]
    if k_cache.shape != (B, Lc, h, dk) or v_cache.shape[:3] != (B, Lc, h):
        raise ValueError("cache shape mismatch")
    if cache_lens.shape != (B,):
        raise ValueError(f"cache_lens must have shape ({B},)")
    _check(out, "out", q.dtype, q.device, (B, 1, h, dv))
    rc = lib().mha_decode_noalloc(_dtype_code(q), B, h, Lc, dk, dv, q.data_ptr(),
                                  k_cache.data_ptr(), v_cache.data_ptr(), cache_lens.data_ptr(),
                                  out.data_ptr(), _stream(q.device))
    if rc != 0:
        raise MHAError(rc, "mha_decode_noalloc")
    return out


def mha_project_qkv(x_q: torch.Tensor, x_kv: torch.Tensor, w_q: torch.Tensor,
                    w_k: torch.Tensor, w_v: torch.Tensor, h: int, out=None):
    """Q = X_q W^Q, K = X_kv W^K, V = X_kv W^V as BLHD tensors.

    x_q [B,Lq,d_model], x_kv [B,Lk,d_model] (pass x_q again for
    self-attention), w_q/w_k [d_model, h*d_k], w_v [d_model, h*d_v]."""
    for t, n in ((x_q, "x_q"), (x_kv, "x_kv"), (w_q, "w_q"), (w_k, "w_k"), (w_v, "w_v")):
        _check(t, n, x_q.dtype, x_q.device)
    if x_q.dim() != 3 or x_kv.dim() != 3 or w_q.dim() != 2 or w_k.dim() != 2 or w_v.dim() != 2:
        raise ValueError("x_q, x_kv must be [B, L, d_model] and the weights 2-D")
    B, Lq, dm = x_q.shape
    Lk = x_kv.shape[1]
    if x_kv.shape != (B, Lk, dm):
        raise ValueError("x_kv shape mismatch")
    nq, nv = w_q.shape[1], w_v.shape[1]
    if w_q.shape != (dm, nq) or w_k.shape != (dm, nq) or w_v.shape[0] != dm:
        raise ValueError("weight shape mismatch")
    if nq % h or nv % h:
        raise ValueError("projection width not divisible by h")
    dk, dv = nq // h, nv // h
    if out is None:
        q = torch.empty((B, Lq, h, dk), dtype=x_q.dtype, device=x_q.device)
        k = torch.empty((B, Lk, h, dk), dtype=x_q.dtype, device=x_q.device)
        v = torch.empty((B, Lk, h, dv), dtype=x_q.dtype, device=x_q.device)
    else:
        q, k, v = out
        for t, n, shape in ((q, "q", (B, Lq, h, dk)), (k, "k", (B, Lk, h, dk)),
                            (v, "v", (B, Lk, h, dv))):
            _check(t, n, x_q.dtype, x_q.device, shape)
    rc = lib().mha_project_qkv(_dtype_code(x_q), B, Lq, Lk, dm, h, dk, dv, x_q.data_ptr(),
                               x_kv.data_ptr(), w_q.data_ptr(), w_k.data_ptr(), w_v.data_ptr(),
                               q.data_ptr(), k.data_ptr(), v.data_ptr(), _stream(x_q.device))
    if rc != 0:
        raise MHAError(rc, "mha_project_qkv")
    return q, k, v


def mha_out_proj(o: torch.Tensor, w_o: torch.Tensor, out: torch.Tensor | None = None
                 ) -> torch.Tensor:
    """Y = Concat(head_1..head_h) W^O; o [B,Lq,h,d_v], w_o [h*d_v, d_model]."""
    _check(o, "o")
    _check(w_o, "w_o", o.dtype, o.device)
    if o.dim() != 4 or w_o.dim() != 2:
        raise ValueError("o must be [B, L, h, d_v] and w_o 2-D")
    B, Lq, h, dv = o.shape
    dm = w_o.shape[1]
    if w_o.shape != (h * dv, dm):
        raise ValueError("w_o shape mismatch")
    if out is None:
        out = torch.empty((B, Lq, dm), dtype=o.dtype, device=o.device)
    else:
        _check(out, "out", o.dtype, o.device, (B, Lq, dm))
    rc = lib().mha_out_proj(_dtype_code(o), B, Lq, h, dv, dm, o.data_ptr(), w_o.data_ptr(),
                            out.data_ptr(), _stream(o.device))
    if rc != 0:
        raise MHAError(rc, "mha_out_proj")
    return out


def mha_out_proj_post_norm(o: torch.Tensor, w_o: torch.Tensor, x_res: torch.Tensor,
                           gamma: torch.Tensor, beta: torch.Tensor, eps: float = 1e-6,
                           out: torch.Tensor | None = None) -> torch.Tensor:
    """LayerNorm(x_res + Concat(head_1..head_h) W^O) with gain gamma and bias
    beta over d_model; o [B,Lq,h,d_v], w_o [h*d_v, d_model], x_res
    [B,Lq,d_model], gamma/beta [d_model].  ``out`` may be ``x_res`` itself
    (in-place update of the residual stream)."""
    _check(o, "o")
    for t, n in ((w_o, "w_o"), (x_res, "x_res"), (gamma, "gamma"), (beta, "beta")):
        _check(t, n, o.dtype, o.device)
    if o.dim() != 4 or w_o.dim() != 2:
        raise ValueError("o must be [B, L, h, d_v] and w_o 2-D")
    B, Lq, h, dv = o.shape
    dm = w_o.shape[1]
    if w_o.shape != (h * dv, dm):
        raise ValueError("w_o shape mismatch")
    if x_res.shape != (B, Lq, dm) or gamma.shape != (dm,) or beta.shape != (dm,):
        raise ValueError("x_res, gamma or beta shape mismatch")
    if out is None:
        out = torch.empty((B, Lq, dm), dtype=o.dtype, device=o.device)
    else:
        _check(out, "out", o.dtype, o.device, (B, Lq, dm))
    rc = lib().mha_out_proj_post_norm(_dtype_code(o), B, Lq, h, dv, dm, o.data_ptr(),
                                      w_o.data_ptr(), x_res.data_ptr(), gamma.data_ptr(),
                                      beta.data_ptr(), float(eps), out.data_ptr(),
                                      _stream(o.device))
    if rc != 0:
        raise MHAError(rc, "mha_out_proj_post_norm")
    return out


def mha_self_attention_fused(x: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                             w_v: torch.Tensor, h: int, mask: int = MASK_NONE,
                             kv_lens: torch.Tensor | None = None,
                             out: torch.Tensor | None = None) -> torch.Tensor | None:
    """Self-attention of every head with the Q/K/V projections fused in:
    x [B,L,d_model], w_* [d_model, h*64] -> o [B,L,h,64] (BLHD).  Returns
    None when the shape is outside the fused kernel (bf16, d_k = 64,
    L <= 128, d_model % 64 == 0): use the two-call path then."""
    for t, n in ((x, "x"), (w_q, "w_q"), (w_k, "w_k"), (w_v, "w_v")):
        _check(t, n, x.dtype, x.device)
    if x.dim() != 3 or w_q.dim() != 2 or w_k.dim() != 2 or w_v.dim() != 2:
        raise ValueError("x must be [B, L, d_model] and the weights 2-D")
    B, L, dm = x.shape
    nq = w_q.shape[1]
    if w_q.shape != (dm, nq) or w_k.shape != (dm, nq) or w_v.shape != (dm, nq) or nq % h:
        raise ValueError("weight shape mismatch")
    dk = nq // h
    lens_ptr = None
    if mask & MASK_KEY_PADDING:
        if kv_lens is None:
            raise ValueError("key padding needs kv_lens")
        _check(kv_lens, "kv_lens", torch.int32, x.device, (B,))
        lens_ptr = kv_lens.data_ptr()
    if out is None:
        out = torch.empty((B, L, h, dk), dtype=x.dtype, device=x.device)
    else:
        _check(out, "out", x.dtype, x.device, (B, L, h, dk))
    rc = lib().mha_self_attention_fused(_dtype_code(x), B, L, dm, h, dk, x.data_ptr(),
                                        w_q.data_ptr(), w_k.data_ptr(), w_v.data_ptr(),
                                        int(mask), lens_ptr, out.data_ptr(), _stream(x.device))
    if rc == 2:  # MHA_ERR_UNSUPPORTED
        return None
    if rc != 0:
        raise MHAError(rc, "mha_self_attention_fused")
    return out


def mha_block(x_q, x_kv, w_q, w_k, w_v, w_o, h: int, mask: int = MASK_NONE, kv_lens=None):
    """MultiHead(X_q, X_kv, X_kv) = Concat(head_1..head_h) W^O on the current
    stream, no host synchronisation: for self-attention rows of at most 128
    tokens, the fused projection + attention kernel and the W^O GEMM (two
    launches); otherwise projection, attention and W^O (three launches)."""
    o = None
    if x_q is x_kv:
        o = mha_self_attention_fused(x_q, w_q, w_k, w_v, h, mask=mask, kv_lens=kv_lens)
    if o is None:
        q, k, v = mha_project_qkv(x_q, x_kv, w_q, w_k, w_v, h)
        o = mha_forward(q, k, v, mask=mask, kv_lens=kv_lens)
    return mha_out_proj(o, w_o)
