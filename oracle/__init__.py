"""fp64 CPU oracle for scaled dot-product multi-head attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It
shares no code with the HIP library (``transformer_scaled_dot_fwd_amd``) and
neither imports the other; the product path never routes through it.

The arithmetic lives in ``oracle.c`` (plain fp64 loops, OpenMP over output
rows); this module only builds that file with gcc, loads it with ctypes and
marshals numpy arrays.  What each function computes, and the passages of the
pages it follows, is written in ``oracle.c``:

* ``attention``      -- softmax(Q K^T / sqrt(d_k) + M) V for every (b, head);
  Deep-reading page section 04, attention equation with the mask M; with
  ``window=w``, restricted self-attention (keys within w positions of the
  query; Deep-reading page section 05, complexity table).
* ``attention_rows`` -- the same definition for a sampled list of rows.
* ``matmul``         -- Y = A W (the projections and W^O of MultiHead;
  slide "Multi-Head Attention").
* ``layer_norm``, ``out_proj_post_norm`` -- LayerNorm(x + Sublayer(x)),
  the post-norm residual output of the sub-layer (Deep-reading page section
  03).
* ``mha_block``      -- MultiHead(X_q, X_kv, X_kv) = Concat(heads) W^O with
  head t = Attention(X_q W_t^Q, X_kv W_t^K, X_kv W_t^V), head t owning column
  block t (paperglide two-head toy example).

Parity pins: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (worked examples, closed forms, invariants,
library cross-checks); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

MASK_NONE = 0
MASK_KEY_PADDING = 1
MASK_CAUSAL = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")


def compile_source(src: str, out: str, verbose: bool = False, quiet: bool = False) -> str:
    """gcc -O2 -fopenmp (no fast-math) of one C file into a shared library."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-o", tmp, src, "-lm"] + ([] if quiet else ["-Wall", "-Wextra"])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL if quiet else None)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so."""
    return compile_source(SOURCE, LIBRARY, verbose)


def _f64(a) -> np.ndarray:
    """Exact upcast to a C-contiguous fp64 numpy array (bf16 and fp32 values
    are representable in fp64, so nothing is rounded)."""
    if hasattr(a, "detach"):  # torch tensor (CPU)
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _lens(kv_lens, B):
    if kv_lens is None:
        return None
    if hasattr(kv_lens, "detach"):
        kv_lens = kv_lens.detach().to("cpu").numpy()
    out = np.ascontiguousarray(kv_lens, dtype=np.int32)
    if out.shape != (B,):
        raise ValueError(f"kv_lens must have shape ({B},), got {out.shape}")
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data


class Oracle:
    """ctypes front end of one compiled copy of oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        L, P = ctypes.c_long, ctypes.c_void_p
        lib.oracle_attention.argtypes = [L, L, L, L, L, L, P, P, P, ctypes.c_int, P, L, P, P,
                                         P]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention_rows.argtypes = [L, L, L, L, L, L, P, P, P, ctypes.c_int, P,
                                              L, L, P, P]
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_matmul.argtypes = [L, L, L, P, P, P]
        lib.oracle_matmul.restype = ctypes.c_int
        lib.oracle_layer_norm.argtypes = [L, L, P, P, P, ctypes.c_double, P]
        lib.oracle_layer_norm.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    def attention(self, q, k, v, mask: int = MASK_NONE, kv_lens=None,
                  return_p: bool = False, return_s: bool = False, window=None):
        """O = softmax(Q K^T / sqrt(d_k) + M) V in fp64.

        q [B, Lq, h, d_k], k [B, Lk, h, d_k], v [B, Lk, h, d_v] (BLHD);
        returns o [B, Lq, h, d_v] and, on request, P and the scaled logits S,
        both [B, h, Lq, Lk] (S is -inf where masked).  window: half-width w
        of restricted self-attention (keys with |i - j| <= w), or None.
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Lq, h, dk = q.shape
        Bk, Lk, hk, dk2 = k.shape
        dv = v.shape[3]
        if (Bk, hk, dk2) != (B, h, dk) or v.shape[:3] != (B, Lk, h):
            raise ValueError("q/k/v shapes disagree")
        lens = _lens(kv_lens, B) if (mask & MASK_KEY_PADDING) else None
        o = np.zeros((B, Lq, h, dv), dtype=np.float64)
        p = np.zeros((B, h, Lq, Lk), dtype=np.float64) if return_p else None
        s = np.zeros((B, h, Lq, Lk), dtype=np.float64) if return_s else None
        rc = self.lib.oracle_attention(B, h, Lq, Lk, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                       int(mask), _ptr(lens), -1 if window is None else int(window),
                                       _ptr(o), _ptr(p), _ptr(s))
        if rc != 0:
            raise ValueError("oracle_attention rejected its arguments")
        if return_p or return_s:
            out = (o,)
            if return_p:
                out += (p,)
            if return_s:
                out += (s,)
            return out
        return o

    def attention_rows(self, q, k, v, rows, mask: int = MASK_NONE, kv_lens=None, window=None):
        """The attention definition for selected rows only.

        rows: int array [n, 3] of (b, head, i).  Returns [n, d_v] fp64, row n
        being o[b, i, head, :].
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Lq, h, dk = q.shape
        Lk = k.shape[1]
        dv = v.shape[3]
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        lens = _lens(kv_lens, B) if (mask & MASK_KEY_PADDING) else None
        o = np.zeros((rows.shape[0], dv), dtype=np.float64)
        rc = self.lib.oracle_attention_rows(B, h, Lq, Lk, dk, dv, _ptr(q), _ptr(k),
                                            _ptr(v), int(mask), _ptr(lens),
                                            -1 if window is None else int(window),
                                            rows.shape[0], _ptr(rows), _ptr(o))
        if rc != 0:
            raise ValueError("oracle_attention_rows rejected its arguments")
        return o

    def matmul(self, a, w):
        """Y = A W for 2-D A [M, K] and W [K, N], fp64 triple loop."""
        a, w = _f64(a), _f64(w)
        M, K = a.shape
        K2, N = w.shape
        if K != K2:
            raise ValueError("inner dimensions disagree")
        y = np.zeros((M, N), dtype=np.float64)
        self.lib.oracle_matmul(M, K, N, _ptr(a), _ptr(w), _ptr(y))
        return y

    def layer_norm(self, z, gamma, beta, eps: float = 1e-6):
        """Per-row layer normalisation of z [..., N] in fp64 (population
        variance, gain gamma [N], bias beta [N], eps inside the root)."""
        z, gamma, beta = _f64(z), _f64(gamma), _f64(beta)
        N = z.shape[-1]
        if gamma.shape != (N,) or beta.shape != (N,):
            raise ValueError("gamma and beta must have shape (N,)")
        zz = np.ascontiguousarray(z.reshape(-1, N))
        out = np.zeros_like(zz)
        if self.lib.oracle_layer_norm(zz.shape[0], N, _ptr(zz), _ptr(gamma), _ptr(beta),
                                      float(eps), _ptr(out)) != 0:
            raise ValueError("oracle_layer_norm rejected its arguments")
        return out.reshape(z.shape)

    def out_proj_post_norm(self, o, w_o, x, gamma, beta, eps: float = 1e-6):
        """LayerNorm(x + Concat(heads) W^O): the attention sub-layer's output
        with its residual connection, post-norm.  x [B, Lq, d_model]."""
        return self.layer_norm(_f64(x) + self.out_proj(o, w_o), gamma, beta, eps)

    def project_qkv(self, x_q, x_kv, w_q, w_k, w_v, h: int):
        """Q = X_q W^Q, K = X_kv W^K, V = X_kv W^V, returned BLHD.

        x_q [B, Lq, d_model], x_kv [B, Lk, d_model]; W^Q, W^K [d_model, h*d_k],
        W^V [d_model, h*d_v].  Head t is column block t of each product.
        """
        x_q, x_kv = _f64(x_q), _f64(x_kv)
        B, Lq, dm = x_q.shape
        Lk = x_kv.shape[1]
        q = self.matmul(x_q.reshape(B * Lq, dm), w_q)
        k = self.matmul(x_kv.reshape(B * Lk, dm), w_k)
        v = self.matmul(x_kv.reshape(B * Lk, dm), w_v)
        return (q.reshape(B, Lq, h, -1), k.reshape(B, Lk, h, -1), v.reshape(B, Lk, h, -1))

    def out_proj(self, o, w_o):
        """Y = Concat(head_1..head_h) W^O; o [B, Lq, h, d_v] is already the
        concat [B*Lq, h*d_v] in memory.  Returns [B, Lq, d_model]."""
        o = _f64(o)
        B, Lq = o.shape[:2]
        y = self.matmul(o.reshape(B * Lq, -1), w_o)
        return y.reshape(B, Lq, -1)

    def mha_block(self, x_q, x_kv, w_q, w_k, w_v, w_o, h: int, mask: int = MASK_NONE,
                  kv_lens=None):
        """MultiHead(X_q, X_kv, X_kv) = Concat(head_1..head_h) W^O in fp64."""
        q, k, v = self.project_qkv(x_q, x_kv, w_q, w_k, w_v, h)
        o = self.attention(q, k, v, mask=mask, kv_lens=kv_lens)
        return self.out_proj(o, w_o)


_default = None


def build_checked(out: str, verbose: bool = False) -> str:
    """oracle.c built with AddressSanitizer and UndefinedBehaviorSanitizer
    (gcc), for a run of the pins under the sanitizers; load it into a
    process that preloads gcc's libasan (``checked_runtime()``)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-o", tmp, SOURCE, "-lm", "-Wall", "-Wextra"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def checked_runtime() -> str:
    """gcc's shared ASan runtime (to preload before a checked build)."""
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                         text=True, check=True).stdout.strip()
    if not os.path.isabs(out):
        raise RuntimeError("gcc's libasan.so not found")
    return out


def default() -> Oracle:
    """The oracle built from oracle.c (rebuilt when the source is newer);
    ORACLE_CHECKED_LIBRARY names a sanitizer build to load instead."""
    global _default
    if _default is None:
        checked = os.environ.get("ORACLE_CHECKED_LIBRARY")
        if checked:
            _default = Oracle(checked)
            return _default
        if not os.path.exists(LIBRARY) or os.path.getmtime(SOURCE) > os.path.getmtime(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def attention(*args, **kw):
    return default().attention(*args, **kw)


def attention_rows(*args, **kw):
    return default().attention_rows(*args, **kw)


def matmul(*args, **kw):
    return default().matmul(*args, **kw)


def project_qkv(*args, **kw):
    return default().project_qkv(*args, **kw)


def out_proj(*args, **kw):
    return default().out_proj(*args, **kw)


def layer_norm(*args, **kw):
    return default().layer_norm(*args, **kw)


def out_proj_post_norm(*args, **kw):
    return default().out_proj_post_norm(*args, **kw)


def mha_block(*args, **kw):
    return default().mha_block(*args, **kw)
