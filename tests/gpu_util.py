"""Helpers for the GPU parity tests: device handle, tolerances, reporting.

Tolerances (written here once, used by every parity test):
  fp32 runs   max |gpu - oracle| <= 1e-5
  bf16 runs   |gpu - oracle| <= 1e-2 + 1e-2 * |oracle|, elementwise
Masked positions are checked bit-exactly through invariance tests.
"""
import sys

import numpy as np
import torch

F32_ATOL = 1e-5
BF16_ATOL = 1e-2
BF16_RTOL = 1e-2


def device():
    # Fail loudly (never skip) when the GPU or the library is missing.
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import transformer_scaled_dot_fwd_amd as mha
    mha.lib()
    return torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def check(gpu, ref, dtype: str, what: str = "", f32_atol: float = F32_ATOL):
    """Compare a GPU result with the fp64 oracle; return (max_abs, max_rel).
    f32_atol replaces the fp32 bound where a test derives a wider one from
    its inputs' magnitudes (and says so)."""
    g = to_np(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err / np.maximum(np.abs(r), 1e-6)).max()) if err.size else 0.0
    if dtype == "f32":
        assert max_abs <= f32_atol, f"{what}: max abs err {max_abs:.3e} > {f32_atol:.3e}"
    else:
        bound = BF16_ATOL + BF16_RTOL * np.abs(r)
        bad = err > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} of {err.size} elements outside "
                               f"1e-2 + 1e-2|o| (max abs {max_abs:.3e})")
    say(f"  {what}: max abs {max_abs:.3e}, max rel {max_rel:.3e}")
    return max_abs, max_rel
