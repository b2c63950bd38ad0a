"""Build libmha.so for gfx950 with hipcc, in-tree.

    python -m transformer_scaled_dot_fwd_amd.build

Each HIP source is compiled to an object under _build/ (in parallel), then
linked into transformer_scaled_dot_fwd_amd/libmha.so.  Packed fp32 vector
instructions are disabled for the device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIBRARY = os.path.join(HERE, "libmha.so")
SOURCES = ["attention.hip", "attn_stream.hip", "decode.hip", "fused.hip", "gemm.hip", "mha_api.hip", "norm.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the device-only feature flag; drop that note.
    err = "\n".join(l for l in proc.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIBRARY + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def build_host_checked(out_dir: str, verbose: bool = False) -> str:
    """A copy of the library whose host code is built with AddressSanitizer
    and UndefinedBehaviorSanitizer (the device code is compiled as usual,
    without them): the C ABI's argument validation can run under the
    sanitizers on a machine without a GPU.  Load it into a process that
    preloads the compiler's shared ASan runtime (``asan_runtime()``)."""
    os.makedirs(out_dir, exist_ok=True)
    host = [*COMMON, "-Xarch_host", "-O1", "-Xarch_host", "-g",
            "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".host.o"))
        objs.append(obj)
        cmds.append([HIPCC, *host, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    out = os.path.join(out_dir, "libmha_host_checked.so")
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-shared-libsan",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-o", out, *objs], verbose)
    return out


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload)."""
    proc = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True, check=True)
    path = proc.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"ASan runtime not found ({path!r})")
    return path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
