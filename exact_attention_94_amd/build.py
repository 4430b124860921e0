"""Build the HIP attention library (libfa.so) in-tree for gfx950.

Usage: python -m exact_attention_94_amd.build   (or call build_library()).
Every HIP source is compiled with hipcc for gfx950 with packed-fp32 instructions disabled, then
linked into exact_attention_94_amd/libfa.so. Object files go to _build/ at the repository root.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libfa.so)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-Wno-unused-command-line-argument",
        # Packed fp32 VALU forms are kept out of every kernel.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, extra, build_dir=BUILD_DIR):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", src, "-o", obj] + compile_flags() + list(extra)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj, res.stderr


def build_library(verbose=False, extra_flags=(), out=LIB, build_dir=BUILD_DIR):
    """Compile all sources and link the library (default: libfa.so in the package); returns its
    path. Always rebuilds. extra_flags reach every hipcc compile (e.g. tuning overrides)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra_flags, build_dir), srcs))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
