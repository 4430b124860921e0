"""Tuning of the forward kernel's tile width (keys per K/V tile) per head dimension.

"FlashAttention 为什么不需要存下注意力矩阵" §05 (first difference) notes that production kernels do
not derive their block sizes from the SRAM formula but choose them per head dimension, dtype and
causality among precompiled configurations, by measurement. This script does that for the 16-bit
forward kernel on the GPU it runs on:

  python -m exact_attention_94_amd.tune build            # compile one library per candidate
  python -m exact_attention_94_amd.tune measure FILE     # time them on the GPU, results -> FILE
  python -m exact_attention_94_amd.tune write FILE       # write csrc/fa_tune.h from FILE
  python -m exact_attention_94_amd.tune all              # the three in a row (GPU machine)

Candidates are 32, 64 and 128 keys per tile, where the kernel's staging allows them (each wave
issues whole 1 KB direct loads: keys * d * 2 bytes must be a multiple of 4 KB). The workload is
B=2, H=16, N=4096, causal, bf16 inputs, seeded normal draws, one per head dimension. After
`write`, rebuild the library (python -m exact_attention_94_amd.build).
"""

from __future__ import annotations

import ctypes
import json
import os
import sys

from . import build as _build

CANDIDATES = (32, 64, 128)
HEAD_DIMS = (32, 64, 96, 128)
TUNE_DIR = os.path.join(_build.ROOT, "_build", "tune")
HEADER = os.path.join(_build.CSRC, "fa_tune.h")


def valid(keys, d):
    return (keys * d * 2) % 4096 == 0


def lib_path(keys):
    return os.path.join(TUNE_DIR, f"keys{keys}", "libfa.so")


def build_candidates():
    for keys in CANDIDATES:
        flags = [f"-DFA_FWD_BC_{d}={keys if valid(keys, d) else 64}" for d in HEAD_DIMS]
        out = lib_path(keys)
        os.makedirs(os.path.dirname(out), exist_ok=True)
        _build.build_library(extra_flags=flags, out=out, build_dir=os.path.dirname(out))
        print(f"built {out}", flush=True)


def _time_forward(lib, d, steps=20, warmup=5):
    import torch
    B, H, N = 2, 16, 4096
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(d)
    q, k, v = (torch.randn((B, H, N, d), device=dev, generator=g).to(torch.bfloat16)
               for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def call():
        st = lib.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, H, N, d, d ** -0.5, 1, 2, 2, stream)
        if st != 0:
            raise RuntimeError(f"fa_forward returned {st}")

    for _ in range(warmup):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def measure(path):
    # torch first: its HIP runtime must be the one the candidate libraries bind to (loading a
    # library first would pull in a second runtime, whose streams torch's are not).
    import torch  # noqa: F401
    results = {}
    for keys in CANDIDATES:
        lib = ctypes.CDLL(lib_path(keys))
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp]
        lib.fa_forward.restype = i
        for d in HEAD_DIMS:
            if not valid(keys, d):
                continue
            ms = _time_forward(lib, d)
            results.setdefault(str(d), {})[str(keys)] = ms
            print(json.dumps({"d": d, "keys": keys, "ms": round(ms, 4)}), flush=True)
    with open(path, "w") as fh:
        json.dump(results, fh, indent=1)
    return results


def write(path, header=HEADER):
    with open(path) as fh:
        results = json.load(fh)
    best = {d: min(results[str(d)].items(), key=lambda kv: kv[1])[0] for d in HEAD_DIMS}
    with open(header) as fh:
        text = fh.read()
    for d in HEAD_DIMS:
        old = next(line for line in text.splitlines() if line.startswith(f"#define FA_FWD_BC_{d} "))
        text = text.replace(old, f"#define FA_FWD_BC_{d} {best[d]}")
    with open(header, "w") as fh:
        fh.write(text)
    print(json.dumps({"chosen": best}))
    return best


def main(argv):
    if not argv or argv[0] not in ("build", "measure", "write", "all"):
        print(__doc__)
        return 2
    cmd = argv[0]
    path = argv[1] if len(argv) > 1 else os.path.join(TUNE_DIR, "results.json")
    if cmd in ("build", "all"):
        build_candidates()
    if cmd in ("measure", "all"):
        measure(path)
    if cmd in ("write", "all"):
        write(path)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
