"""Tuning of the 16-bit kernels' tiles per head dimension, input dtype and causality.

"FlashAttention 为什么不需要存下注意力矩阵" §05 (first difference) notes that production kernels do
not derive their block sizes from the SRAM formula but choose them per head dimension, dtype and
causality among precompiled configurations, by measurement. This script does that on the GPU it
runs on, for three tiles:

  forward   keys per K/V tile (32, 64, 128);
  dK/dV     queries per step of the backward's keys-outer kernel (32, 64);
  dQ        keys per K/V tile of the backward's queries-outer kernel (32, 64).

  python -m exact_attention_94_amd.tune build            # compile one library per candidate set
  python -m exact_attention_94_amd.tune measure FILE     # time them on the GPU, results -> FILE
  python -m exact_attention_94_amd.tune write FILE       # write csrc/fa_tune.h from FILE
  python -m exact_attention_94_amd.tune all              # the three in a row (GPU machine)

Each candidate library sets one value for every entry of each table (-DFA_FWD_BC_ALL=...,
-DFA_DKDV_BQ_ALL=..., -DFA_DQ_BC_ALL=...); entries whose tile is not a whole number of 1 KB
direct loads per wave of four (tile * d * 2 bytes a multiple of 4 KB) fall back to 64 inside the
library and are not candidates. For every key (d in 32, 64, 96, 128; f16 and bf16; causal and
not) the workload is B=2, H=16, N=4096 with seeded normal draws: the forward is timed alone, the
backward in full and its dK/dV kernel alone (events the library records around it); dQ's share
is the backward minus the dK/dV kernel (the preprocess is the same in every candidate). After
`write`, rebuild the library (python -m exact_attention_94_amd.build).
"""

from __future__ import annotations

import ctypes
import json
import os
import sys

from . import build as _build

# Candidate sets: forward keys, dK/dV queries, dQ keys.
CANDIDATE_SETS = ((32, 32, 32), (64, 64, 64), (128, 64, 64))
FWD_CANDIDATES = (32, 64, 128)
BWD_CANDIDATES = (32, 64)
HEAD_DIMS = (32, 64, 96, 128)
DTYPES = ("f16", "bf16")
CAUSAL = (False, True)
TUNE_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tuning", "build")
HEADER = os.path.join(_build.CSRC, "fa_tune.h")
RESULTS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tuning", "tiles_mi355x.json")
WORKLOAD = {"B": 2, "H": 16, "N": 4096}


def valid(tile, d):
    """Whole 1 KB direct loads for each of four waves."""
    return (tile * d * 2) % 4096 == 0


def key(d, dtype, causal):
    return f"{d}/{dtype}/{'causal' if causal else 'noncausal'}"


def lib_path(cset):
    return os.path.join(TUNE_DIR, "set_" + "_".join(str(x) for x in cset), "libfa.so")


def build_candidates():
    for cset in CANDIDATE_SETS:
        f, q, k = cset
        flags = [f"-DFA_FWD_BC_ALL={f}", f"-DFA_DKDV_BQ_ALL={q}", f"-DFA_DQ_BC_ALL={k}"]
        out = lib_path(cset)
        os.makedirs(os.path.dirname(out), exist_ok=True)
        _build.build_library(extra_flags=flags, out=out, build_dir=os.path.dirname(out))
        print(f"built {out}", flush=True)


class _Events:
    """hipEvent_t handles from the HIP runtime torch has loaded (the library's runtime)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.rt.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev

    def record(self, ev, stream):
        self.rt.hipEventRecord(ev, stream)

    def ms(self, a, b):
        out = ctypes.c_float()
        self.rt.hipEventSynchronize(b)
        self.rt.hipEventElapsedTime(ctypes.byref(out), a, b)
        return float(out.value)


def _declare(lib):
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp]
    lib.fa_forward.restype = i
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, i,
                                vp, sz, vp]
    lib.fa_backward.restype = i
    lib.fa_backward_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_backward_workspace_bytes.restype = sz
    lib.fa_backward_timed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i,
                                      i, vp, sz, vp, vp, vp]
    lib.fa_backward_timed.restype = i


def _time_key(lib, ev, d, dtype, causal, steps=10, warmup=3):
    """(forward ms, backward ms, dK/dV kernel ms) at the tuning workload."""
    import torch
    B, H, N = WORKLOAD["B"], WORKLOAD["H"], WORKLOAD["N"]
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    code = 2 if dtype == "bf16" else 1
    g = torch.Generator(device=dev)
    g.manual_seed(d)
    q, k, v, do = (torch.randn((B, H, N, d), device=dev, generator=g).to(tdt) for _ in range(4))
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    grads = [torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for _ in range(3)]
    ws = torch.empty(lib.fa_backward_workspace_bytes(B, H, N, d, code, 0), dtype=torch.uint8,
                     device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    c = int(causal)

    def fwd():
        st = lib.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr(), B, H, N, d, d ** -0.5, c, code, 0, stream)
        if st != 0:
            raise RuntimeError(f"fa_forward returned {st}")

    def bwd(ev0=None, ev1=None):
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                lse.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(), B,
                H, N, d, d ** -0.5, c, code, 0, 0, ws.data_ptr(), ws.numel(), stream)
        if ev0 is None:
            st = lib.fa_backward(*args)
        else:  # the same computation, with events around the dK/dV kernel
            st = lib.fa_backward_timed(*args, ev0, ev1)
        if st != 0:
            raise RuntimeError(f"fa_backward returned {st}")

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    e = [[ev.create() for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        ev.record(e[i][0], stream)
        fwd()
        ev.record(e[i][1], stream)
        bwd(e[i][2], e[i][3])
        ev.record(e[i][4], stream)
    torch.cuda.synchronize()
    med = lambda xs: sorted(xs)[len(xs) // 2]  # noqa: E731
    return (med([ev.ms(x[0], x[1]) for x in e]), med([ev.ms(x[1], x[4]) for x in e]),
            med([ev.ms(x[2], x[3]) for x in e]))


def measure(path=RESULTS):
    # torch first: its HIP runtime must be the one the candidate libraries bind to (loading a
    # library first would pull in a second runtime, whose streams torch's are not).
    import torch
    ev = _Events()
    res = {"workload": dict(WORKLOAD, unit="ms, median of 10 calls"),
           "device": torch.cuda.get_device_name(0), "fwd": {}, "dkdv": {}, "dq": {}}
    for cset in CANDIDATE_SETS:
        lib = ctypes.CDLL(lib_path(cset))
        _declare(lib)
        f_keys, q_step, q_keys = cset
        for d in HEAD_DIMS:
            for dtype in DTYPES:
                for causal in CAUSAL:
                    fwd_ms, bwd_ms, dkdv_ms = _time_key(lib, ev, d, dtype, causal)
                    kk = key(d, dtype, causal)
                    if valid(f_keys, d):
                        res["fwd"].setdefault(kk, {})[str(f_keys)] = round(fwd_ms, 5)
                    if valid(q_step, d):
                        res["dkdv"].setdefault(kk, {})[str(q_step)] = round(dkdv_ms, 5)
                    if valid(q_keys, d):
                        res["dq"].setdefault(kk, {})[str(q_keys)] = round(bwd_ms - dkdv_ms, 5)
                    print(json.dumps({"set": cset, "key": kk, "fwd_ms": round(fwd_ms, 4),
                                      "bwd_ms": round(bwd_ms, 4),
                                      "dkdv_ms": round(dkdv_ms, 4)}), flush=True)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(res, fh, indent=1, sort_keys=True)
    return res


def _table_literal(best):
    """C initialiser [head dim][dtype f16, bf16][causal no, yes] from {key: tile}."""
    rows = []
    for d in HEAD_DIMS:
        per_dt = []
        for dtype in DTYPES:
            per_dt.append("{" + ", ".join(str(best[key(d, dtype, c)]) for c in CAUSAL) + "}")
        rows.append("{" + ", ".join(per_dt) + "}")
    return "{" + ", ".join(rows) + "}"


def choose(results):
    """Fastest candidate per table and key (64 where a key has no measurement)."""
    out = {}
    for table in ("fwd", "dkdv", "dq"):
        best = {}
        for d in HEAD_DIMS:
            for dtype in DTYPES:
                for causal in CAUSAL:
                    cand = results.get(table, {}).get(key(d, dtype, causal), {})
                    best[key(d, dtype, causal)] = (int(min(cand.items(), key=lambda kv: kv[1])[0])
                                                   if cand else 64)
        out[table] = best
    return out


def write(path=RESULTS, header=HEADER):
    with open(path) as fh:
        results = json.load(fh)
    best = choose(results)
    with open(header) as fh:
        text = fh.read()
    for table, macro in (("fwd", "FA_FWD_BC_TABLE"), ("dkdv", "FA_DKDV_BQ_TABLE"),
                         ("dq", "FA_DQ_BC_TABLE")):
        start = text.index(f"#define {macro}")
        end = text.index("\n", text.index("}}}", start))
        text = text[:start] + f"#define {macro} {_table_literal(best[table])}" + text[end:]
    with open(header, "w") as fh:
        fh.write(text)
    print(json.dumps({t: best[t] for t in best}))
    return best


def main(argv):
    if not argv or argv[0] not in ("build", "measure", "write", "all"):
        print(__doc__)
        return 2
    cmd = argv[0]
    path = argv[1] if len(argv) > 1 else RESULTS
    if cmd in ("build", "all"):
        build_candidates()
    if cmd in ("measure", "all"):
        measure(path)
    if cmd in ("write", "all"):
        write(path)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
