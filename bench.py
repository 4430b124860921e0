#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = fa_forward + fa_backward over the headline workload (B=2, H=16, N=4096, d=64, causal,
bf16 inputs; O and the gradients in fp32), inputs resident in HBM before timing starts.
Prints ONE JSON line with the step throughput, the forward and backward TFLOP/s and their share of
the MI355X dense bf16/fp16 MFMA peak, a roofline record for the dominant kernel (the backward's
dK/dV kernel, timed alone with HIP events that the library records around its launch), and the
float64 CPU oracle timed on a bounded sample of the same workload on this host.

FLOP convention: forward 4*B*H*N^2*d, halved when causal (two N x N x d products); backward 2.5x
the forward (five products). The dK/dV kernel performs four products (S, dP, dV, dK), i.e. 2x
the forward's FLOPs; the dQ kernel recomputes S and dP and forms dQ (three products), work the
backward figure above does not count.

The line also carries the same step with dropout p = 0.1 ("dropout"), with a block-sparse mask
("blocksparse": forward and backward times and the rate over the visited blocks), and split-KV
decoding of a long bf16 K/V cache ("decode": HBM bytes per second against the 8 TB/s peak); none
of them is part of the headline value.

Before timing, W warm-up steps run and then untimed steps continue for --settle-ms (default
500 ms): the first tens of milliseconds of load from idle run ~15% slower than the steady state.
Each of the secondary timings below first repeats its own calls untimed for about 150 ms, for the
same reason (a small workload right after a different one otherwise reads up to ~50% slow).

Next to the mean step time the line gives the median and minimum of the per-step times of the
breakdown loop, the mean step time with the caches flushed before each step (cold_step_ms), and
the shader clock the driver reports after the timing (gpu_sclk_mhz, read from sysfs in-process).

The line also carries ("workloads") the forward and backward rates of the other named workloads:
B=4 H=16 N=1024 d=64 (causal and not), B=1 H=32 N=8192 d=128 with peaked rows, and the
B=1 H=8 N=32768 d=128 causal forward.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--no-cpu-baseline]
                       [--no-dropout] [--no-blocksparse] [--no-decode] [--no-workloads]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
HBM_PEAK_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOP/s + % bf16 MFMA peak (B2 H16 N4096 d64 causal)"
WORKLOAD = "b2h16n4k_d64"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_dkdv_b2h16n4k_d64_traffic.txt")
KERNEL_SOURCES = tuple(os.path.join(ROOT, "exact_attention_94_amd", "csrc", f)
                       for f in ("fa_bwd.hip", "fa_device.h", "fa_kernels.h", "fa_tune.h"))


def flops(w):
    fwd = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if True in w.causal else 1.0)
    return fwd, 2.5 * fwd


class HipEvents:
    """hipEvent_t handles through the HIP runtime already loaded by torch."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.rt.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def record(self, ev, stream):
        if self.rt.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        out = ctypes.c_float()
        self.rt.hipEventSynchronize(b)
        if self.rt.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def destroy(self, ev):
        self.rt.hipEventDestroy(ev)


def source_digest(paths=KERNEL_SOURCES):
    """Digest of the code (comments and blank lines dropped) of the sources the dK/dV kernel is
    built from: a comment edit keeps the measured traffic valid, a code change voids it."""
    h = hashlib.sha256()
    for path in paths:
        for line in open(path, encoding="utf-8"):
            code = re.sub(r"//.*", "", line).strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dK/dV kernel from the committed rocprofv3 counter summary, or
    None when it is absent or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE, encoding="utf-8").read()
    m_src = re.search(r"^kernel_source_sha256_16:\s*(\w+)", text, re.M)
    m_tot = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not (m_src and m_tot) or m_src.group(1) != source_digest():
        return None
    return float(m_tot.group(1))


def cpu_model():
    """CPU model name of this host, read from /proc/cpuinfo (no child process)."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def best_of(fn, repeats=3):
    """Best wall time of `repeats` calls of fn, by time.perf_counter (the pages' own timing
    method: best of three runs)."""
    best = float("inf")
    for _ in range(repeats):
        t0 = time.perf_counter()
        fn()
        best = min(best, time.perf_counter() - t0)
    return best


def cpu_baseline(w, t, heads=2, repeats=3):
    """The float64 NumPy oracle timed on this host's cores, best of `repeats` per measurement.

    Configurations 1-4 of the named workloads: the forward alone and forward+backward (configs
    3 and 4 have a backward; configs 1 and 2 are timed on the forward only), each on a fixed
    sample of heads and scaled to the whole batch by the head count (every head does the same
    work). Configuration 5 (N=32768) is a per-row extrapolation: the oracle's per-row forward
    timed on the seeded row subset of one head, times B*H*N rows, labelled as such. The headline
    `value` is configuration 3 (this bench's workload), forward+backward, in TFLOP/s of the
    nominal FLOPs."""
    from exact_attention_94_amd import inputs as inp
    from oracle import attn_bwd_ref, attn_fwd_ref, attn_rows_ref
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        threads = None

    def fl(wl, causal):
        return 4.0 * wl.B * wl.H * wl.N * wl.N * wl.d * (0.5 if causal else 1.0)

    def sample(wl, n_heads, tens):
        sel = []
        for hh in range(min(n_heads, wl.B * wl.H)):
            b, h = divmod(hh, wl.H)
            sel.append({k: tens[k].values[b, h] for k in tens})
        return sel

    configs = {}
    t_start = time.perf_counter()
    plan = (("single_head_f32", 1, False), ("b4h16n1k_d64", 4, False),
            ("b2h16n4k_d64", heads, True), ("b1h32n8k_d128_peaked", 1, True))
    for name, n_heads, with_bwd in plan:
        wl = inp.WORKLOADS[name]
        tens = t if name == WORKLOAD else inp.workload_inputs(wl)
        sel = sample(wl, n_heads, tens)
        scale_to_all = (wl.B * wl.H) / len(sel)
        for causal in wl.causal:
            def fwd():
                for x in sel:
                    attn_fwd_ref(x["q"], x["k"], x["v"], wl.scale, causal)

            def fwd_bwd():
                for x in sel:
                    attn_fwd_ref(x["q"], x["k"], x["v"], wl.scale, causal)
                    attn_bwd_ref(x["q"], x["k"], x["v"], x["do"], wl.scale, causal)

            f_fwd = fl(wl, causal)
            t_f = best_of(fwd, repeats) * scale_to_all
            row = {"heads_timed": len(sel), "fwd_s": round(t_f, 4),
                   "fwd_tflops": round(f_fwd / t_f / 1e12, 6)}
            if with_bwd:
                t_fb = best_of(fwd_bwd, repeats) * scale_to_all
                row.update({"fwd_bwd_s": round(t_fb, 4),
                            "fwd_bwd_tflops": round(3.5 * f_fwd / t_fb / 1e12, 6)})
            configs[f"{name} {'causal' if causal else 'non-causal'}"] = row

    # Configuration 5: per-row oracle on the seeded subset of head 0, extrapolated to every row.
    wl = inp.WORKLOADS["b1h8n32k_d128"]
    t5_in = inp.workload_inputs(wl)
    q1, k1, v1 = (t5_in[n].values[0, 0] for n in ("q", "k", "v"))
    del t5_in
    rows = inp.subset_rows(wl.N, 0)
    t_rows = best_of(lambda: attn_rows_ref(q1, k1, v1, wl.scale, True, rows), repeats)
    # Causal row i costs in proportion to its i + 1 keys: scale by the keys of all rows over the
    # keys of the sampled rows.
    keys_all = wl.B * wl.H * wl.N * (wl.N + 1) / 2.0
    keys_rows = float(sum(r + 1 for r in rows))
    t5 = t_rows * keys_all / keys_rows
    configs["b1h8n32k_d128 causal (extrapolated)"] = {
        "rows_timed": len(rows), "rows_s": round(t_rows, 4), "fwd_s": round(t5, 2),
        "fwd_tflops": round(fl(wl, True) / t5 / 1e12, 6),
        "note": "per-row forward on 64 seeded rows of one head, scaled by the causal key count "
                "of all B*H*N rows: an extrapolation, not a full run"}
    head = configs[f"{WORKLOAD} causal"]
    total = time.perf_counter() - t_start
    return {"value": head["fwd_bwd_tflops"], "unit": "TFLOP/s",
            "cores": threads or os.cpu_count(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"float64 NumPy oracle, best of {repeats} (time.perf_counter); headline: "
                      f"forward+backward of {min(heads, w.B * w.H)} of the {w.B * w.H} heads of "
                      f"B={w.B} H={w.H} N={w.N} d={w.d} causal, scaled to all heads (nominal "
                      f"FLOPs / time); {total:.1f} s of CPU timing in all",
            "configs": configs}


def settle(fn, ms=150.0, batch=10, cap=3000):
    """Untimed calls of fn for about `ms` milliseconds before a timed loop: the first tens of
    milliseconds of a new load run slower (clocks and power ramp up), as before the headline."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms and n < cap:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        n += batch
    return n


def time_dropout(fa, ev, stream, w, q, k, v, do, o, lse, grads, ws, steps, p=0.1):
    """The same step with dropout (keep mask regenerated from seed and offset in every kernel):
    forward and backward times, reported beside the headline (which has no dropout)."""
    import torch
    f_fwd, f_bwd = flops(w)

    def fwd(i):
        fa.forward(q, k, v, scale=w.scale, causal=True, out=o, lse=lse, dropout_p=p, seed=77,
                   offset=i)

    def bwd(i):
        fa.backward(q, k, v, o, do, lse, scale=w.scale, causal=True, grad_dtype=torch.float32,
                    workspace=ws, grads=grads, dropout_p=p, seed=77, offset=i)

    for i in range(2):
        fwd(i)
        bwd(i)
    torch.cuda.synchronize()
    settle(lambda: (fwd(0), bwd(0)))
    e = [[ev.create() for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        ev.record(e[i][0], stream)
        fwd(i)
        ev.record(e[i][1], stream)
        bwd(i)
        ev.record(e[i][2], stream)
    torch.cuda.synchronize()
    fwd_ms = sum(ev.ms(x[0], x[1]) for x in e) / steps
    bwd_ms = sum(ev.ms(x[1], x[2]) for x in e) / steps
    for x in e:
        for y in x:
            ev.destroy(y)
    return {"p": p, "steps": steps, "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
            "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2)}


def local_global_mask(n_blocks):
    """Sliding window of two 128-blocks (own and previous) plus global block 0 per query block."""
    import numpy as np
    m = np.zeros((n_blocks, n_blocks), dtype=np.uint8)
    for qb in range(n_blocks):
        m[qb, max(0, qb - 1):qb + 1] = 1
        m[qb, 0] = 1
    return m


def time_blocksparse(fa, ev, stream, w, q, k, v, do, o, lse, grads, ws, steps):
    """The same step with a block-sparse mask (local window + global block, 128 x 128 blocks, on
    top of the causal rule). FLOPs count only the visited blocks (diagonal blocks at half, as the
    causal convention does), so the rates compare with the dense figures."""
    import numpy as np
    import torch
    nb = (w.N + 127) // 128
    m = local_global_mask(nb)
    live = np.tril(m)  # causal: blocks above the diagonal are never visited
    diag = np.trace(live)
    eff_blocks = float(live.sum() - diag) + 0.5 * diag
    f_fwd = 4.0 * w.B * w.H * 128 * 128 * w.d * eff_blocks
    f_bwd = 2.5 * f_fwd
    mask_t = torch.from_numpy(m).to(q.device)

    def fwd():
        fa.forward(q, k, v, scale=w.scale, causal=True, out=o, lse=lse, block_mask=mask_t)

    def bwd():
        fa.backward(q, k, v, o, do, lse, scale=w.scale, causal=True, grad_dtype=torch.float32,
                    workspace=ws, grads=grads, block_mask=mask_t)

    for _ in range(2):
        fwd()
        bwd()
    torch.cuda.synchronize()
    settle(lambda: (fwd(), bwd()))
    e = [[ev.create() for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        ev.record(e[i][0], stream)
        fwd()
        ev.record(e[i][1], stream)
        bwd()
        ev.record(e[i][2], stream)
    torch.cuda.synchronize()
    fwd_ms = sum(ev.ms(x[0], x[1]) for x in e) / steps
    bwd_ms = sum(ev.ms(x[1], x[2]) for x in e) / steps
    for x in e:
        for y in x:
            ev.destroy(y)
    return {"pattern": "window of 2 blocks + global block 0, 128x128 blocks, causal",
            "live_block_fraction": round(float(live.sum()) / (nb * (nb + 1) / 2), 4),
            "steps": steps, "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
            "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2)}


def time_cold(ev, stream, dev, step, steps):
    """Mean step time with the caches flushed before every step: a 512 MiB buffer is written
    between steps (outside the timed events), so the inputs start in HBM rather than in the
    256 MB last-level cache."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    total = 0.0
    for _ in range(steps):
        flush.fill_(1)
        e0, e1 = ev.create(), ev.create()
        ev.record(e0, stream)
        step()
        ev.record(e1, stream)
        torch.cuda.synchronize()
        total += ev.ms(e0, e1)
        ev.destroy(e0)
        ev.destroy(e1)
    return total / steps


def gpu_clock_mhz():
    """Current shader clock of the first GPU, read in-process from the amdgpu driver's sysfs
    table (the line marked '*' of pp_dpm_sclk); None where that file is not readable. No child
    process is started: under a profiler that preloads itself into every process, starting one
    would run a second GPU-initialising program."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path, encoding="utf-8") as fh:
                for line in fh:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*Mhz", line, re.I)
                        if m:
                            return int(m.group(1))
        except OSError:
            continue
    return None


def time_workloads(fa, ev, stream, dev, steps):
    """The other named workloads, timed the same way (a settle phase, then one event pair around
    `steps` back-to-back calls): B=4 H=16 N=1024 d=64 forward, causal and not (O in bf16);
    B=1 H=32 N=8192 d=128 with
    Q and K scaled by 2 (peaked rows), forward (fp32 O) and backward (fp32 gradients), causal;
    B=1 H=8 N=32768 d=128 causal forward (O in bf16). Inputs are normal draws of the workloads'
    shapes; FLOPs follow the headline convention."""
    import torch
    out = {}

    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        settle(fn)
        e0, e1 = ev.create(), ev.create()
        ev.record(e0, stream)
        for _ in range(n):
            fn()
        ev.record(e1, stream)
        torch.cuda.synchronize()
        ms = ev.ms(e0, e1) / n
        ev.destroy(e0)
        ev.destroy(e1)
        return ms

    def rate(f, ms):
        return {"ms": round(ms, 4), "tflops": round(f / (ms * 1e-3) / 1e12, 2),
                "pct_peak": round(100 * f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}

    g = torch.Generator(device=dev)
    g.manual_seed(1024)
    B, H, N, d = 4, 16, 1024, 64
    q, k, v = (torch.randn((B, H, N, d), device=dev, generator=g).to(torch.bfloat16)
               for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    f = 4.0 * B * H * N * N * d
    row = {}
    for causal in (True, False):
        ms = timed(lambda: fa.forward(q, k, v, scale=d ** -0.5, causal=causal, out=o, lse=lse),
                   steps)
        row["fwd_causal" if causal else "fwd_noncausal"] = rate(f * (0.5 if causal else 1.0), ms)
    out["B=4 H=16 N=1024 d=64 bf16"] = row
    del q, k, v, o, lse

    g.manual_seed(8192)
    B, H, N, d = 1, 32, 8192, 128
    q, k = ((2.0 * torch.randn((B, H, N, d), device=dev, generator=g)).to(torch.bfloat16)
            for _ in range(2))
    v, do = (torch.randn((B, H, N, d), device=dev, generator=g).to(torch.bfloat16)
             for _ in range(2))
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(fa.workspace_bytes(B, H, N, d, fa.FA_BF16, fa.FA_F32), dtype=torch.uint8,
                     device=dev)
    f = 4.0 * B * H * N * N * d * 0.5
    n = max(2, steps // 2)
    ms_f = timed(lambda: fa.forward(q, k, v, scale=d ** -0.5, causal=True, out=o, lse=lse), n)
    ms_b = timed(lambda: fa.backward(q, k, v, o, do, lse, scale=d ** -0.5, causal=True,
                                     grad_dtype=torch.float32, workspace=ws, grads=grads), n)
    out["B=1 H=32 N=8192 d=128 bf16 causal, Q and K x2"] = {"fwd": rate(f, ms_f),
                                                             "bwd": rate(2.5 * f, ms_b)}
    del q, k, v, do, o, lse, grads, ws

    g.manual_seed(32768)
    B, H, N, d = 1, 8, 32768, 128
    q, k, v = (torch.randn((B, H, N, d), device=dev, generator=g).to(torch.bfloat16)
               for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    f = 4.0 * B * H * N * N * d * 0.5
    ms = timed(lambda: fa.forward(q, k, v, scale=d ** -0.5, causal=True, out=o, lse=lse), n)
    out["B=1 H=8 N=32768 d=128 bf16 causal"] = {"fwd": rate(f, ms)}
    return out


def time_decode(fa, ev, stream, dev, steps, B=4, H=32, nk=16384, d=128):
    """Split-KV decoding of one query row per sequence against a bf16 K/V cache of nk keys:
    HBM-bound, so the rate is bytes moved (K, V, Q read once, O and LSE written) per second
    against the 8 TB/s HBM peak. The cache (537 MB here) exceeds the 256 MB last-level cache."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(nk)
    k = torch.randn((B, H, nk, d), device=dev, generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, nk, d), device=dev, generator=g).to(torch.bfloat16)
    q = torch.randn((B, H, 1, d), device=dev, generator=g).to(torch.bfloat16)
    out = torch.empty((B, H, 1, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, 1), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(B, H, 1, nk, d), dtype=torch.uint8, device=dev)
    for _ in range(3):
        fa.decode(q, k, v, causal=True, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    settle(lambda: fa.decode(q, k, v, causal=True, out=out, lse=lse, workspace=ws))
    e0, e1 = ev.create(), ev.create()
    ev.record(e0, stream)
    for _ in range(steps):
        fa.decode(q, k, v, causal=True, out=out, lse=lse, workspace=ws)
    ev.record(e1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(e0, e1) / steps
    ev.destroy(e0)
    ev.destroy(e1)
    nbytes = 2 * B * H * nk * d * 2 + B * H * d * 2 * 2 + B * H * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"B={B} H={H} Nq=1 Nk={nk} d={d} bf16 causal", "steps": steps,
            "ms": round(ms, 4), "bytes": nbytes, "achieved_GBs": round(gbs, 1),
            "hbm_peak_GBs": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="after the warm-up steps, keep running untimed steps for this long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=2,
                    help="heads of the headline workload timed on the CPU oracle (scaled to all)")
    ap.add_argument("--no-dropout", action="store_true",
                    help="skip the extra timing of the dropout path (p = 0.1)")
    ap.add_argument("--no-blocksparse", action="store_true",
                    help="skip the extra timing of the block-sparse path")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the extra timing of split-KV decoding")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the timing of the other named workloads (N=1024, 8192, 32768)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the attention "
              "path runs on a single GPU (heads would shard across GPUs with no communication, "
              "but no multi-GPU path is provided)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import exact_attention_94_amd as fa
    from exact_attention_94_amd import inputs as inp

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    fa.binding.load()
    dev = torch.device("cuda:0")

    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 3}))
        return 0

    w = inp.WORKLOADS[WORKLOAD]
    t = inp.workload_inputs(w)

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x.bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    q, k, v, do = (up(t[n]) for n in ("q", "k", "v", "do"))
    shape = (w.B, w.H, w.N, w.d)
    o = torch.empty(shape, dtype=torch.float32, device=dev)
    lse = torch.empty(shape[:3], dtype=torch.float32, device=dev)
    grads = tuple(torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(fa.workspace_bytes(*shape, fa.FA_BF16, fa.FA_F32), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step():
        fa.forward(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
        fa.backward(q, k, v, o, do, lse, scale=w.scale, causal=True, grad_dtype=torch.float32,
                    workspace=ws, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Settle: the first tens of milliseconds of sustained load run ~15% slower (clocks and power
    # state still ramping from idle), so untimed steps continue until the GPU has been busy for
    # at least --settle-ms.
    t_settle = time.perf_counter()
    settle_steps = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms and settle_steps < 5000:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        settle_steps += 10

    ev = HipEvents()
    K = args.steps
    e_start, e_end = ev.create(), ev.create()

    # Headline: K whole steps back to back, bracketed by one event pair and nothing inside.
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    ev.record(e_start, stream)
    for _ in range(K):
        step()
    ev.record(e_end, stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    step_ms = ev.ms(e_start, e_end) / K

    # Breakdown: the same steps with events between the passes and around the dK/dV launch
    # (each event adds a queue packet, so these times carry a little overhead of their own).
    ef0 = [ev.create() for _ in range(K)]
    ef1 = [ev.create() for _ in range(K)]
    eb0 = [ev.create() for _ in range(K)]
    eb1 = [ev.create() for _ in range(K)]
    eb2 = [ev.create() for _ in range(K)]

    torch.cuda.synchronize()
    for i in range(K):
        ev.record(ef0[i], stream)
        fa.forward(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
        ev.record(ef1[i], stream)
        fa.backward(q, k, v, o, do, lse, scale=w.scale, causal=True, grad_dtype=torch.float32,
                    workspace=ws, grads=grads, main_events=(eb0[i], eb1[i]))
        ev.record(eb2[i], stream)
    torch.cuda.synchronize()

    fwd_ms = sum(ev.ms(ef0[i], ef1[i]) for i in range(K)) / K
    bwd_ms = sum(ev.ms(ef1[i], eb2[i]) for i in range(K)) / K
    main_ms = sum(ev.ms(eb0[i], eb1[i]) for i in range(K)) / K
    per_step = sorted(ev.ms(ef0[i], eb2[i]) for i in range(K))
    step_median_ms = per_step[K // 2] if K % 2 else 0.5 * (per_step[K // 2 - 1] + per_step[K // 2])
    step_min_ms = per_step[0]
    for e in [e_start, e_end] + ef0 + ef1 + eb0 + eb1 + eb2:
        ev.destroy(e)
    assert torch.isfinite(o).all() and all(torch.isfinite(g).all() for g in grads)

    f_fwd, f_bwd = flops(w)
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12  # noqa: E731
    value = tf(f_fwd + f_bwd, step_ms)
    f_dkdv = 2.0 * f_fwd  # S, dP, dV, dK
    main_tf = tf(f_dkdv, main_ms)
    traffic = measured_traffic()
    cold = time_cold(ev, stream, dev, step, steps=min(K, 10))
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "B=2 H=16 N=4096 d=64 causal, bf16 inputs, forward+backward",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": True,
                   "o_dtype": "f32", "grad_dtype": "f32", "bwd_mfma_operands": "f16",
                   "seed": w.N, "parallelism": "single GPU"},
        "fwd_tflops": round(tf(f_fwd, fwd_ms), 2),
        "fwd_pct_peak": round(100 * tf(f_fwd, fwd_ms) / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(fwd_ms, 4),
        "bwd_tflops": round(tf(f_bwd, bwd_ms), 2),
        "bwd_pct_peak": round(100 * tf(f_bwd, bwd_ms) / PEAK_BF16_TFLOPS, 2),
        "bwd_ms": round(bwd_ms, 4),
        "step_pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "host_wall_ms_per_step": round(1e3 * t_wall / K, 4),
        "step_ms_median": round(step_median_ms, 4),
        "step_ms_min": round(step_min_ms, 4),
        "cold_step_ms": round(cold, 4),
        "gpu_sclk_mhz": gpu_clock_mhz(),
        "roofline": {
            "kernel": "bwd_dkdv_kernel<64, bf16, f32 grads, causal>",
            "bound": "mfma",
            "achieved": round(main_tf, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(main_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel_ms": round(main_ms, 4),
            "flops_per_launch": f_dkdv,
        },
    }
    if not args.no_dropout:
        out["dropout"] = time_dropout(fa, ev, stream, w, q, k, v, do, o, lse, grads, ws,
                                      steps=min(K, 10))
    if not args.no_blocksparse:
        out["blocksparse"] = time_blocksparse(fa, ev, stream, w, q, k, v, do, o, lse, grads, ws,
                                              steps=min(K, 10))
    if not args.no_decode:
        out["decode"] = time_decode(fa, ev, stream, dev, steps=min(K, 20))
    if not args.no_workloads:
        out["workloads"] = time_workloads(fa, ev, stream, dev, steps=min(K, 10))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, t, heads=args.cpu_heads)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
