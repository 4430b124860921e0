"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it draws random tensors, rounds them to the storage
dtype and describes the workloads. Both the HIP path and the float64 oracle receive exactly the
values produced here.

Recipe: numpy ``default_rng(seed)`` float32 ``standard_normal`` draws, one whole [B,H,N,d]
tensor at a time, in the order Q, K, V, dO (the pages seed their examples with
``default_rng(N)``, so the default seed is N). Optional power-of-two multipliers on Q and K
(exact in every dtype) make the softmax rows peaked. The float32 values are then rounded to the
storage dtype with round-to-nearest-even.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Inputs must be finite (the generators only produce finite values).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensor:
    """One input tensor: `values` (float32, exact) and `bits` (the storage bytes for upload)."""

    values: np.ndarray
    bits: np.ndarray  # uint16 for f16/bf16, float32 for f32
    dtype: str


def quantize(x32, dtype):
    """Round a float32 array to `dtype` storage; returns a Tensor with exact float32 values."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f32":
        return Tensor(x32, x32, dtype)
    if dtype == "f16":
        h = x32.astype(np.float16)  # IEEE RNE
        return Tensor(h.astype(np.float32), h.view(np.uint16), dtype)
    if dtype == "bf16":
        b = f32_to_bf16_bits(x32)
        return Tensor(bf16_bits_to_f32(b), b, dtype)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class Workload:
    """A named attention workload (shapes, dtype, masking, value recipe)."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: tuple
    backward: bool = False
    qk_mult: float = 1.0
    row_subset: bool = False
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def scale(self):
        return 1.0 / float(np.sqrt(self.d))

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


WORKLOADS = {
    "single_head_f32": Workload("single_head_f32", 1, 1, 256, 64, "f32", (False,),
                                note="single-head fp32 forward, non-causal"),
    "b4h16n1k_d64": Workload("b4h16n1k_d64", 4, 16, 1024, 64, "bf16", (True, False),
                             note="bf16 forward, causal and non-causal share inputs"),
    "b2h16n4k_d64": Workload("b2h16n4k_d64", 2, 16, 4096, 64, "bf16", (True,), backward=True,
                             note="bf16 causal forward + backward (headline workload)"),
    "b1h32n8k_d128_peaked": Workload("b1h32n8k_d128_peaked", 1, 32, 8192, 128, "bf16", (True,),
                                     backward=True, qk_mult=2.0,
                                     note="bf16 causal fwd+bwd, Q and K scaled by 2 (peaked rows)"),
    "b1h8n32k_d128": Workload("b1h8n32k_d128", 1, 8, 32768, 128, "bf16", (True,),
                              row_subset=True,
                              note="long-sequence causal forward, checked on a row subset"),
}


def draw(shape, dtype, seed, qk_mult=1.0, with_do=False):
    """Draw Q, K, V (and dO) from default_rng(seed) in that order and round to `dtype`.

    Returns a dict of Tensor objects keyed "q", "k", "v" (and "do").
    """
    rng = np.random.default_rng(seed)
    out = {}
    for name in ("q", "k", "v") + (("do",) if with_do else ()):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if name in ("q", "k") and qk_mult != 1.0:
            x = x * np.float32(qk_mult)
        out[name] = quantize(x, dtype)
    return out


def workload_inputs(w: Workload, seed=None):
    """The inputs of a named workload (seed defaults to N, the pages' convention)."""
    return draw(w.shape, w.dtype, w.N if seed is None else seed, w.qk_mult, with_do=w.backward)


def subset_rows(N, head, count=64):
    """Query rows checked per head for a workload whose full oracle is too slow.

    Fixed rows cover both ends and tile boundaries; the rest are drawn without replacement
    from default_rng(N + 1 + head).
    """
    fixed = [r for r in (0, 1, 63, 64, 127, 128, 255, 256, N - 2, N - 1) if 0 <= r < N]
    fixed = sorted(set(fixed))
    rest = [r for r in range(N) if r not in set(fixed)]
    need = max(0, min(count, N) - len(fixed))
    pick = np.random.default_rng(N + 1 + head).choice(len(rest), size=need, replace=False)
    return sorted(fixed + [rest[i] for i in pick])
