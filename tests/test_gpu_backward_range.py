"""GPU tests of the backward's operand range handling.

The gradient products use fp16 operands. Upstream gradients far from 1 in size are scaled per
head by a power of two before their fp16 copy is taken (exactly undone in the results), so that
neither dO nor the derived dP and dS underflow or overflow fp16: the gradients keep the same
relative accuracy as for dO ~ N(0, 1). Q, K and V must stay below 65520 in magnitude; with
FA_DEBUG_CHECKS=1 a bf16 call that breaks this returns FA_ERR_RANGE instead of computing with
infinities.
"""

import math
import os

import numpy as np
import pytest

from exact_attention_94_amd import inputs as inp
from oracle import attn_bwd_ref
from tests.gpu_util import host64, max_err, nan_like, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_94_amd as fa_mod
    fa_mod.binding.load()
    return fa_mod


def _inputs(shape, dtype, seed, do_mult):
    rng = np.random.default_rng(seed)
    q, k, v = (inp.quantize(rng.standard_normal(shape, dtype=np.float32), dtype)
               for _ in range(3))
    do = inp.quantize(rng.standard_normal(shape, dtype=np.float32) * np.float32(do_mult), dtype)
    return {"q": q, "k": k, "v": v, "do": do}


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("do_mult", [1e-5, 3e4])
@pytest.mark.parametrize("causal", [False, True])
def test_upstream_gradient_scale(fa, dtype, do_mult, causal):
    """dO ~ 1e-5 N(0,1) (dS would underflow fp16) and dO ~ 3e4 N(0,1) (beyond 65504 for bf16 and
    fp16 would overflow dP): the gradients, divided by the dO multiplier, must meet the usual
    2e-2 bound, i.e. the same accuracy as for dO ~ N(0,1)."""
    import torch
    B, H, N, d = 1, 4, 1024, 64
    if dtype == "f16" and do_mult > 1e4:
        do_mult = 2e3  # fp16 inputs cannot hold 3e4 * N(0,1); 2e3 still overflows dP at s = 0
    t = _inputs((B, H, N, d), dtype, 77 + int(math.log10(do_mult) + 10), do_mult)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (to_device(t[n]) for n in ("q", "k", "v", "do"))
    out = nan_like((B, H, N, d), torch.float32)
    lse = nan_like((B, H, N), torch.float32)
    fa.forward(q, k, v, scale=scale, causal=causal, out=out, lse=lse)
    grads = tuple(nan_like(q.shape, torch.float32) for _ in range(3))
    dq, dk, dv = fa.backward(q, k, v, out, do, lse, scale=scale, causal=causal,
                             grad_dtype=torch.float32, grads=grads)
    torch.cuda.synchronize()
    g = attn_bwd_ref(t["q"].values, t["k"].values, t["v"].values, t["do"].values, scale, causal)
    for name, got in (("dQ", dq), ("dK", dk), ("dV", dv)):
        ref = g[name.lower()]
        e = max_err(host64(got), ref) / do_mult
        rel = max_err(host64(got), ref) / np.abs(ref).max()
        print(f"    {name}: max_abs_err / mult = {e:.3e}, relative to max |ref| {rel:.3e}",
              flush=True)
        assert e <= 2e-2, f"{name}: {e:.3e}"


def test_scale_is_exact_for_ordinary_gradients(fa):
    """A dO whose largest magnitude is 12 is used as it is (12 lies in [1/2, 16]); the same dO
    times 2^-20 is scaled back by 2^20 into exactly the same fp16 operands, so every gradient is
    exactly 2^-20 times the first (the per-head scale only moves exponents)."""
    import torch
    B, H, N, d = 1, 2, 300, 64
    t = _inputs((B, H, N, d), "bf16", 5, 1.0)
    x = t["do"].values
    t["do"] = inp.quantize(x * np.float32(12.0 / np.abs(x).max()), "bf16")
    assert np.abs(t["do"].values).max() == 12.0
    q, k, v, do = (to_device(t[n]) for n in ("q", "k", "v", "do"))
    out, lse = fa.forward(q, k, v, causal=True, o_dtype=torch.float32)
    g1 = fa.backward(q, k, v, out, do, lse, causal=True, grad_dtype=torch.float32)
    g2 = fa.backward(q, k, v, out, (do.float() * 2.0 ** -20).to(torch.bfloat16), lse,
                     causal=True, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for x, y in zip(g1, g2):
        assert torch.equal(x * 2.0 ** -20, y)


@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_debug_range_check(fa, which):
    """FA_DEBUG_CHECKS=1: a bf16 input of 70000 (beyond fp16) makes the backward return
    FA_ERR_RANGE; the same call on in-range inputs runs and gives the same result as without the
    check; without the flag no check runs."""
    import torch
    B, H, N, d = 1, 2, 200, 64
    t = _inputs((B, H, N, d), "bf16", 9, 1.0)
    x = {n: to_device(t[n]) for n in ("q", "k", "v", "do")}
    out, lse = fa.forward(x["q"], x["k"], x["v"], causal=True, o_dtype=torch.float32)
    ref = fa.backward(x["q"], x["k"], x["v"], out, x["do"], lse, causal=True,
                      grad_dtype=torch.float32)
    saved = os.environ.get("FA_DEBUG_CHECKS")
    try:
        os.environ["FA_DEBUG_CHECKS"] = "1"
        same = fa.backward(x["q"], x["k"], x["v"], out, x["do"], lse, causal=True,
                           grad_dtype=torch.float32)
        torch.cuda.synchronize()
        for a, b in zip(ref, same):
            assert torch.equal(a, b)
        bad = x[which].clone()
        bad[0, 1, 17, 5] = 70000.0
        args = {**x, which: bad}
        with pytest.raises(fa.FAError) as exc:
            fa.backward(args["q"], args["k"], args["v"], out, args["do"], lse, causal=True,
                        grad_dtype=torch.float32)
        assert exc.value.status == fa.FA_ERR_RANGE
        bad[0, 1, 17, 5] = float("inf")
        with pytest.raises(fa.FAError) as exc:
            fa.backward(args["q"], args["k"], args["v"], out, args["do"], lse, causal=True,
                        grad_dtype=torch.float32)
        assert exc.value.status == fa.FA_ERR_RANGE
        os.environ["FA_DEBUG_CHECKS"] = "0"
        fa.backward(args["q"], args["k"], args["v"], out, args["do"], lse, causal=True,
                    grad_dtype=torch.float32)  # no check: runs (its result is unspecified)
        torch.cuda.synchronize()
    finally:
        if saved is None:
            os.environ.pop("FA_DEBUG_CHECKS", None)
        else:
            os.environ["FA_DEBUG_CHECKS"] = saved
