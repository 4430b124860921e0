"""GPU parity of dropout (fa_forward_dropout / fa_backward_dropout) against the float64 oracle.

The oracle builds the keep mask from the same (p, seed, offset) with its own Philox-4x32-10;
any disagreement in a single mask bit moves an output by about |v| and fails the comparison.
Tolerances as for the plain path: 2e-2 on O / dQ / dK / dV and 1e-3 on LSE (16-bit inputs).
"""

import math

import numpy as np
import pytest

from exact_attention_94_amd import inputs as inp
from oracle import attn_bwd_ref, attn_fwd_ref, dropout_keep_ref, keep_scale
from tests.gpu_util import check, host64, nan_like, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_94_amd as fa_mod
    fa_mod.binding.load()
    return fa_mod


def _mask(B, H, N, seed, offset, p, heads=None):
    m = np.empty((B, H, N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            if heads is None or (b, h) in heads:
                m[b, h] = dropout_keep_ref(N, N, b * H + h, seed, offset, p)
    return m


def _fwd_bwd(fa, t, causal, scale, p, seed, offset, o_f32=True):
    import torch
    q, k, v, do = (to_device(t[n]) for n in ("q", "k", "v", "do"))
    od = torch.float32 if o_f32 else q.dtype
    out = nan_like(q.shape, od)
    lse = nan_like(q.shape[:3], torch.float32)
    fa.forward(q, k, v, scale=scale, causal=causal, out=out, lse=lse, dropout_p=p, seed=seed,
               offset=offset)
    grads = tuple(nan_like(q.shape, torch.float32) for _ in range(3))
    fa.backward(q, k, v, out, do, lse, scale=scale, causal=causal, grad_dtype=torch.float32,
                grads=grads, dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    return out, lse, grads


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_sweep(fa, dtype, d, causal):
    p, seed, offset = 0.2, 0x1234_5678_9ABC_DEF0, 3
    ks = keep_scale(p)
    for n in [1, 17, 64, 65, 129, 300]:
        for (B, H) in ((1, 2), (2, 3)):
            print(f"  N={n} B={B} H={H}", flush=True)
            t = inp.draw((B, H, n, d), dtype, n * 13 + d, with_do=True)
            scale = 1.0 / math.sqrt(d)
            out, lse, (dq, dk, dv) = _fwd_bwd(fa, t, causal, scale, p, seed, offset)
            keep = _mask(B, H, n, seed, offset, p)
            o_ref, l_ref = attn_fwd_ref(t["q"].values, t["k"].values, t["v"].values, scale,
                                        causal, keep=keep, keep_scale=ks)
            g = attn_bwd_ref(t["q"].values, t["k"].values, t["v"].values, t["do"].values, scale,
                             causal, keep=keep, keep_scale=ks)
            check("O", host64(out), o_ref, 2e-2)
            check("LSE", host64(lse), l_ref, 1e-3)
            check("dQ", host64(dq), g["dq"], 2e-2)
            check("dK", host64(dk), g["dk"], 2e-2)
            check("dV", host64(dv), g["dv"], 2e-2)


def test_dropout_p0_is_bitwise_the_plain_path(fa):
    import torch
    t = inp.draw((2, 2, 333, 64), "bf16", 8, with_do=True)
    q, k, v, do = (to_device(t[n]) for n in ("q", "k", "v", "do"))
    o0, l0 = fa.forward(q, k, v, causal=True, o_dtype=torch.float32)
    o1, l1 = fa.forward(q, k, v, causal=True, o_dtype=torch.float32, dropout_p=0.0, seed=5)
    g0 = fa.backward(q, k, v, o0, do, l0, causal=True, grad_dtype=torch.float32)
    g1 = fa.backward(q, k, v, o1, do, l1, causal=True, grad_dtype=torch.float32, dropout_p=0.0,
                     seed=5)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for x, y in zip(g0, g1):
        assert torch.equal(x, y)


def test_dropout_seed_and_offset_select_the_mask(fa):
    import torch
    t = inp.draw((1, 2, 256, 64), "f16", 21)
    q, k, v = (to_device(t[n]) for n in ("q", "k", "v"))
    outs = {}
    for key in ((1, 0), (1, 0), (2, 0), (1, 1)):
        o, _ = fa.forward(q, k, v, causal=False, dropout_p=0.3, seed=key[0], offset=key[1])
        torch.cuda.synchronize()
        outs.setdefault(key, []).append(o.clone())
    assert torch.equal(outs[(1, 0)][0], outs[(1, 0)][1])
    assert not torch.equal(outs[(1, 0)][0], outs[(2, 0)][0])
    assert not torch.equal(outs[(1, 0)][0], outs[(1, 1)][0])


def test_dropout_b2h16n4k_sampled_heads(fa):
    """The benchmark workload's shape with p = 0.1, checked on two whole heads."""
    w = inp.WORKLOADS["b2h16n4k_d64"]
    t = inp.workload_inputs(w)
    p, seed, offset = 0.1, 2024, 7
    out, lse, (dq, dk, dv) = _fwd_bwd(fa, t, True, w.scale, p, seed, offset)
    ks = keep_scale(p)
    for (b, h) in ((0, 5), (1, 12)):
        keep = dropout_keep_ref(w.N, w.N, b * w.H + h, seed, offset, p)
        sel = lambda x: x[b, h]  # noqa: E731
        o_ref, l_ref = attn_fwd_ref(sel(t["q"].values), sel(t["k"].values), sel(t["v"].values),
                                    w.scale, True, keep=keep, keep_scale=ks)
        g = attn_bwd_ref(sel(t["q"].values), sel(t["k"].values), sel(t["v"].values),
                         sel(t["do"].values), w.scale, True, keep=keep, keep_scale=ks)
        print(f"  head (b={b}, h={h})", flush=True)
        check("O", host64(out[b, h]), o_ref, 2e-2)
        check("LSE", host64(lse[b, h]), l_ref, 1e-3)
        check("dQ", host64(dq[b, h]), g["dq"], 2e-2)
        check("dK", host64(dk[b, h]), g["dk"], 2e-2)
        check("dV", host64(dv[b, h]), g["dv"], 2e-2)
