"""GPU parity of fa_forward_kv and fa_backward_kv (Nq query rows against Nk keys) against the
float64 oracle (attn_decode_ref and attn_bwd_ref: with causal, the queries are the last Nq
positions). Tolerances as for self-attention: 2e-2 on O, dQ, dK, dV and 1e-3 on LSE for 16-bit
inputs."""

import math

import numpy as np
import pytest

from exact_attention_94_amd import inputs as inp
from oracle import attn_bwd_ref, attn_decode_ref
from tests.gpu_util import check, host64, nan_like, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_94_amd as fa_mod
    fa_mod.binding.load()
    return fa_mod


CASES_CAUSAL = [(1, 5), (17, 300), (64, 64), (100, 1000), (129, 4099), (300, 301)]
CASES_FULL = CASES_CAUSAL + [(300, 17), (5, 1)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_kv_sweep(fa, dtype, d, causal):
    import torch
    for (nq, nk) in (CASES_CAUSAL if causal else CASES_FULL):
        for (B, H) in ((1, 2), (2, 3)):
            print(f"  Nq={nq} Nk={nk} B={B} H={H}", flush=True)
            tq = inp.draw((B, H, nq, d), dtype, nq * 7 + d)
            tk = inp.draw((B, H, nk, d), dtype, nk * 7 + d + 1)
            q = to_device(tq["q"])
            k, v = to_device(tk["k"]), to_device(tk["v"])
            out = nan_like((B, H, nq, d), torch.float32)
            lse = nan_like((B, H, nq), torch.float32)
            scale = 1.0 / math.sqrt(d)
            fa.forward(q, k, v, scale=scale, causal=causal, out=out, lse=lse)
            torch.cuda.synchronize()
            o_ref, l_ref = attn_decode_ref(tq["q"].values, tk["k"].values, tk["v"].values, scale,
                                           causal)
            check("O", host64(out), o_ref, 2e-2)
            check("LSE", host64(lse), l_ref, 1e-3)


# A grid large enough for the two-group forward kernel (4 query tiles of 256 x 128 heads = 512
# workgroups), so that its query offset (causal: Nk - Nq) and key count Nk != Nq are exercised;
# ragged last query and key tiles (1000 = 3 * 256 + 232, 1500 = 11 * 128 + 92).
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_kv_two_group_grid(fa, dtype, d, causal):
    import torch
    B, H, nq, nk = 4, 32, 1000, 1500
    tq = inp.draw((B, H, nq, d), dtype, 9000 + d)
    tk = inp.draw((B, H, nk, d), dtype, 9001 + d)
    q = to_device(tq["q"])
    k, v = to_device(tk["k"]), to_device(tk["v"])
    out = nan_like((B, H, nq, d), torch.float32)
    lse = nan_like((B, H, nq), torch.float32)
    scale = 1.0 / math.sqrt(d)
    fa.forward(q, k, v, scale=scale, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = attn_decode_ref(tq["q"].values, tk["k"].values, tk["v"].values, scale, causal)
    check("O", host64(out), o_ref, 2e-2)
    check("LSE", host64(lse), l_ref, 1e-3)


def test_forward_kv_is_the_tail_of_the_full_causal_forward(fa):
    """Rows N-Nq.. of a causal forward over N positions, recomputed from only those query rows
    against all N keys, are bitwise the same: each row visits the same key tiles in the same
    order, and the tiles a row cannot see change nothing."""
    import torch
    N, d = 1000, 64
    t = inp.draw((2, 4, N, d), "bf16", 31)
    q, k, v = (to_device(t[n]) for n in ("q", "k", "v"))
    o_full, l_full = fa.forward(q, k, v, causal=True, o_dtype=torch.float32)
    for nq in (1, 77, 256):
        qt = q[:, :, N - nq:].contiguous()
        o_kv, l_kv = fa.forward(qt, k, v, causal=True, o_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o_kv, o_full[:, :, N - nq:]) and torch.equal(l_kv, l_full[:, :, N - nq:])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_kv_sweep(fa, dtype, d, causal):
    import torch
    for (nq, nk) in (CASES_CAUSAL if causal else CASES_FULL):
        for (B, H) in ((1, 2), (2, 3)):
            print(f"  Nq={nq} Nk={nk} B={B} H={H}", flush=True)
            tq = inp.draw((B, H, nq, d), dtype, nq * 5 + d, with_do=True)
            tk = inp.draw((B, H, nk, d), dtype, nk * 5 + d + 1)
            q, do = to_device(tq["q"]), to_device(tq["do"])
            k, v = to_device(tk["k"]), to_device(tk["v"])
            scale = 1.0 / math.sqrt(d)
            out, lse = fa.forward(q, k, v, scale=scale, causal=causal, o_dtype=torch.float32)
            grads = (nan_like(q.shape, torch.float32), nan_like(k.shape, torch.float32),
                     nan_like(k.shape, torch.float32))
            dq, dk, dv = fa.backward(q, k, v, out, do, lse, scale=scale, causal=causal,
                                     grad_dtype=torch.float32, grads=grads)
            torch.cuda.synchronize()
            g = attn_bwd_ref(tq["q"].values, tk["k"].values, tk["v"].values, tq["do"].values,
                             scale, causal)
            check("dQ", host64(dq), g["dq"], 2e-2)
            check("dK", host64(dk), g["dk"], 2e-2)
            check("dV", host64(dv), g["dv"], 2e-2)


def test_backward_kv_bf16_gradients(fa):
    """16-bit gradient outputs and a 16-bit forward output on a chunked-prefill shape."""
    import torch
    B, H, nq, nk, d = 2, 4, 200, 1100, 128
    tq = inp.draw((B, H, nq, d), "bf16", 41, with_do=True)
    tk = inp.draw((B, H, nk, d), "bf16", 42)
    q, do = to_device(tq["q"]), to_device(tq["do"])
    k, v = to_device(tk["k"]), to_device(tk["v"])
    out, lse = fa.forward(q, k, v, causal=True)
    dq, dk, dv = fa.backward(q, k, v, out, do, lse, causal=True)
    torch.cuda.synchronize()
    assert dq.dtype == dk.dtype == torch.bfloat16 and dk.shape == k.shape
    g = attn_bwd_ref(tq["q"].values, tk["k"].values, tk["v"].values, tq["do"].values,
                     1.0 / math.sqrt(d), True)
    check("dQ", host64(dq), g["dq"], 2e-2)
    check("dK", host64(dk), g["dk"], 2e-2)
    check("dV", host64(dv), g["dv"], 2e-2)


def test_backward_kv_dq_is_the_tail_of_the_full_causal_dq(fa):
    """dQ of the last Nq rows of a causal self-attention backward, recomputed from only those
    rows (with their O, dO and LSE) against all N keys, is bitwise the same: each dQ row depends
    on its own row and on K, V only, and the tiles it cannot see add exact zeros."""
    import torch
    N, d = 1000, 64
    t = inp.draw((2, 4, N, d), "bf16", 37, with_do=True)
    q, k, v, do = (to_device(t[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=True, o_dtype=torch.float32)
    dq_full, _, _ = fa.backward(q, k, v, o, do, lse, causal=True, grad_dtype=torch.float32)
    for nq in (1, 77, 256):
        sl = slice(N - nq, N)
        dq, dk, dv = fa.backward(q[:, :, sl].contiguous(), k, v, o[:, :, sl].contiguous(),
                                 do[:, :, sl].contiguous(), lse[:, :, sl].contiguous(),
                                 causal=True, grad_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq_full[:, :, sl])
        assert dk.shape == k.shape and bool(torch.isfinite(dk).all() and torch.isfinite(dv).all())
