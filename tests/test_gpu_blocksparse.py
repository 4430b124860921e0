"""GPU parity of block-sparse attention (fa_forward_blocksparse / fa_backward_blocksparse)
against the float64 oracle with the tile mask expanded to elements.

Masks are seeded random patterns with about half the 128 x 128 blocks live, some with whole
query blocks dead (those rows must give O = 0 and LSE = -inf). Tolerances as for the plain path.
"""

import math

import numpy as np
import pytest

from exact_attention_94_amd import inputs as inp
from oracle import attn_bwd_ref, attn_fwd_ref, block_mask_to_elements
from tests.gpu_util import check, host64, nan_like, to_device

pytestmark = pytest.mark.gpu
BLOCK = 128


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_94_amd as fa_mod
    fa_mod.binding.load()
    return fa_mod


def _masks(heads, nb, seed, density=0.5, dead_row=True):
    rng = np.random.default_rng(seed)
    m = (rng.random((heads, nb, nb)) < density).astype(np.uint8)
    if dead_row and nb > 1:
        m[:, nb // 2, :] = 0  # a query block that sees nothing
    return m


def _visible(m, B, H, N):
    heads = m.shape[0]
    vis = np.empty((B, H, N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            vis[b, h] = block_mask_to_elements(m[0 if heads == 1 else b * H + h], N, BLOCK)
    return vis


def _check_lse(got, ref, tol):
    got = np.asarray(got, dtype=np.float64)
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), "rows without keys must have LSE = -inf"
    if (~empty).any():
        check("LSE", got[~empty], ref[~empty], tol)


def _run(fa, t, causal, scale, mask_t):
    import torch
    q, k, v, do = (to_device(t[n]) for n in ("q", "k", "v", "do"))
    out = nan_like(q.shape, torch.float32)
    lse = nan_like(q.shape[:3], torch.float32)
    fa.forward(q, k, v, scale=scale, causal=causal, out=out, lse=lse, block_mask=mask_t)
    grads = tuple(nan_like(q.shape, torch.float32) for _ in range(3))
    fa.backward(q, k, v, out, do, lse, scale=scale, causal=causal, grad_dtype=torch.float32,
                grads=grads, block_mask=mask_t)
    torch.cuda.synchronize()
    return out, lse, grads


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_sweep(fa, dtype, d, causal):
    import torch
    for n in [1, 65, 128, 129, 300, 520]:
        for (B, H) in ((1, 2), (2, 3)):
            for per_head in (False, True):
                nb = (n + BLOCK - 1) // BLOCK
                heads = B * H if per_head else 1
                m = _masks(heads, nb, seed=n + d + heads)
                print(f"  N={n} B={B} H={H} mask_heads={heads} live={m.mean():.2f}", flush=True)
                t = inp.draw((B, H, n, d), dtype, n * 5 + d, with_do=True)
                scale = 1.0 / math.sqrt(d)
                mask_t = torch.from_numpy(m if per_head else m[0]).cuda()
                out, lse, (dq, dk, dv) = _run(fa, t, causal, scale, mask_t)
                vis = _visible(m, B, H, n)
                o_ref, l_ref = attn_fwd_ref(t["q"].values, t["k"].values, t["v"].values, scale,
                                            causal, visible=vis)
                g = attn_bwd_ref(t["q"].values, t["k"].values, t["v"].values, t["do"].values,
                                 scale, causal, visible=vis)
                check("O", host64(out), o_ref, 2e-2)
                _check_lse(host64(lse), l_ref, 1e-3)
                check("dQ", host64(dq), g["dq"], 2e-2)
                check("dK", host64(dk), g["dk"], 2e-2)
                check("dV", host64(dv), g["dv"], 2e-2)


def test_all_live_mask_is_bitwise_the_plain_path(fa):
    """With every block live the block-sparse kernels visit the same tiles in the same order as
    the plain ones. The forward is compared at d = 128, where the plain forward also uses 64-key
    tiles (its tuned tile width at d = 64 is 128 keys); the backward at d = 64 and 128, from the
    same O and LSE. At d = 64 the block-sparse keys-outer kernel splits each key tile's query
    steps between two groups of waves and adds the two partial dK / dV at the end, so there dK
    and dV agree with the plain path to fp32 summation order only (bound 1e-5, far below the 2e-2
    oracle tolerance); dQ stays bitwise."""
    import torch
    for d in (64, 128):
        t = inp.draw((2, 2, 600, d), "bf16", 12 + d, with_do=True)
        q, k, v, do = (to_device(t[n]) for n in ("q", "k", "v", "do"))
        nb = (600 + BLOCK - 1) // BLOCK
        ones = torch.ones((nb, nb), dtype=torch.uint8, device="cuda")
        for causal in (False, True):
            o0, l0 = fa.forward(q, k, v, causal=causal, o_dtype=torch.float32)
            o1, l1 = fa.forward(q, k, v, causal=causal, o_dtype=torch.float32, block_mask=ones)
            g0 = fa.backward(q, k, v, o0, do, l0, causal=causal, grad_dtype=torch.float32)
            g1 = fa.backward(q, k, v, o0, do, l0, causal=causal, grad_dtype=torch.float32,
                             block_mask=ones)
            torch.cuda.synchronize()
            if d == 128:
                assert torch.equal(o0, o1) and torch.equal(l0, l1)
            for name, x, y in zip(("dQ", "dK", "dV"), g0, g1):
                if d == 64 and name != "dQ":
                    diff = float((x - y).abs().max())
                    print(f"  d={d} causal={causal} {name}: max |plain - sparse| = {diff:.3e}",
                          flush=True)
                    assert diff <= 1e-5, (name, diff)
                else:
                    assert torch.equal(x, y), name


def test_local_global_pattern_b2h16n4k(fa):
    """The benchmark shape with a sliding-window + global-column pattern (each query block sees
    its own and the previous block plus block 0), checked on two whole heads."""
    import torch
    w = inp.WORKLOADS["b2h16n4k_d64"]
    t = inp.workload_inputs(w)
    nb = w.N // BLOCK
    m = np.zeros((nb, nb), dtype=np.uint8)
    for qb in range(nb):
        m[qb, max(0, qb - 1):qb + 1] = 1
        m[qb, 0] = 1
    out, lse, (dq, dk, dv) = _run(fa, t, True, w.scale, torch.from_numpy(m).cuda())
    vis = block_mask_to_elements(m, w.N, BLOCK)
    for (b, h) in ((0, 2), (1, 9)):
        sel = lambda x: x[b, h]  # noqa: E731
        o_ref, l_ref = attn_fwd_ref(sel(t["q"].values), sel(t["k"].values), sel(t["v"].values),
                                    w.scale, True, visible=vis)
        g = attn_bwd_ref(sel(t["q"].values), sel(t["k"].values), sel(t["v"].values),
                         sel(t["do"].values), w.scale, True, visible=vis)
        print(f"  head (b={b}, h={h})", flush=True)
        check("O", host64(out[b, h]), o_ref, 2e-2)
        _check_lse(host64(lse[b, h]), l_ref, 1e-3)
        check("dQ", host64(dq[b, h]), g["dq"], 2e-2)
        check("dK", host64(dk[b, h]), g["dk"], 2e-2)
        check("dV", host64(dv[b, h]), g["dv"], 2e-2)
