"""Pins of the oracle's block-sparse attention (a tile mask generalising the causal whole-tile
skip, "FlashAttention 为什么不需要存下注意力矩阵" §06).

The mask expansion is rebuilt element by element; masked attention is checked against a
per-row softmax over only the visible keys (a separate code path), against the causal rule
(a lower-triangular mask at block size 1 is exactly causal), against the plain oracle for an
all-visible mask, and by finite differences; rows that see no key give O = 0, LSE = -inf and no
gradient.
"""

import math

import numpy as np
import pytest

from oracle import attn_bwd_ref, attn_fwd_ref, block_mask_to_elements


def _qkv(seed, n, d):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(n, d)) for _ in range(4))


def test_mask_expansion_element_by_element():
    n, block = 7, 3
    rng = np.random.default_rng(1)
    bm = rng.integers(0, 2, size=(3, 3))
    vis = block_mask_to_elements(bm, n, block)
    for i in range(n):
        for j in range(n):
            assert vis[i, j] == bool(bm[i // block][j // block])


@pytest.mark.parametrize("causal", [False, True])
def test_all_visible_is_the_plain_oracle(causal):
    q, k, v, do = _qkv(2, 20, 4)
    vis = block_mask_to_elements(np.ones((3, 3)), 20, 8)
    o0, l0 = attn_fwd_ref(q, k, v, 0.5, causal)
    o1, l1 = attn_fwd_ref(q, k, v, 0.5, causal, visible=vis)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    g0 = attn_bwd_ref(q, k, v, do, 0.5, causal)
    g1 = attn_bwd_ref(q, k, v, do, 0.5, causal, visible=vis)
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(g0[name], g1[name])


def test_lower_triangular_mask_at_block_one_is_causal():
    q, k, v, do = _qkv(3, 9, 3)
    vis = block_mask_to_elements(np.tril(np.ones((9, 9))), 9, 1)
    o0, l0 = attn_fwd_ref(q, k, v, 0.7, True)
    o1, l1 = attn_fwd_ref(q, k, v, 0.7, False, visible=vis)
    assert np.abs(o0 - o1).max() == 0 and np.abs(l0 - l1).max() == 0


@pytest.mark.parametrize("causal", [False, True])
def test_rows_equal_softmax_over_visible_keys(causal):
    n, d, block, scale = 23, 5, 4, 0.45
    q, k, v, _ = _qkv(4, n, d)
    rng = np.random.default_rng(9)
    bm = rng.integers(0, 2, size=(6, 6))
    bm[:, 0] = 1  # every query sees its first key block: no empty rows here
    vis = block_mask_to_elements(bm, n, block)
    o, lse = attn_fwd_ref(q, k, v, scale, causal, visible=vis)
    for i in range(n):
        keys = [j for j in range(n) if vis[i, j] and (not causal or j <= i)]
        s = np.array([scale * float(q[i] @ k[j]) for j in keys])
        mx = s.max()
        w = np.exp(s - mx)
        ref = sum(wj * v[j] for wj, j in zip(w, keys)) / w.sum()
        assert np.abs(o[i] - ref).max() < 1e-14
        assert abs(lse[i] - (mx + math.log(w.sum()))) < 1e-14


def test_row_without_visible_keys():
    n, d, block = 12, 3, 4
    q, k, v, do = _qkv(5, n, d)
    bm = np.ones((3, 3))
    bm[1, :] = 0  # queries 4..7 see nothing
    vis = block_mask_to_elements(bm, n, block)
    o, lse = attn_fwd_ref(q, k, v, 0.5, False, visible=vis)
    assert np.all(o[4:8] == 0) and np.all(np.isneginf(lse[4:8]))
    assert np.all(np.isfinite(lse[:4])) and np.all(np.isfinite(lse[8:]))
    g = attn_bwd_ref(q, k, v, do, 0.5, False, visible=vis)
    assert np.all(g["dq"][4:8] == 0)
    # Those rows contribute nothing to dK / dV: zeroing their dO changes nothing.
    do2 = do.copy()
    do2[4:8] = 0
    g2 = attn_bwd_ref(q, k, v, do2, 0.5, False, visible=vis)
    assert np.array_equal(g["dk"], g2["dk"]) and np.array_equal(g["dv"], g2["dv"])


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_backward_matches_finite_differences(causal):
    n, d, block, scale = 9, 3, 2, 0.6
    q, k, v, do = _qkv(6, n, d)
    bm = np.random.default_rng(3).integers(0, 2, size=(5, 5))
    np.fill_diagonal(bm, 1)
    vis = block_mask_to_elements(bm, n, block)

    def loss(qq, kk, vv):
        o, _ = attn_fwd_ref(qq, kk, vv, scale, causal, visible=vis)
        return float((do * o).sum())

    g = attn_bwd_ref(q, k, v, do, scale, causal, visible=vis)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a_p = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            a_m = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            num[idx] = (loss(*a_p) - loss(*a_m)) / (2 * h)
        assert np.abs(num - g[name]).max() < 1e-7
