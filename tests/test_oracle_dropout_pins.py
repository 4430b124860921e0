"""Pins of the oracle's dropout: the Philox-4x32-10 generator, the keep mask built from it, and
attention with the mask.

The generator is pinned by its published known-answer vectors and by a one-round value derived
by hand; the mask by a per-element pure-Python rebuild and by its keep-rate statistics; attention
with dropout by p = 0 reducing to no dropout, by finite differences of the forward with a fixed
mask, by the D identity and by the expectation over seeds equalling undropped attention.
"""

import math
import os

import numpy as np
import pytest

from oracle import attn_bwd_ref, attn_fwd_ref, dropout_keep_ref, keep_scale, keep_threshold, philox4x32
from tests.conftest import ROOT


def _kat_rows():
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", "philox4x32_10_kat.txt")) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(t, 16) for t in line.split()])
    return rows


def test_philox_known_answer_vectors():
    rows = _kat_rows()
    assert len(rows) == 3
    for r in rows:
        out = philox4x32(np.array(r[:4], dtype=np.uint64), (r[4], r[5]))
        assert [int(x) for x in out] == r[6:10]


def test_philox_one_round_by_hand():
    """One round on counter (1, 0, 0, 0), key (0, 0): hi(M0*1) = 0, lo(M0*1) = M0 and M1*0 = 0,
    so the output is (0 ^ 0 ^ 0, 0, 0 ^ 0 ^ 0, M0) = (0, 0, 0, 0xD2511F53)."""
    out = philox4x32(np.array([1, 0, 0, 0]), (0, 0), rounds=1)
    assert [int(x) for x in out] == [0, 0, 0, 0xD2511F53]
    # Counter (0, 0, 1, 0): the M1 product feeds words 0 and 1.
    out = philox4x32(np.array([0, 0, 1, 0]), (5, 7), rounds=1)
    assert [int(x) for x in out] == [0 ^ 0 ^ 5, 0xCD9E8D57, 0 ^ 0 ^ 7, 0]


def test_keep_threshold_values():
    assert keep_threshold(0.0) == 65536
    assert keep_threshold(0.5) == 32768
    assert keep_threshold(0.1) == 58982  # (1 - float32(0.1)) * 65536 = 58982.3999...
    assert keep_scale(0.5) == 2.0
    with pytest.raises(ValueError):
        keep_threshold(1.0)


def test_mask_rebuilt_element_by_element():
    """Each mask entry equals the 16-bit half-word of its own Philox call (pure-Python loop)."""
    seed, offset, bh, p = 0x0123456789ABCDEF, 77, 5, 0.3
    n = 19
    mask = dropout_keep_ref(n, n, bh, seed, offset, p)
    t = keep_threshold(p)
    for i in range(n):
        for j in range(n):
            w = philox4x32(np.array([j // 8, i, bh, offset], dtype=np.uint64),
                           (seed & 0xFFFFFFFF, seed >> 32))
            word = int(w[(j % 8) // 2])
            val = (word >> 16) if (j % 2) else (word & 0xFFFF)
            assert mask[i, j] == (val < t)


def test_mask_keep_rate_and_independence():
    p = 0.2
    m = dropout_keep_ref(256, 256, 3, 42, 0, p)
    q = keep_threshold(p) / 65536.0
    sigma = math.sqrt(q * (1 - q) / m.size)
    assert abs(m.mean() - q) < 5 * sigma
    # Row and column rates carry no structure beyond noise.
    assert abs(m.mean(axis=0) - q).max() < 6 * math.sqrt(q * (1 - q) / 256)
    assert abs(m.mean(axis=1) - q).max() < 6 * math.sqrt(q * (1 - q) / 256)
    # Same (seed, offset, head) -> same mask; changing any of them changes it.
    assert np.array_equal(m, dropout_keep_ref(256, 256, 3, 42, 0, p))
    for other in (dropout_keep_ref(256, 256, 4, 42, 0, p), dropout_keep_ref(256, 256, 3, 43, 0, p),
                  dropout_keep_ref(256, 256, 3, 42, 1, p)):
        agree = (other == m).mean()
        assert abs(agree - (q * q + (1 - q) * (1 - q))) < 0.01


def _qkv(seed, n, d):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(n, d)) for _ in range(4))


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_no_dropout(causal):
    q, k, v, do = _qkv(3, 12, 5)
    keep = dropout_keep_ref(12, 12, 0, 9, 0, 0.0)
    assert keep.all()
    o0, l0 = attn_fwd_ref(q, k, v, 0.4, causal)
    o1, l1 = attn_fwd_ref(q, k, v, 0.4, causal, keep=keep, keep_scale=keep_scale(0.0))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    g0 = attn_bwd_ref(q, k, v, do, 0.4, causal)
    g1 = attn_bwd_ref(q, k, v, do, 0.4, causal, keep=keep, keep_scale=1.0)
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(g0[name], g1[name])


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_backward_matches_finite_differences(causal):
    """With the mask fixed, L = sum(dO * O) is a smooth function of Q, K, V; the oracle's gradients
    equal its central differences."""
    n, d, scale, p = 7, 3, 0.6, 0.4
    q, k, v, do = _qkv(11, n, d)
    keep = dropout_keep_ref(n, n, 2, 1234, 5, p)
    assert 0 < keep.mean() < 1
    ks = keep_scale(p)

    def loss(qq, kk, vv):
        o, _ = attn_fwd_ref(qq, kk, vv, scale, causal, keep=keep, keep_scale=ks)
        return float((do * o).sum())

    g = attn_bwd_ref(q, k, v, do, scale, causal, keep=keep, keep_scale=ks)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            args_m = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(num - g[name]).max() < 1e-7


def test_dropout_delta_identity():
    """rowsum(dO * O) = rowsum(dP * P) also with dropout (the backward's D needs only O)."""
    q, k, v, do = _qkv(21, 16, 4)
    keep = dropout_keep_ref(16, 16, 1, 99, 3, 0.3)
    ks = keep_scale(0.3)
    for causal in (False, True):
        o, _ = attn_fwd_ref(q, k, v, 0.5, causal, keep=keep, keep_scale=ks)
        g = attn_bwd_ref(q, k, v, do, 0.5, causal, o=o, keep=keep, keep_scale=ks)
        assert np.abs(g["D"] - g["D_o"]).max() < 1e-13


def test_dropout_expectation_over_seeds():
    """Averaged over seeds, dropout attention equals undropped attention (each kept probability is
    scaled by 1/keep-rate). The tolerance is 5 standard errors from the exact per-element variance
    sum_j P_ij^2 v_j^2 (65536/T - 1)."""
    n, d, p = 6, 2, 0.5
    q, k, v, _ = _qkv(5, n, d)
    o_ref, _ = attn_fwd_ref(q, k, v, 0.7, False)
    seeds = 600
    acc = np.zeros((n, d))
    for s in range(seeds):
        keep = dropout_keep_ref(n, n, 0, 1000 + s, 0, p)
        o, _ = attn_fwd_ref(q, k, v, 0.7, False, keep=keep, keep_scale=keep_scale(p))
        acc += o
    mean = acc / seeds
    s_ = 0.7 * (q @ k.T)
    P = np.exp(s_ - s_.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    var = (P ** 2) @ (v ** 2) * (keep_scale(p) - 1.0)
    assert np.all(np.abs(mean - o_ref) < 5 * np.sqrt(var / seeds) + 1e-12)
