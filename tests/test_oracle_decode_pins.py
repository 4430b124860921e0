"""Pins of the oracle's decoding functions (Nq query rows over Nk keys, and the split-KV form).

attn_decode_ref is tied to the square oracle (its queries are the last rows of a full causal
problem, and Nq = Nk is exactly the causal forward), to the per-row oracle and to brute force;
attn_split_merge_ref is tied to attn_decode_ref for several chunk sizes, including chunks that
a causal query cannot see at all.
"""

import math

import numpy as np
import pytest

from oracle import attn_decode_ref, attn_fwd_ref, attn_rows_ref, attn_split_merge_ref


def _rand(seed, *shape):
    return np.random.default_rng(seed).normal(size=shape)


def test_square_decode_is_the_causal_forward():
    q, k, v = _rand(1, 2, 3, 40, 8), _rand(2, 2, 3, 40, 8), _rand(3, 2, 3, 40, 8)
    o0, l0 = attn_fwd_ref(q, k, v, 0.3, True)
    o1, l1 = attn_decode_ref(q, k, v, 0.3, True)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("nq", [1, 3, 8])
def test_decode_rows_are_the_last_rows_of_the_full_problem(nq):
    n, d = 50, 6
    q, k, v = _rand(4, n, d), _rand(5, n, d), _rand(6, n, d)
    o_full, l_full = attn_fwd_ref(q, k, v, 0.4, True)
    o, l = attn_decode_ref(q[n - nq:], k, v, 0.4, True)
    assert np.abs(o - o_full[n - nq:]).max() < 1e-15
    assert np.abs(l - l_full[n - nq:]).max() < 1e-14
    # Non-causal: every row sees every key, as attn_rows_ref computes row by row.
    o2, l2 = attn_decode_ref(q[n - nq:], k, v, 0.4, False)
    o3, l3 = attn_rows_ref(q, k, v, 0.4, False, range(n - nq, n))
    assert np.abs(o2 - o3).max() < 1e-14 and np.abs(l2 - l3).max() < 1e-14


def test_decode_brute_force():
    nq, nk, d, scale = 2, 5, 3, 0.9
    q, k, v = _rand(7, nq, d), _rand(8, nk, d), _rand(9, nk, d)
    o, l = attn_decode_ref(q, k, v, scale, True)
    for i in range(nq):
        keys = range(nk - nq + i + 1)
        s = [scale * sum(q[i, t] * k[j, t] for t in range(d)) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = sum(w)
        for t in range(d):
            assert abs(o[i, t] - sum(wj * v[j, t] for wj, j in zip(w, keys)) / tot) < 1e-14
        assert abs(l[i] - (mx + math.log(tot))) < 1e-14


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("chunk", [1, 7, 64, 300])
def test_split_merge_equals_direct(causal, chunk):
    nq, nk, d = 4, 300, 16
    q, k, v = _rand(10, 2, nq, d), _rand(11, 2, nk, d), _rand(12, 2, nk, d)
    o0, l0 = attn_decode_ref(q, k, v, 0.25, causal)
    o1, l1 = attn_split_merge_ref(q, k, v, 0.25, causal, chunk)
    assert np.abs(o0 - o1).max() < 1e-13
    assert np.abs(l0 - l1).max() < 1e-13


def test_split_merge_with_chunks_invisible_to_some_queries():
    """Square causal problem split in chunks: early queries cannot see late chunks at all."""
    n, d = 64, 4
    q, k, v = _rand(13, n, d), _rand(14, n, d), _rand(15, n, d)
    o0, l0 = attn_fwd_ref(q, k, v, 0.5, True)
    o1, l1 = attn_split_merge_ref(q, k, v, 0.5, True, 16)
    assert np.abs(o0 - o1).max() < 1e-13 and np.abs(l0 - l1).max() < 1e-13


def test_noncausal_more_queries_than_keys_brute_force():
    nq, nk, d, scale = 5, 3, 2, 0.8
    q, k, v = _rand(16, nq, d), _rand(17, nk, d), _rand(18, nk, d)
    o, l = attn_decode_ref(q, k, v, scale, False)
    for i in range(nq):
        s = [scale * sum(q[i, t] * k[j, t] for t in range(d)) for j in range(nk)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = sum(w)
        for t in range(d):
            assert abs(o[i, t] - sum(wj * v[j, t] for j, wj in enumerate(w)) / tot) < 1e-14
        assert abs(l[i] - (mx + math.log(tot))) < 1e-14
    with pytest.raises(ValueError):
        attn_decode_ref(q, k, v, scale, True)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_with_fewer_queries_than_keys_matches_finite_differences(causal):
    """attn_bwd_ref with Nq < Nk is the gradient of attn_decode_ref (queries at the end)."""
    from oracle import attn_bwd_ref
    nq, nk, d, scale = 3, 7, 3, 0.6
    q, k, v, do = _rand(20, nq, d), _rand(21, nk, d), _rand(22, nk, d), _rand(23, nq, d)

    def loss(qq, kk, vv):
        o, _ = attn_decode_ref(qq, kk, vv, scale, causal)
        return float((do * o).sum())

    g = attn_bwd_ref(q, k, v, do, scale, causal)
    assert g["dq"].shape == (nq, d) and g["dk"].shape == (nk, d)
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
    if causal:
        # The first key rows that no query can reach would have zero gradient only if none sees
        # them; with the queries at the end, the last query sees every key.
        assert np.abs(g["dk"]).sum() > 0
