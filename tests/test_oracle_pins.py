"""Pins of the float64 oracle against facts fixed outside the oracle itself.

Each test ties an oracle function to something it cannot satisfy by construction: values the
pages print for a worked example (tests/golden/, each file citing its source), closed forms,
invariants of softmax and of its gradient, central finite differences and brute force on tiny
inputs. A plausible mistake (dropped rescale, wrong mask direction, transposed operand, missing
scale in a gradient, natural vs base-2 logarithm) fails at least one of them.
"""

import math

import numpy as np
import pytest

from oracle import attn_bwd_ref, attn_fwd_ref, attn_rows_ref, attn_tiled_ref
from tests.conftest import golden_rows


def _qkv(seed, n, d, dist="normal"):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d))


# --- printed worked example ---------------------------------------------------------------

def test_trace_matches_printed_example():
    """m / l / corr of query 0 per K/V block equal the page's printed trace to 4 decimals."""
    q, k, v = _qkv(0, 8, 4)
    o, lse, info = attn_tiled_ref(q, k, v, 1.0 / math.sqrt(4), False, block_r=8, block_c=2,
                                  trace=True)
    gold = golden_rows("trace_rng0_n8_d4_bc2.txt")
    assert len(info["trace"]) == len(gold)
    for step, (j0, m, l, corr) in zip(info["trace"], gold):
        assert step["j0"] == int(j0)
        assert round(float(step["m"][0]), 4) == pytest.approx(m, abs=1e-12)
        assert round(float(step["l"][0]), 4) == pytest.approx(l, abs=1e-12)
        assert round(float(step["corr"][0]), 4) == pytest.approx(corr, abs=1e-12)
    # The same example through the naive oracle: the recurrence's result is the naive one.
    o_ref, lse_ref = attn_fwd_ref(q, k, v, 0.5, False)
    assert np.abs(o - o_ref).max() < 1e-15
    assert np.abs(lse - lse_ref).max() < 1e-15
    # LSE of row 0 is m + log l from the last printed step.
    assert lse_ref[0] == pytest.approx(0.6071 + math.log(5.3007), abs=2e-4)


@pytest.mark.parametrize("n", [256, 1024])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_naive_printed_magnitude(n, causal):
    """Blockwise (64x64) vs naive agree at float64 rounding, as the page's table reports."""
    gold = {(int(r[0]), int(r[2])): r[3] for r in golden_rows("exactness_table.txt")}
    q, k, v = _qkv(n, n, 64)
    o_t, lse_t, _ = attn_tiled_ref(q, k, v, 1.0 / 8.0, causal, 64, 64)
    o_n, lse_n = attn_fwd_ref(q, k, v, 1.0 / 8.0, causal)
    err = np.abs(o_t - o_n).max()
    assert err <= 1e-15
    assert err <= 4 * gold[(n, int(causal))]
    assert np.abs(lse_t - lse_n).max() < 1e-13


@pytest.mark.parametrize("blocks", [(1, 1), (7, 5), (5, 7), (33, 33), (None, None)])
@pytest.mark.parametrize("causal", [False, True])
def test_any_blocking_agrees(blocks, causal):
    """The recurrence holds for any blocking, block size 1 up to N ([FA-why] §03 3.2)."""
    n, d = 67, 16
    q, k, v = _qkv(11, n, d)
    br, bc = (n, n) if blocks[0] is None else blocks
    o_t, lse_t, _ = attn_tiled_ref(q, k, v, 0.37, causal, br, bc)
    o_n, lse_n = attn_fwd_ref(q, k, v, 0.37, causal)
    assert np.abs(o_t - o_n).max() < 5e-15
    assert np.abs(lse_t - lse_n).max() < 5e-15


def test_causal_tile_count_matches_page():
    gold = golden_rows("causal_tiles_n4096_b64.txt")[0]
    n, b = 4096, 64
    rng = np.random.default_rng(4096)
    q = rng.normal(size=(n, 8))
    _, _, info = attn_tiled_ref(q, q, q, 0.1, True, b, b)
    assert info["tiles_total"] == int(gold[0])
    assert info["tiles_kept"] == int(gold[1])
    t = n // b
    assert info["tiles_kept"] == t * (t + 1) // 2
    assert round(100.0 * (1 - info["tiles_kept"] / info["tiles_total"]), 1) == gold[2]


def test_rescale_ablation_reproduces_page_error():
    """Forcing corr = 1 gives the page's error (0.276 max, 0.0136 mean): the oracle harness
    distinguishes a missing rescale, and the oracle's recurrence is the page's."""
    max_gold, mean_gold = golden_rows("ablation_no_rescale.txt")[0]
    n = 1024
    q, k, v = _qkv(n, n, 64)
    o_n, _ = attn_fwd_ref(q, k, v, 1.0 / 8.0, False)
    o_bad, _, _ = attn_tiled_ref(q, k, v, 1.0 / 8.0, False, 64, 64,
                                 corr_fn=lambda m_old, m_new: np.ones_like(m_new))
    err = np.abs(o_bad - o_n)
    assert round(float(err.max()), 3) == pytest.approx(max_gold, abs=1e-9)
    assert round(float(err.mean()), 4) == pytest.approx(mean_gold, abs=1e-9)


# --- invariants of the recurrence ----------------------------------------------------------

@pytest.mark.parametrize("blocks", [(1, 1), (7, 5), (16, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_m_monotone_corr_bounded(blocks, causal):
    n = 40
    q, k, v = _qkv(3, n, 8)
    _, _, info = attn_tiled_ref(q, k, v, 0.9, causal, *blocks, trace=True)
    last_m = np.full(n, -np.inf)
    seen = np.zeros(n, dtype=bool)
    for st in info["trace"]:
        rows = np.arange(st["i0"], st["i0"] + len(st["m"]))
        assert np.all(st["m"] >= last_m[rows])
        assert np.all(st["corr"] <= 1.0)
        assert np.all(st["corr"] >= 0.0)
        first = ~seen[rows]
        assert np.all(st["corr"][first] == 0.0)
        last_m[rows] = st["m"]
        seen[rows] = True
    assert seen.all()


# --- closed forms --------------------------------------------------------------------------

def _brute_softmax_attention(q, k, v, scale, causal):
    """Pure-Python softmax attention on tiny inputs (math.exp, math.fsum), row by row."""
    n, d = len(q), len(q[0])
    o = [[0.0] * d for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        s = {j: scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys}
        top = max(s.values())
        w = {j: math.exp(s[j] - top) for j in keys}
        z = math.fsum(w.values())
        for t in range(d):
            o[i][t] = math.fsum(w[j] * v[j][t] for j in keys) / z
        lse[i] = top + math.log(z)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(causal):
    q, k, v = _qkv(5, 6, 3)
    o, lse = attn_fwd_ref(q, k, v, 0.7, causal)
    ob, lb = _brute_softmax_attention(q.tolist(), k.tolist(), v.tolist(), 0.7, causal)
    assert np.abs(o - ob).max() < 1e-15
    assert np.abs(lse - lb).max() < 1e-15
    orow, lrow = attn_rows_ref(q, k, v, 0.7, causal, range(6))
    assert np.abs(orow - ob).max() < 1e-15
    assert np.abs(lrow - lb).max() < 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    """With V = I (d = N) the output is P itself: every row sums to 1; masked entries are 0."""
    n = 48
    rng = np.random.default_rng(8)
    q = rng.normal(size=(n, 5))
    k = rng.normal(size=(n, 5))
    p, _ = attn_fwd_ref(q, k, np.eye(n), 1.3, causal)
    assert np.abs(p.sum(axis=1) - 1.0).max() < 1e-15
    assert (p >= 0).all()
    if causal:
        assert np.all(p[np.triu_indices(n, 1)] == 0.0)


def test_causal_row0_is_v0():
    q, k, v = _qkv(9, 20, 8)
    scale = 0.35
    o, lse = attn_fwd_ref(q, k, v, scale, True)
    assert np.array_equal(o[0], v[0])
    assert lse[0] == pytest.approx(scale * float(q[0] @ k[0]), abs=1e-15)
    g = attn_bwd_ref(q, k, v, np.random.default_rng(1).normal(size=(20, 8)), scale, True)
    assert np.all(g["dq"][0] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_keys_give_mean_of_values(causal):
    n, d = 37, 6
    rng = np.random.default_rng(12)
    q = rng.normal(size=(n, d))
    v = rng.normal(size=(n, d))
    o, lse = attn_fwd_ref(q, np.zeros((n, d)), v, 0.5, causal)
    if causal:
        cnt = np.arange(1, n + 1)
        assert np.abs(o - np.cumsum(v, axis=0) / cnt[:, None]).max() < 1e-14
        assert np.abs(lse - np.log(cnt)).max() < 1e-14
    else:
        assert np.abs(o - v.mean(axis=0)[None, :]).max() < 1e-14
        assert np.abs(lse - math.log(n)).max() < 1e-14


def test_constant_values_give_constant_output():
    n, d = 29, 7
    rng = np.random.default_rng(13)
    c = rng.normal(size=d)
    for causal in (False, True):
        o, _ = attn_fwd_ref(rng.normal(size=(n, d)), rng.normal(size=(n, d)),
                            np.tile(c, (n, 1)), 0.9, causal)
        assert np.abs(o - c[None, :]).max() < 1e-14


@pytest.mark.parametrize("shift", [1.0, 1e3 * 8.0])
def test_key_shift_invariance(shift):
    """K' = K + 1 c^T leaves O unchanged and moves LSE_i by scale*q_i.c; a huge shift checks
    that the max subtraction prevents overflow ([FA-why] §03 3.1)."""
    n, d = 33, 8
    q, k, v = _qkv(14, n, d)
    c = np.random.default_rng(15).normal(size=d) * shift
    scale = 1.0 / math.sqrt(d)
    o, lse = attn_fwd_ref(q, k, v, scale, False)
    o2, lse2 = attn_fwd_ref(q, k + c[None, :], v, scale, False)
    assert np.isfinite(o2).all()
    assert np.abs(o2 - o).max() < 1e-12 * max(1.0, shift)
    assert np.abs(lse2 - (lse + scale * (q @ c))).max() < 1e-11 * max(1.0, shift)


# --- backward ------------------------------------------------------------------------------

def _loss(q, k, v, do, scale, causal):
    o, _ = attn_fwd_ref(q, k, v, scale, causal)
    return float((do * o).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(5, 3), (8, 4)])
def test_backward_matches_finite_differences(causal, n, d):
    rng = np.random.default_rng(100 + n + d)
    q, k, v, do = (rng.normal(size=(n, d)) for _ in range(4))
    scale = 0.6
    g = attn_bwd_ref(q, k, v, do, scale, causal)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            orig = x[idx]
            x[idx] = orig + h
            up = _loss(q, k, v, do, scale, causal)
            x[idx] = orig - h
            dn = _loss(q, k, v, do, scale, causal)
            x[idx] = orig
            fd[idx] = (up - dn) / (2 * h)
        assert np.abs(fd - g[name]).max() < 1e-8, name


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    n, d = 50, 8
    rng = np.random.default_rng(21)
    q, k, v, do = (rng.normal(size=(n, d)) for _ in range(4))
    o, _ = attn_fwd_ref(q, k, v, 0.4, causal)
    g = attn_bwd_ref(q, k, v, do, 0.4, causal, o=o)
    # Rows of dS sum to zero, so the key-gradients sum to zero.
    assert np.abs(g["dk"].sum(axis=0)).max() < 1e-13
    # Rows of P sum to one, so the value-gradients sum to the upstream gradients' sum.
    assert np.abs(g["dv"].sum(axis=0) - do.sum(axis=0)).max() < 1e-13
    # rowsum(dP*P) = rowsum(dO*O).
    assert np.abs(g["D"] - g["D_o"]).max() < 1e-13
    if causal:
        assert np.all(g["dq"][0] == 0.0)


def test_backward_scale_zero_uniform_attention():
    """scale = 0: P is uniform (1/N); dQ = dK = 0 and dV_j = mean_i dO_i for every j."""
    n, d = 16, 4
    rng = np.random.default_rng(22)
    q, k, v, do = (rng.normal(size=(n, d)) for _ in range(4))
    g = attn_bwd_ref(q, k, v, do, 0.0, False)
    assert np.abs(g["dq"]).max() == 0.0
    assert np.abs(g["dk"]).max() < 1e-15
    assert np.abs(g["dv"] - do.mean(axis=0)[None, :]).max() < 1e-15


def test_batched_shapes_are_per_head():
    rng = np.random.default_rng(23)
    q, k, v, do = (rng.normal(size=(2, 3, 10, 4)) for _ in range(4))
    o, lse = attn_fwd_ref(q, k, v, 0.5, True)
    g = attn_bwd_ref(q, k, v, do, 0.5, True)
    for b in range(2):
        for h in range(3):
            o1, l1 = attn_fwd_ref(q[b, h], k[b, h], v[b, h], 0.5, True)
            assert np.array_equal(o[b, h], o1) and np.array_equal(lse[b, h], l1)
            g1 = attn_bwd_ref(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True)
            for key in ("dq", "dk", "dv"):
                assert np.array_equal(g[key][b, h], g1[key])


def test_rows_ref_matches_full_oracle():
    n, d = 300, 32
    q, k, v = _qkv(31, n, d)
    for causal in (False, True):
        o, lse = attn_fwd_ref(q, k, v, 0.2, causal)
        rows = [0, 1, 63, 64, 150, 298, 299]
        orow, lrow = attn_rows_ref(q, k, v, 0.2, causal, rows)
        assert np.abs(orow - o[rows]).max() < 1e-14
        assert np.abs(lrow - lse[rows]).max() < 1e-14


def test_torch_autograd_cross_check():
    """Library cross-check (not a pin on its own): float64 torch autograd of the explicit formula."""
    torch = pytest.importorskip("torch")
    n, d = 24, 8
    rng = np.random.default_rng(41)
    q, k, v, do = (rng.normal(size=(n, d)) for _ in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = 0.3 * tq @ tk.T
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
        out = torch.softmax(s, dim=1) @ tv
        out.backward(torch.tensor(do))
        g = attn_bwd_ref(q, k, v, do, 0.3, causal)
        assert np.abs(tq.grad.numpy() - g["dq"]).max() < 1e-13
        assert np.abs(tk.grad.numpy() - g["dk"]).max() < 1e-13
        assert np.abs(tv.grad.numpy() - g["dv"]).max() < 1e-13
