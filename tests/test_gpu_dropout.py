"""GPU parity of dropout (fa_forward_dropout / fa_backward_dropout) against the float64 oracle.

The oracle builds the keep mask from the same (p, seed, offset) with its own Philox-4x32-10.
On random inputs one flipped mask bit moves an output row by only about P_ij |v_j| / q (of order
|v| / N), far below the 2e-2 tolerance, so the random-input tests below check the arithmetic
around the mask, and the read-out tests check the mask itself bit for bit: with structured
inputs (zero scores, rows that are powers of two times unit vectors) the forward's O and the
backward's dV and dQ hold, in each element, an integer whose binary digits are keep bits, and
those integers must equal the oracle's mask exactly.
Tolerances of the random-input tests as for the plain path: 2e-2 on O / dQ / dK / dV and 1e-3
on LSE (16-bit inputs).
"""

import math

import numpy as np
import pytest

from exact_attention_94_amd import inputs as inp
from oracle import attn_bwd_ref, attn_fwd_ref, dropout_keep_ref, keep_scale
from tests.gpu_util import check, host64, nan_like, to_device, torch_dtype

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


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_high_rate(fa, dtype, causal):
    """p = 0.9: kept scores are scaled by 1/q = 65536/T (T = 6554), which the backward folds
    into its exp2 offset and its dP start; the oracle checks every output at the usual
    tolerances on ragged lengths."""
    p, seed, offset = 0.9, 0x0BAD_5EED_1234_5678, 11
    ks = keep_scale(p)
    d = 64
    for n in [65, 300]:
        B, H = 1, 2
        print(f"  N={n} {dtype} causal={causal}", flush=True)
        t = inp.draw((B, H, n, d), dtype, n * 7 + 5, with_do=True)
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


def test_dropout_p0_matches_the_plain_path(fa):
    """With p = 0 the dropout kernels keep every score. The forward is bitwise the plain path.
    In the backward the keep rate q = 1 turns the dropout kernels' exp2 offset log2(1/q) into 0
    and their dP start -D q into the plain kernels' -D, but they are other instantiations (the
    dK/dV kernel takes 64-query steps, and its row vectors and keep words take other paths), so
    the gradients are held to a bound far below the oracle tolerance (2e-2) rather than to
    equality."""
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
    for name, x, y in zip(("dQ", "dK", "dV"), g0, g1):
        diff = float((x - y).abs().max())
        print(f"  {name}: max |plain - dropout p=0| = {diff:.3e}", flush=True)
        assert diff <= 1e-4, (name, diff)


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


# --- bit-exact read-out of the keep mask ------------------------------------------------------

def _pow2_rows(n, d):
    """[n, d] float32 with row r = 2^(r // d) * e_(r mod d). A product that sums such rows with
    0/1 weights w_r gives, in column c, the integer sum_k w_(c + k d) 2^k: the weights become
    the binary digits of the result (exact in fp32 while n <= 24 d)."""
    x = np.zeros((n, d), dtype=np.float32)
    r = np.arange(n)
    x[r, r % d] = np.float32(2.0) ** (r // d)
    return x


def _mask_digits(m, d):
    """For a boolean [R, n] mask, the [R, d] integers sum_(j = c mod d) m[:, j] 2^(j // d)."""
    n = m.shape[1]
    w = (2 ** (np.arange(n) // d)).astype(np.int64)
    out = np.zeros((m.shape[0], d), dtype=np.int64)
    for c in range(min(d, n)):
        out[:, c] = (m[:, c::d].astype(np.int64) * w[c::d]).sum(axis=1)
    return out


def _digits(x, unit):
    """Round x / unit to integers, insisting that x was within 0.3 units of one."""
    y = np.asarray(x, dtype=np.float64) / unit
    r = np.rint(y)
    assert np.abs(y - r).max() < 0.3, f"read-out off the integer grid by {np.abs(y - r).max()}"
    return r.astype(np.int64)


READOUT_N = {64: [64, 300, 1000], 128: [128, 700, 2000]}


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_keep_mask_bit_exact(fa, dtype, d, causal):
    """K = 0 makes every visible probability exp(0) = 1 before normalisation, and V row j =
    2^(j // d) e_(j mod d), so the fp32 O_ic = (keep scale / l_i) * sum_(j = c mod d) Z_ij 2^(j//d)
    with l_i the number of visible keys: the integer O_ic * l_i / keep scale spells out the
    forward's keep bits of row i, which must equal the oracle's Z (restricted to visible keys)."""
    import torch
    p, seed, offset = 0.3, 0xFEDC_BA98_7654_3210, 11
    B, H = 2, 3
    ks32 = float(np.float32(keep_scale(p)))
    for n in READOUT_N[d]:
        print(f"  N={n}", flush=True)
        rng = np.random.default_rng(n + d)
        qv = inp.quantize(rng.standard_normal((B, H, n, d), dtype=np.float32), dtype)
        vv = inp.quantize(np.broadcast_to(_pow2_rows(n, d), (B, H, n, d)).copy(), dtype)
        q, v = to_device(qv), to_device(vv)
        k = torch.zeros_like(q)
        out = nan_like((B, H, n, d), torch.float32)
        lse = nan_like((B, H, n), torch.float32)
        fa.forward(q, k, v, causal=causal, out=out, lse=lse, dropout_p=p, seed=seed,
                   offset=offset)
        torch.cuda.synchronize()
        o = host64(out)
        vis = np.tril(np.ones((n, n), dtype=bool)) if causal else np.ones((n, n), dtype=bool)
        l_rows = vis.sum(axis=1).astype(np.float64)
        for b in range(B):
            for h in range(H):
                z = dropout_keep_ref(n, n, b * H + h, seed, offset, p) & vis
                got = _digits(o[b, h] * l_rows[:, None], ks32)
                want = _mask_digits(z, d)
                bad = np.argwhere(got != want)
                assert bad.size == 0, f"head {(b, h)}: keep bits differ at (row, col) {bad[:5]}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_keep_mask_bit_exact(fa, dtype, d):
    """Q = 0 gives P = 1/N everywhere (non-causal); V = all ones, dO row i = 2^(i // d) e_(i mod d),
    K row j = 2^(j // d) e_(j mod d), and O passed as zeros so that D = rowsum(dO * O) = 0. Then
      dV_jc = f * sum_(i = c mod d) Z_ij 2^(i // d)            (keys-outer kernel's mask),
      dQ_ic = scale * f * 2^(i // d) * sum_(j = c mod d) Z_ij 2^(j // d)   (queries-outer kernel's),
    with f = keep scale / N rounded once to fp16 (the operand precision of the gradient products;
    within 2^-11 of keep scale / N, so the integers stay recoverable for N <= 8 d). Both must equal
    the oracle's mask, transposed for dV."""
    import torch
    p, seed, offset = 0.25, 0x0123_4567_89AB_CDEF, 5
    B, H = 2, 3
    ks32 = float(np.float32(keep_scale(p)))
    scale = 1.0 / math.sqrt(d)
    for n in ([64, 200, 512] if d == 64 else [128, 300, 1000]):
        print(f"  N={n}", flush=True)
        rows = _pow2_rows(n, d)
        q = torch.zeros((B, H, n, d), dtype=torch_dtype(dtype), device="cuda")
        k = to_device(inp.quantize(np.broadcast_to(rows, (B, H, n, d)).copy(), dtype))
        v = to_device(inp.quantize(np.ones((B, H, n, d), dtype=np.float32), dtype))
        do = to_device(inp.quantize(np.broadcast_to(rows, (B, H, n, d)).copy(), dtype))
        _, lse = fa.forward(q, k, v, scale=scale, causal=False, o_dtype=torch.float32)
        o_zero = torch.zeros((B, H, n, d), dtype=torch.float32, device="cuda")
        grads = tuple(nan_like((B, H, n, d), torch.float32) for _ in range(3))
        dq, dk, dv = fa.backward(q, k, v, o_zero, do, lse, scale=scale, causal=False,
                                 grad_dtype=torch.float32, grads=grads, dropout_p=p, seed=seed,
                                 offset=offset)
        torch.cuda.synchronize()
        dq_h, dv_h = host64(dq), host64(dv)
        unit = ks32 / n
        row_pow = (2.0 ** (np.arange(n) // d))[:, None]
        for b in range(B):
            for h in range(H):
                z = dropout_keep_ref(n, n, b * H + h, seed, offset, p)
                got_v = _digits(dv_h[b, h], unit)
                want_v = _mask_digits(z.T, d)
                bad = np.argwhere(got_v != want_v)
                assert bad.size == 0, f"dV head {(b, h)}: keep bits differ at (key, col) {bad[:5]}"
                got_q = _digits(dq_h[b, h] / (scale * row_pow), unit)
                want_q = _mask_digits(z, d)
                bad = np.argwhere(got_q != want_q)
                assert bad.size == 0, f"dQ head {(b, h)}: keep bits differ at (row, col) {bad[:5]}"
        assert np.abs(host64(dk)).max() == 0.0  # Q = 0: dK = scale * dS^T Q vanishes


# --- full-chip grids --------------------------------------------------------------------------

def _full_grid_heads(n, causal):
    """B, H (B*H a multiple of 8) giving at least 512 causal, or 256 non-causal, 256-query tiles:
    grids that fill the chip, where the plain forward switches to its two-group kernel."""
    need = 512 if causal else 256
    tiles = -(-n // 256)
    H = 8
    while tiles * 4 * H < need:
        H += 8
    return 4, H


def _spread_heads(B, H, count=8):
    """count (b, h) pairs spread over all B*H heads (one per XCD group of heads)."""
    bh = B * H
    return [divmod(i * bh // count + (i % 3), H) for i in range(count)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96])
@pytest.mark.parametrize("causal", [False, True])
def test_full_grid_forward_keep_mask_bit_exact(fa, dtype, d, causal):
    """The read-out of test_forward_keep_mask_bit_exact on a full-chip grid (ragged N, 8 heads
    spread over the grid compared bit for bit, every head finite)."""
    import torch
    p, seed, offset = 0.3, 0x0BAD_CAFE_1234_5678, 9
    # Rows reach 2^((N - 1) // d): at most 2^15 keeps them finite in fp16, and the read-out
    # integers exact in fp32.
    n = min(1000, 16 * d - 8)
    B, H = _full_grid_heads(n, causal)
    print(f"  B={B} H={H} N={n}", flush=True)
    ks32 = float(np.float32(keep_scale(p)))
    rng = np.random.default_rng(n + d + causal)
    qv = inp.quantize(rng.standard_normal((B, H, n, d), dtype=np.float32), dtype)
    q = to_device(qv)
    v = to_device(inp.quantize(np.broadcast_to(_pow2_rows(n, d), (B, H, n, d)).copy(), dtype))
    k = torch.zeros_like(q)
    out = nan_like((B, H, n, d), torch.float32)
    lse = nan_like((B, H, n), torch.float32)
    fa.forward(q, k, v, causal=causal, out=out, lse=lse, dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    o = host64(out)
    vis = np.tril(np.ones((n, n), dtype=bool)) if causal else np.ones((n, n), dtype=bool)
    l_rows = vis.sum(axis=1).astype(np.float64)
    for (b, h) in _spread_heads(B, H):
        z = dropout_keep_ref(n, n, b * H + h, seed, offset, p) & vis
        got = _digits(o[b, h] * l_rows[:, None], ks32)
        bad = np.argwhere(got != _mask_digits(z, d))
        assert bad.size == 0, f"head {(b, h)}: keep bits differ at (row, col) {bad[:5]}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96])
@pytest.mark.parametrize("causal", [False, True])
def test_full_grid_forward_dropout_parity(fa, dtype, d, causal):
    """Random inputs on a full-chip grid with dropout: O and LSE of 8 heads spread over the grid
    against the oracle (ragged N = 1000), every head finite."""
    import torch
    p, seed, offset = 0.15, 77, 4
    n = 1000
    B, H = _full_grid_heads(n, causal)
    print(f"  B={B} H={H} N={n}", flush=True)
    t = inp.draw((B, H, n, d), dtype, 5 * d + causal)
    q, k, v = (to_device(t[nm]) for nm in ("q", "k", "v"))
    out = nan_like((B, H, n, d), torch.float32)
    lse = nan_like((B, H, n), torch.float32)
    scale = 1.0 / math.sqrt(d)
    fa.forward(q, k, v, scale=scale, causal=causal, out=out, lse=lse, dropout_p=p, seed=seed,
               offset=offset)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    ks = keep_scale(p)
    for (b, h) in _spread_heads(B, H):
        keep = dropout_keep_ref(n, n, b * H + h, seed, offset, p)
        o_ref, l_ref = attn_fwd_ref(t["q"].values[b, h], t["k"].values[b, h],
                                    t["v"].values[b, h], scale, causal, keep=keep, keep_scale=ks)
        check("O", host64(out[b, h]), o_ref, 2e-2)
        check("LSE", host64(lse[b, h]), l_ref, 1e-3)

