"""Float64 CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke entry point and the benchmark's CPU-baseline leg may
import this module. The product path (the HIP library and its Python binding) never imports,
links or calls it, and this module imports nothing from the product path.

Sources (web pages on FlashAttention; cited by title and section):

* [FA-why]  "FlashAttention 为什么不需要存下注意力矩阵" (AIGC 基本功 series, jefxiong.cn):
  §03 3.1 (safe softmax and the row statistics m, l, O), §03 3.2 (the online-softmax
  recurrence, its initial state and the causal mask), §03 3.3 (the recompute backward),
  §04 4.1 (the per-block trace), §04 4.5 (causal whole-tile skip).
* [FA-V1]   "FlashAttention V1 技术深度解析" (spark.aweffr.cn): §2.1-2.2 (standard attention,
  S and P materialised), §3.3 (outer loop over K/V blocks, inner loop over Q blocks),
  §4.2 (backward recomputes S and P blocks from saved statistics).

Everything is float64 NumPy. Inputs are upcast exactly (bf16/fp16/fp32 values are exactly
representable in float64), so the oracle sees precisely the values the GPU sees.

Functions
---------
attn_fwd_ref    naive forward: S = scale*Q K^T, P = softmax(S) (row-wise, max-shifted), O = P V,
                LSE = m + log l (natural log of the scaled scores).
attn_bwd_ref    naive backward: dV = P^T dO, dP = dO V^T, D = rowsum(dP*P),
                dS = P*(dP - D), dQ = scale*dS K, dK = scale*dS^T Q.
attn_tiled_ref  the blockwise online-softmax recurrence in the pages' V1 loop order (outer K/V
                block, inner Q block), exposing the m / l / corr trajectory.
attn_rows_ref   the forward for a chosen subset of query rows, one row at a time, O(N d) per row.
attn_decode_ref Nq query rows (the last Nq positions) over Nk >= Nq keys: the decoding case.
attn_split_merge_ref  the same via per-chunk partial results merged by their LSEs (split-KV).

The forward and backward take an optional dropout keep mask (philox.py generates it from a seed
and an offset with the Philox-4x32-10 counter-based generator) and an optional visibility mask
for block-sparse attention (block_mask_to_elements expands a tile mask to elements).

Every function is pinned by tests that do not re-type its formula (see tests/test_oracle_pins.py):
a printed worked trace, closed forms, invariants, finite differences and brute force.
"""

from __future__ import annotations

import numpy as np

__all__ = ["attn_fwd_ref", "attn_bwd_ref", "attn_tiled_ref", "attn_rows_ref",
           "block_mask_to_elements", "attn_decode_ref", "attn_split_merge_ref"]


def _heads(x):
    """View a [..., N, d] array as float64 [G, N, d] (G = product of the leading dims)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim < 2:
        raise ValueError("expected an array of shape [..., N, d]")
    return x.reshape((-1,) + x.shape[-2:]), x.shape[:-2]


def _scores(qh, kh, scale, causal, visible=None):
    """S = scale * Q K^T for one head; with causal, key index j > query index i is -inf.

    [FA-V1] §2.2 step 1 (S = Q K^T, here with the softmax scale folded in, [FA-why] §03 3.3 uses
    1/sqrt(d)); the causal rule (masked score = -inf) is [FA-why] §03 3.2, last paragraph. With
    fewer query rows than keys (Nq < Nk) the queries are the last Nq positions: row i is at
    position i + Nk - Nq.
    `visible` (bool [N, N], optional) masks further: scores of invisible keys are -inf.
    """
    s = scale * (qh @ kh.T)
    if causal:
        n_q, n_k = s.shape
        if n_q > n_k:
            raise ValueError("causal attention with the queries at the end needs Nq <= Nk")
        s[np.triu(np.ones((n_q, n_k), dtype=bool), 1 + n_k - n_q)] = -np.inf
    if visible is not None:
        s[~np.asarray(visible, dtype=bool)] = -np.inf
    return s


def _visible_heads(visible, G, N):
    """Visibility mask as bool [G, N, N] (a single [N, N] mask applies to every head)."""
    if visible is None:
        return None
    vm = np.asarray(visible, dtype=bool)
    if vm.shape == (N, N):
        return np.broadcast_to(vm, (G, N, N))
    return vm.reshape((G, N, N))


def _softmax_rows(s):
    """Safe softmax along each row: m = max, l = sum exp(s - m), P = exp(s - m) / l.

    [FA-why] §03 3.1 (subtract the row maximum, then normalise by the sum of exponentials).
    A row whose scores are all -inf (no visible key, possible only with a block mask) gets
    P = 0, m = -inf and l = 0, so that its output is 0 and its LSE = m + log l = -inf.
    Returns P, m, l.
    """
    m = s.max(axis=1)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    p = e / np.where(empty, 1.0, l)[:, None]
    return p, m, l


def block_mask_to_elements(block_mask, n, block):
    """Element visibility [n, n] of a tile mask [ceil(n/block), ceil(n/block)]: query i may see
    key j iff block_mask[i // block][j // block] is nonzero ([FA-why] §06: the whole-block skip of
    the causal case, generalised to an arbitrary pattern of blocks, is block-sparse attention)."""
    bm = np.asarray(block_mask) != 0
    idx = np.arange(n) // block
    return bm[np.ix_(idx, idx)]


def _keep_heads(keep, G, N):
    """Dropout keep mask as bool [G, N, N] (None -> None)."""
    if keep is None:
        return None
    kp = np.asarray(keep, dtype=bool)
    return kp.reshape((G, N, N))


def attn_fwd_ref(q, k, v, scale, causal, keep=None, keep_scale=1.0, visible=None):
    """Naive attention with S and P materialised per (b, h).

    q, k, v: [..., N, d] (any real dtype; upcast to float64).
    Returns (O [..., N, d] float64, LSE [..., N] float64) where LSE = m + log(l) is the natural-log
    logsumexp of the *scaled* scores ([FA-why] §03 3.2: m + log l is the logsumexp).
    [FA-V1] §2.2 steps 1-3: S = QK^T, P = softmax(S), O = PV.

    Dropout ([FA-why] §05, fourth difference): with a keep mask Z ([..., N, N] bool) the output
    is O = (P * Z * keep_scale) V, applied to the normalised probabilities; LSE stays that of the
    undropped softmax (it only normalises P).

    Block-sparse attention ([FA-why] §06): `visible` ([N, N] or [..., N, N] bool, see
    block_mask_to_elements) hides keys from queries exactly like the causal rule; a query that
    sees no key at all has O = 0 and LSE = -inf.
    """
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    G, N, _ = qh.shape
    dv = vh.shape[-1]
    kp = _keep_heads(keep, G, N)
    vis = _visible_heads(visible, G, N)
    o = np.empty((G, N, dv))
    lse = np.empty((G, N))
    for g in range(G):
        s = _scores(qh[g], kh[g], scale, causal, None if vis is None else vis[g])
        p, m, l = _softmax_rows(s)
        if kp is not None:
            p = np.where(kp[g], p * keep_scale, 0.0)
        o[g] = p @ vh[g]
        with np.errstate(divide="ignore"):
            lse[g] = m + np.log(l)
    return o.reshape(lead + (N, dv)), lse.reshape(lead + (N,))


def attn_bwd_ref(q, k, v, do, scale, causal, o=None, keep=None, keep_scale=1.0, visible=None):
    """Naive backward of O = softmax(scale*Q K^T) V with the upstream gradient dO.

    [FA-why] §03 3.3: with G = dO and A = G V^T = dL/dP,
        dS = P * (A - rowsum(A * P))         (row sum broadcast along the key axis)
        dQ = dS K * scale,  dK = dS^T Q * scale,  dV = P^T G
    where the page's 1/sqrt(d) is the softmax scale (here an explicit argument).

    With a dropout keep mask Z (same mask as the forward, regenerated from seed and offset,
    [FA-why] §05): O = P_d V with P_d = P * Z * keep_scale, so by the chain rule
        dV = P_d^T G,  A = (G V^T) * Z * keep_scale = dL/dP,  and dS, dQ, dK as above.

    With a block-sparse visibility mask (`visible`, as in attn_fwd_ref), invisible keys have
    P = 0; a query that sees no key has zero gradients. k and v may hold Nk != N rows (the
    backward of attn_decode_ref: with causal, the N queries are the last positions).

    Returns dict with dq, dk, dv ([..., N, d]) and D = rowsum(dP * P) ([..., N]).
    If `o` (the forward output) is given, also returns D_o = rowsum(dO * O), which equals D in
    real arithmetic (with or without dropout); callers compare the two.
    """
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    doh, _ = _heads(do)
    G, N, d = qh.shape
    Nk = kh.shape[1]
    dq = np.empty_like(qh)
    dk = np.empty_like(kh)
    dv = np.empty_like(vh)
    D = np.empty((G, N))
    kp = _keep_heads(keep, G, N)
    vis = _visible_heads(visible, G, N)
    for g in range(G):
        s = _scores(qh[g], kh[g], scale, causal, None if vis is None else vis[g])
        p, _, _ = _softmax_rows(s)
        if kp is None:
            dv[g] = p.T @ doh[g]
            dp = doh[g] @ vh[g].T
        else:
            dv[g] = np.where(kp[g], p * keep_scale, 0.0).T @ doh[g]
            dp = np.where(kp[g], (doh[g] @ vh[g].T) * keep_scale, 0.0)
        D[g] = (dp * p).sum(axis=1)
        ds = p * (dp - D[g][:, None])
        dq[g] = scale * (ds @ kh[g])
        dk[g] = scale * (ds.T @ qh[g])
    out = {
        "dq": dq.reshape(lead + (N, d)),
        "dk": dk.reshape(lead + (Nk, d)),
        "dv": dv.reshape(lead + (Nk, vh.shape[-1])),
        "D": D.reshape(lead + (N,)),
    }
    if o is not None:
        oh, _ = _heads(o)
        out["D_o"] = (doh * oh).sum(axis=2).reshape(lead + (N,))
    return out


def _default_corr(m_old, m_new):
    """Rescale factor exp(m_old - m_new), defined as 0 when m_old is the initial -inf.

    [FA-why] §03 3.2: the first block's rescale factor is taken as 0 (the old accumulators are 0).
    """
    out = np.zeros_like(m_new)
    live = ~np.isneginf(m_old)
    out[live] = np.exp(m_old[live] - m_new[live])
    return out


def attn_tiled_ref(q, k, v, scale, causal, block_r, block_c, corr_fn=None, trace=False):
    """Online-softmax attention for ONE head, blockwise, in the pages' V1 loop order.

    q, k, v: [N, d]. Blocks: Q rows in blocks of `block_r`, K/V rows in blocks of `block_c`.
    Outer loop over K/V blocks, inner loop over Q blocks ([FA-V1] §3.3 steps 3-4). The state
    per query row is (m, l, O) with the invariants of [FA-why] §03 3.2:
        O = sum_j exp(s_j - m) v_j,  l = sum_j exp(s_j - m)   over the keys seen so far,
    initial m = -inf, l = 0, O = 0; for each new block with block maximum m_blk:
        m_new = max(m, m_blk);  corr = exp(m - m_new)  (0 when m = -inf)
        l <- corr*l + sum exp(s - m_new);  O <- corr*O + exp(s - m_new) V_blk;  m <- m_new.
    Result: O / l and LSE = m + log l.

    Causal: masked scores are -inf ([FA-why] §03 3.2) and a (Q block, K block) pair whose every
    query precedes every key (i0 + block_r <= j0) is skipped whole ([FA-why] §04 4.5).

    A row whose scores seen so far are all masked keeps m = -inf and contributes nothing (its
    exponentials are taken as 0); with keys visited in ascending order and N_q = N_k this never
    happens, because key 0 is visible to every query.

    corr_fn: optional replacement for the rescale rule (tests plant mutants through it).
    Returns (O [N,d], LSE [N], info) where info = {"tiles_kept", "tiles_total", "trace"};
    with trace=True, info["trace"] lists one dict per processed block pair:
    {"j0", "i0", "m": m_new[rows], "l": l_new[rows], "corr": corr[rows]} over the block's rows.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    corr_rule = _default_corr if corr_fn is None else corr_fn
    O = np.zeros((N, d))
    l = np.zeros(N)
    m = np.full(N, -np.inf)
    kept = 0
    total = 0
    steps = []
    for j0 in range(0, N, block_c):
        j1 = min(j0 + block_c, N)
        for i0 in range(0, N, block_r):
            i1 = min(i0 + block_r, N)
            total += 1
            if causal and i0 + block_r <= j0:
                continue
            kept += 1
            s = scale * (q[i0:i1] @ k[j0:j1].T)
            if causal:
                qi = np.arange(i0, i1)[:, None]
                kj = np.arange(j0, j1)[None, :]
                s = np.where(kj > qi, -np.inf, s)
            m_blk = s.max(axis=1)
            m_old = m[i0:i1].copy()
            m_new = np.maximum(m_old, m_blk)
            p = np.zeros_like(s)
            fin = ~np.isneginf(m_new)
            p[fin] = np.exp(s[fin] - m_new[fin][:, None])
            corr = corr_rule(m_old, m_new)
            l[i0:i1] = corr * l[i0:i1] + p.sum(axis=1)
            O[i0:i1] = corr[:, None] * O[i0:i1] + p @ v[j0:j1]
            m[i0:i1] = m_new
            if trace:
                steps.append({"j0": j0, "i0": i0, "m": m_new.copy(),
                              "l": l[i0:i1].copy(), "corr": np.asarray(corr).copy()})
    info = {"tiles_kept": kept, "tiles_total": total, "trace": steps}
    return O / l[:, None], m + np.log(l), info


def attn_rows_ref(q, k, v, scale, causal, rows):
    """Forward output and LSE for selected query rows of ONE head, one row at a time.

    q, k, v: [N, d]; rows: iterable of query indices. For row i the visible keys are 0..i when
    causal, else all N ([FA-why] §03 3.2 causal rule). Per row: s = scale*K q_i, m = max s,
    e = exp(s - m), l = sum e, o = (e V)/l, LSE = m + log l ([FA-why] §03 3.1, 3.2).
    Returns (O_rows [R, d], LSE_rows [R]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = [int(r) for r in rows]
    N, d = q.shape
    o = np.empty((len(rows), d))
    lse = np.empty(len(rows))
    for n, i in enumerate(rows):
        hi = i + 1 if causal else N
        s = scale * (k[:hi] @ q[i])
        mx = s.max()
        e = np.exp(s - mx)
        den = e.sum()
        o[n] = (e @ v[:hi]) / den
        lse[n] = mx + np.log(den)
    return o, lse


def attn_decode_ref(q, k, v, scale, causal):
    """Attention of Nq query rows over Nk keys (decoding, N_q << N_k; chunked prefill; or, not
    causal, any cross-attention).

    q: [..., Nq, d]; k, v: [..., Nk, d]. Same definition as attn_fwd_ref ([FA-V1] §2.2 steps
    1-3, [FA-why] §03 3.1) with the queries taken as the LAST Nq positions of the sequence: when
    causal (which needs Nq <= Nk), query i (0-based among the Nq) sees keys j <= Nk - Nq + i, the
    top-left rule of [FA-why] §03 3.2 when Nq = Nk; otherwise every query sees all Nk keys.
    Returns (O [..., Nq, d], LSE [..., Nq]).
    """
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    G, nq, _ = qh.shape
    nk = kh.shape[1]
    if causal and nq > nk:
        raise ValueError("causal attention with the queries at the end needs Nq <= Nk")
    o = np.empty((G, nq, vh.shape[-1]))
    lse = np.empty((G, nq))
    for g in range(G):
        s = scale * (qh[g] @ kh[g].T)
        if causal:
            qi = np.arange(nq)[:, None] + (nk - nq)
            s[np.arange(nk)[None, :] > qi] = -np.inf
        p, m, l = _softmax_rows(s)
        o[g] = p @ vh[g]
        lse[g] = m + np.log(l)
    return o.reshape(lead + (nq, vh.shape[-1])), lse.reshape(lead + (nq,))


def attn_split_merge_ref(q, k, v, scale, causal, chunk):
    """Split-KV decoding: attention over each chunk of `chunk` keys separately, then one merge.

    Per chunk c the partial result is (O_c, LSE_c) = attention restricted to the chunk's keys
    (a chunk that a query cannot see has LSE_c = -inf and weight 0). The merge is the rescale of
    the online-softmax recurrence applied to whole chunks ([FA-why] §03 3.2: the result does not
    depend on how the keys are blocked):  LSE = log sum_c exp(LSE_c),
    O = sum_c exp(LSE_c - LSE) O_c. Flash-Decoding is named, without details, in
    "FlashAttention V1 技术深度解析" (conclusion) and "Flash Attention：一个数学技巧把内存省 5 倍" §七.
    q: [..., Nq, d], k, v: [..., Nk, d]. Returns (O, LSE) like attn_decode_ref.
    """
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    G, nq, _ = qh.shape
    nk = kh.shape[1]
    starts = list(range(0, nk, chunk))
    o = np.zeros((G, nq, vh.shape[-1]))
    lse = np.empty((G, nq))
    for g in range(G):
        parts = []
        for j0 in starts:
            j1 = min(j0 + chunk, nk)
            s = scale * (qh[g] @ kh[g][j0:j1].T)
            if causal:
                qi = np.arange(nq)[:, None] + (nk - nq)
                s[np.arange(j0, j1)[None, :] > qi] = -np.inf
            p, m, l = _softmax_rows(s)
            with np.errstate(divide="ignore"):
                parts.append((p @ vh[g][j0:j1], m + np.log(l)))
        lses = np.stack([pl for _, pl in parts])           # [C, nq]
        top = lses.max(axis=0)
        w = np.exp(lses - top[None, :])                    # exp(-inf) = 0 for empty chunks
        tot = w.sum(axis=0)
        lse[g] = top + np.log(tot)
        for (po, _), wc in zip(parts, w):
            o[g] += (wc / tot)[:, None] * po
    return o.reshape(lead + (nq, vh.shape[-1])), lse.reshape(lead + (nq,))
