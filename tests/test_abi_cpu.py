"""The C ABI without a GPU: the library loads, exports what include/fa.h declares, and rejects
invalid calls with the documented status before any HIP call (fake, never-dereferenced device
pointers are safe here because validation precedes every launch)."""

import ctypes
import os
import re

import pytest

from exact_attention_94_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

P = 0x100000  # fake 16-byte-aligned device addresses (never dereferenced)


def _r256(x):
    return (x + 255) // 256 * 256


def ws_expected(B_, H, nq, nk, d, bf16, f32=False):
    """Workspace bytes of the backward as include/fa.h documents them: D (fp32 [B,H,Nq]), the dO
    scale (fp32 [B,H]), 256 partial maxima per head, a flag word, each section 256-byte aligned,
    then the fp16 copies of 16-bit inputs: dO always, Q, K and V for bf16 inputs (fp32 inputs:
    none)."""
    bh = B_ * H
    head = _r256(4 * bh * nq) + _r256(4 * bh) + _r256(4 * 256 * bh) + 256
    copies = 0 if f32 else bh * nq * d + ((bh * nq * d + 2 * bh * nk * d) if bf16 else 0)
    return head + 2 * copies


def _lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libfa.so is not built (run python -m exact_attention_94_amd.build)")
    return B.load()


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?)\b(fa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = _lib()
    names = ["FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE",
             "FA_ERR_HIP", "FA_ERR_RANGE"]
    for code, name in enumerate(names):
        s = lib.fa_status_string(code).decode()
        assert s.startswith(name)
        assert getattr(B, name) == code
        assert re.search(rf"\b{name}\s*=\s*{code}\b", open(HEADER, encoding="utf-8").read())
    assert "unknown" in lib.fa_status_string(99).decode()


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, N=100, d=64, scale=0.125, causal=1,
             in_dtype=B.FA_BF16, o_dtype=B.FA_BF16)
    a.update(kw)
    return _lib().fa_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                             a["d"], a["scale"], a["causal"], a["in_dtype"], a["o_dtype"], None)


def bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=2, H=3, N=100, d=64,
             scale=0.125, causal=1, in_dtype=B.FA_BF16, o_dtype=B.FA_F32, g_dtype=B.FA_F32,
             ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return _lib().fa_backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                              a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                              a["causal"], a["in_dtype"], a["o_dtype"], a["g_dtype"], a["ws"],
                              a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.FA_ERR_INVALID_ARG),
    (dict(lse=None), B.FA_ERR_INVALID_ARG),
    (dict(v=P + 8), B.FA_ERR_INVALID_ARG),
    (dict(N=0), B.FA_ERR_INVALID_ARG),
    (dict(B=-1), B.FA_ERR_INVALID_ARG),
    (dict(B=1 << 16, H=1 << 10, N=1 << 10), B.FA_ERR_INVALID_ARG),
    (dict(B=1, H=1, N=(1 << 24) + 1), B.FA_ERR_INVALID_ARG),
    # N*d = 2^30: a head of fp32 O would span exactly 4 GiB, past a 32-bit buffer range.
    (dict(B=1, H=1, N=1 << 24), B.FA_ERR_INVALID_ARG),
    (dict(B=1, H=1, N=(1 << 23), d=128), B.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), B.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), B.FA_ERR_INVALID_ARG),
    (dict(causal=2), B.FA_ERR_INVALID_ARG),
    (dict(in_dtype=7), B.FA_ERR_INVALID_ARG),
    (dict(d=80), B.FA_ERR_UNSUPPORTED),
    (dict(d=16), B.FA_ERR_UNSUPPORTED),
    (dict(d=512), B.FA_ERR_UNSUPPORTED),
    (dict(d=256, in_dtype=B.FA_F32, o_dtype=B.FA_F32), B.FA_ERR_UNSUPPORTED),
    (dict(o_dtype=B.FA_F16), B.FA_ERR_UNSUPPORTED),
    (dict(in_dtype=B.FA_F32, o_dtype=B.FA_BF16), B.FA_ERR_UNSUPPORTED),
])
def test_forward_rejects(kw, status):
    assert fwd(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dq=None), B.FA_ERR_INVALID_ARG),
    (dict(do=P + 4), B.FA_ERR_INVALID_ARG),
    (dict(N=0), B.FA_ERR_INVALID_ARG),
    (dict(B=1, H=1, N=1 << 24), B.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), B.FA_ERR_INVALID_ARG),
    (dict(causal=-1), B.FA_ERR_INVALID_ARG),
    (dict(g_dtype=5), B.FA_ERR_INVALID_ARG),
    (dict(d=256, in_dtype=B.FA_F32, o_dtype=B.FA_F32), B.FA_ERR_UNSUPPORTED),
    # d = 256 (16-bit) passes the checks and reaches the workspace check.
    (dict(d=256, ws=None), B.FA_ERR_WORKSPACE),
    (dict(in_dtype=B.FA_F32, o_dtype=B.FA_F32, g_dtype=B.FA_F16), B.FA_ERR_UNSUPPORTED),
    (dict(in_dtype=B.FA_F32, o_dtype=B.FA_BF16), B.FA_ERR_UNSUPPORTED),
    # fp32 inputs pass the dtype checks and reach the workspace check.
    (dict(in_dtype=B.FA_F32, o_dtype=B.FA_F32, ws=None), B.FA_ERR_WORKSPACE),
    (dict(in_dtype=B.FA_F32, o_dtype=B.FA_F32,
          ws_bytes=ws_expected(2, 3, 100, 100, 64, False, f32=True) - 1), B.FA_ERR_WORKSPACE),
    (dict(g_dtype=B.FA_F16), B.FA_ERR_UNSUPPORTED),
    (dict(o_dtype=B.FA_F16), B.FA_ERR_UNSUPPORTED),
    (dict(ws=None), B.FA_ERR_WORKSPACE),
    (dict(ws=P + 2), B.FA_ERR_WORKSPACE),
    (dict(ws_bytes=16), B.FA_ERR_WORKSPACE),
    (dict(g_dtype=B.FA_BF16, ws_bytes=2 * 3 * 100 * 4 + 256), B.FA_ERR_WORKSPACE),
    (dict(in_dtype=B.FA_F16, o_dtype=B.FA_F32,
          ws_bytes=ws_expected(2, 3, 100, 100, 64, False) - 1), B.FA_ERR_WORKSPACE),
    (dict(ws_bytes=ws_expected(2, 3, 100, 100, 64, True) - 1), B.FA_ERR_WORKSPACE),
])
def test_backward_rejects(kw, status):
    assert bwd(**kw) == status


def fwd_drop(p=0.1, seed=1, offset=0, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, N=100, d=64, scale=0.125, causal=1,
             in_dtype=B.FA_BF16, o_dtype=B.FA_BF16)
    a.update(kw)
    return _lib().fa_forward_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                     a["N"], a["d"], a["scale"], a["causal"], a["in_dtype"],
                                     a["o_dtype"], p, seed, offset, None)


def bwd_drop(p=0.1, seed=1, offset=0, **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=2, H=3, N=100, d=64,
             scale=0.125, causal=1, in_dtype=B.FA_BF16, o_dtype=B.FA_F32, g_dtype=B.FA_F32,
             ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return _lib().fa_backward_dropout(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                      a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"],
                                      a["scale"], a["causal"], a["in_dtype"], a["o_dtype"],
                                      a["g_dtype"], p, seed, offset, a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("p", [-0.1, 1.0, 1.5, float("nan"), float("inf"), 0.99999999])
def test_dropout_rejects_bad_probability(p):
    # 0.99999999 rounds to 1.0 in float32: nothing would be kept.
    assert fwd_drop(p=p) == B.FA_ERR_INVALID_ARG
    assert bwd_drop(p=p) == B.FA_ERR_INVALID_ARG


def test_dropout_rejects_like_the_plain_calls():
    assert fwd_drop(q=None) == B.FA_ERR_INVALID_ARG
    assert fwd_drop(d=80) == B.FA_ERR_UNSUPPORTED
    assert fwd_drop(d=256) == B.FA_ERR_UNSUPPORTED  # d = 256: plain forward only
    # The fp32 forward has no dropout instance.
    assert fwd_drop(in_dtype=B.FA_F32, o_dtype=B.FA_F32) == B.FA_ERR_UNSUPPORTED
    assert bwd_drop(ws=None) == B.FA_ERR_WORKSPACE
    assert bwd_drop(in_dtype=B.FA_F32, o_dtype=B.FA_F32) == B.FA_ERR_UNSUPPORTED
    assert bwd_drop(causal=3) == B.FA_ERR_INVALID_ARG


def fwd_sparse(mask=P, heads=1, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, N=300, d=64, scale=0.125, causal=0,
             in_dtype=B.FA_F16, o_dtype=B.FA_F16)
    a.update(kw)
    return _lib().fa_forward_blocksparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                         a["H"], a["N"], a["d"], a["scale"], a["causal"],
                                         a["in_dtype"], a["o_dtype"], mask, heads, None)


def bwd_sparse(mask=P, heads=1, **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=2, H=3, N=300, d=64,
             scale=0.125, causal=0, in_dtype=B.FA_BF16, o_dtype=B.FA_F32, g_dtype=B.FA_F32,
             ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return _lib().fa_backward_blocksparse(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"],
                                          a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["N"],
                                          a["d"], a["scale"], a["causal"], a["in_dtype"],
                                          a["o_dtype"], a["g_dtype"], mask, heads, a["ws"],
                                          a["ws_bytes"], None)


@pytest.mark.parametrize("call", [fwd_sparse, bwd_sparse])
def test_blocksparse_rejects(call):
    assert call(mask=None) == B.FA_ERR_INVALID_ARG
    assert call(heads=2) == B.FA_ERR_INVALID_ARG  # neither 1 nor B*H = 6
    assert call(heads=0) == B.FA_ERR_INVALID_ARG
    assert call(N=65537, B=1, H=1) == B.FA_ERR_UNSUPPORTED
    assert call(in_dtype=B.FA_F32, o_dtype=B.FA_F32) == B.FA_ERR_UNSUPPORTED
    assert call(d=80) == B.FA_ERR_UNSUPPORTED
    assert call(d=256) == B.FA_ERR_UNSUPPORTED
    assert call(N=0) == B.FA_ERR_INVALID_ARG
    assert call(q=None, heads=6) == B.FA_ERR_INVALID_ARG


def dec(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, Nq=1, Nk=1000, d=128, scale=0.1, causal=0,
             in_dtype=B.FA_BF16, o_dtype=B.FA_BF16, ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return _lib().fa_decode_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                    a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                                    a["in_dtype"], a["o_dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.FA_ERR_INVALID_ARG),
    (dict(k=P + 8), B.FA_ERR_INVALID_ARG),
    (dict(Nq=0), B.FA_ERR_INVALID_ARG),
    (dict(Nk=0), B.FA_ERR_INVALID_ARG),
    (dict(Nq=4, Nk=3), B.FA_ERR_INVALID_ARG),
    (dict(Nq=5), B.FA_ERR_UNSUPPORTED),
    (dict(d=96), B.FA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), B.FA_ERR_INVALID_ARG),
    (dict(causal=2), B.FA_ERR_INVALID_ARG),
    (dict(in_dtype=B.FA_F32, o_dtype=B.FA_F32), B.FA_ERR_UNSUPPORTED),
    (dict(o_dtype=B.FA_F16), B.FA_ERR_UNSUPPORTED),
    (dict(ws=None), B.FA_ERR_WORKSPACE),
    (dict(ws_bytes=100), B.FA_ERR_WORKSPACE),
    (dict(B=1, H=1, Nk=(1 << 23) + 1), B.FA_ERR_INVALID_ARG),
    (dict(B=1, H=1, Nk=1 << 23), B.FA_ERR_INVALID_ARG),
])
def test_decode_rejects(kw, status):
    assert dec(**kw) == status


def test_decode_workspace_bytes():
    lib = _lib()
    ws = lib.fa_decode_workspace_bytes
    # 6 heads, Nk = 1000: the plan asks for ceil(2048 / 6) = 342 chunks but at least 256 keys
    # each -> 4 chunks; chunk = 250 rounded up to 256 -> ceil(1000 / 256) = 4 chunks.
    # Nq = 1: one slot; O partials 6*4*1*128 floats, then 6*4*1*2 floats, 256-byte sections.
    assert ws(2, 3, 1, 1000, 128) == 12288 + 256
    # Nq = 2..4 use four query slots.
    assert ws(2, 3, 3, 1000, 128) == 4 * 12288 + 768
    assert ws(2, 3, 5, 1000, 128) == 0
    assert ws(2, 3, 1, 1000, 96) == 0
    assert ws(2, 3, 2, 1, 64) == 0
    need = ws(2, 3, 1, 1000, 128)
    assert dec(ws_bytes=need - 1) == B.FA_ERR_WORKSPACE


def fwd_kv(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, Nq=100, Nk=300, d=64, scale=0.125, causal=1,
             in_dtype=B.FA_BF16, o_dtype=B.FA_BF16)
    a.update(kw)
    return _lib().fa_forward_kv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["in_dtype"],
                                a["o_dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Nq=301), B.FA_ERR_INVALID_ARG),          # causal needs Nq <= Nk
    (dict(Nk=0), B.FA_ERR_INVALID_ARG),
    (dict(Nq=0), B.FA_ERR_INVALID_ARG),
    (dict(k=None), B.FA_ERR_INVALID_ARG),
    (dict(in_dtype=B.FA_F32, o_dtype=B.FA_F32), B.FA_ERR_UNSUPPORTED),
    (dict(d=80), B.FA_ERR_UNSUPPORTED),
    (dict(B=1, H=1, Nk=(1 << 24) + 1), B.FA_ERR_INVALID_ARG),
])
def test_forward_kv_rejects(kw, status):
    assert fwd_kv(**kw) == status


def bwd_kv(**kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=2, H=3, Nq=100, Nk=300, d=64,
             scale=0.125, causal=1, in_dtype=B.FA_BF16, o_dtype=B.FA_F32, g_dtype=B.FA_F32,
             ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return _lib().fa_backward_kv(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                 a["dk"], a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                                 a["scale"], a["causal"], a["in_dtype"], a["o_dtype"],
                                 a["g_dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Nq=301), B.FA_ERR_INVALID_ARG),          # causal needs Nq <= Nk
    (dict(Nk=0), B.FA_ERR_INVALID_ARG),
    (dict(Nq=0), B.FA_ERR_INVALID_ARG),
    (dict(dk=None), B.FA_ERR_INVALID_ARG),
    (dict(dv=P + 4), B.FA_ERR_INVALID_ARG),
    (dict(in_dtype=B.FA_F32, o_dtype=B.FA_F32), B.FA_ERR_UNSUPPORTED),
    (dict(d=256, ws=None), B.FA_ERR_WORKSPACE),  # d = 256 is provided (16-bit)
    (dict(d=80), B.FA_ERR_UNSUPPORTED),
    (dict(B=1, H=1, Nk=(1 << 24) + 1), B.FA_ERR_INVALID_ARG),
    (dict(ws=None), B.FA_ERR_WORKSPACE),
    # Q / dO copies over Nq rows, K / V copies over Nk rows: one byte short is rejected.
    (dict(ws_bytes=ws_expected(2, 3, 100, 300, 64, True) - 1), B.FA_ERR_WORKSPACE),
])
def test_backward_kv_rejects(kw, status):
    assert bwd_kv(**kw) == status


def test_backward_kv_workspace_bytes():
    lib = _lib()
    ws = lib.fa_backward_kv_workspace_bytes
    assert ws(2, 3, 100, 300, 64, B.FA_F16, B.FA_F32) == ws_expected(2, 3, 100, 300, 64, False)
    assert ws(2, 3, 100, 300, 64, B.FA_BF16, B.FA_F32) == ws_expected(2, 3, 100, 300, 64, True)
    # Non-causal calls may have more queries than keys.
    assert ws(1, 1, 300, 17, 32, B.FA_BF16, B.FA_BF16) == ws_expected(1, 1, 300, 17, 32, True)
    for n in (1, 100, 4099):
        for dt in (B.FA_F16, B.FA_BF16):
            assert ws(2, 3, n, n, 96, dt, B.FA_F32) == \
                lib.fa_backward_workspace_bytes(2, 3, n, 96, dt, B.FA_F32)
    assert ws(1, 1, 10, 10, 256, B.FA_F16, B.FA_F32) == ws_expected(1, 1, 10, 10, 256, False)
    assert ws(1, 1, 10, 0, 64, B.FA_F16, B.FA_F32) == 0
    assert ws(1, 1, 10, 10, 64, B.FA_F16, 9) == 0
    # Pairs fa_backward_kv rejects get 0, as the header promises.
    assert ws(1, 1, 10, 20, 64, B.FA_BF16, B.FA_F16) == 0


def test_workspace_bytes():
    lib = _lib()
    ws = lib.fa_backward_workspace_bytes
    assert ws(2, 3, 100, 64, B.FA_F16, B.FA_F32) == ws_expected(2, 3, 100, 100, 64, False)
    assert ws(2, 3, 100, 64, B.FA_F16, B.FA_F16) == ws_expected(2, 3, 100, 100, 64, False)
    assert ws(2, 3, 100, 64, B.FA_BF16, B.FA_F32) == ws_expected(2, 3, 100, 100, 64, True)
    assert ws(2, 3, 100, 64, B.FA_BF16, B.FA_BF16) == ws_expected(2, 3, 100, 100, 64, True)
    assert ws(1, 1, 1, 128, B.FA_F16, B.FA_F16) == ws_expected(1, 1, 1, 1, 128, False)
    assert ws(1, 1, 1, 80, B.FA_F16, B.FA_F32) == 0
    assert ws(1, 1, 1, 256, B.FA_F16, B.FA_F32) == ws_expected(1, 1, 1, 1, 256, False)
    assert ws(1, 1, 1, 256, B.FA_F32, B.FA_F32) == 0  # no fp32 attention at d = 256
    # Head dims 32 and 96 are provided; the workspace depends on d only through the copies.
    assert ws(1, 1, 1, 96, B.FA_F16, B.FA_F32) == ws_expected(1, 1, 1, 1, 96, False)
    assert ws(1, 2, 10, 32, B.FA_BF16, B.FA_F32) == ws_expected(1, 2, 10, 10, 32, True)
    assert ws(0, 1, 1, 64, B.FA_F16, B.FA_F32) == 0
    assert ws(1, 1, 1, 64, B.FA_F16, 9) == 0
    assert ws(1, 1, 1, 64, 9, B.FA_F32) == 0
    # Every dtype pair fa_backward rejects gets 0: 16-bit gradients of the other 16-bit type.
    assert ws(1, 1, 8, 64, B.FA_BF16, B.FA_F16) == 0
    assert ws(1, 1, 8, 64, B.FA_F16, B.FA_BF16) == 0
    assert ws(1, 1, 8, 64, B.FA_F32, B.FA_F16) == 0
    assert ws(1, 1, 8, 64, B.FA_F32, B.FA_BF16) == 0
    # fp32 inputs need no operand copies.
    assert ws(2, 3, 100, 64, B.FA_F32, B.FA_F32) == ws_expected(2, 3, 100, 100, 64, False, True)


def test_exact_workspace_size_is_accepted_by_validation():
    """With exactly the advertised bytes, validation passes (the call then needs a GPU, so the
    only acceptable outcomes here are FA_OK on a GPU machine or FA_ERR_HIP without one)."""
    lib = _lib()
    need = lib.fa_backward_workspace_bytes(2, 3, 100, 64, B.FA_BF16, B.FA_BF16)
    st = bwd(g_dtype=B.FA_BF16, ws_bytes=need - 1)
    assert st == B.FA_ERR_WORKSPACE


def test_binding_fails_loudly_without_library(tmp_path):
    saved = B._lib
    try:
        B._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            B.load(str(tmp_path / "missing.so"))
    finally:
        B._lib = saved


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "exact_attention_94_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b|oracle[/.]attention|"
                                     r"attn_(fwd|bwd|tiled|rows)_ref", text, re.M), \
                    os.path.join(dirpath, f)


def bwd_timed(ev0=P, ev1=P, **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=2, H=3, N=100, d=64,
             scale=0.125, causal=1, in_dtype=B.FA_BF16, o_dtype=B.FA_F32, g_dtype=B.FA_F32,
             ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return _lib().fa_backward_timed(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                    a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"],
                                    a["scale"], a["causal"], a["in_dtype"], a["o_dtype"],
                                    a["g_dtype"], a["ws"], a["ws_bytes"], None, ev0, ev1)


def test_timed_backward_rejects_before_any_hip_call():
    """fa_backward_timed needs both events, takes 16-bit inputs only, and otherwise validates
    exactly like fa_backward (every case below returns before a HIP call or launch)."""
    assert bwd_timed(ev0=None) == B.FA_ERR_INVALID_ARG
    assert bwd_timed(ev1=None) == B.FA_ERR_INVALID_ARG
    assert bwd_timed(in_dtype=B.FA_F32, o_dtype=B.FA_F32) == B.FA_ERR_UNSUPPORTED
    assert bwd_timed(N=0) == B.FA_ERR_INVALID_ARG
    assert bwd_timed(dq=None) == B.FA_ERR_INVALID_ARG
    assert bwd_timed(d=80) == B.FA_ERR_UNSUPPORTED
    assert bwd_timed(ws=None) == B.FA_ERR_WORKSPACE
    assert bwd_timed(ws_bytes=16) == B.FA_ERR_WORKSPACE


def test_decode_noalloc_rejects():
    """The allocation-free decoding entry point validates like fa_decode_forward and refuses calls
    whose partials would not fit its fixed device scratch, before any HIP call."""
    lib = _lib()
    f = lib.fa_decode_forward_noalloc

    def call(**kw):
        a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=1, Nk=100, d=64, scale=0.125, causal=1,
                 in_dtype=B.FA_BF16, o_dtype=B.FA_BF16)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                 a["d"], a["scale"], a["causal"], a["in_dtype"], a["o_dtype"], None)

    assert call(q=None) == B.FA_ERR_INVALID_ARG
    assert call(lse=P + 4) == B.FA_ERR_INVALID_ARG
    assert call(Nq=5) == B.FA_ERR_UNSUPPORTED
    assert call(Nq=3, Nk=2) == B.FA_ERR_INVALID_ARG
    assert call(d=32) == B.FA_ERR_UNSUPPORTED
    assert call(in_dtype=B.FA_F32, o_dtype=B.FA_F32) == B.FA_ERR_UNSUPPORTED
    assert call(scale=float("inf")) == B.FA_ERR_INVALID_ARG
    big = dict(B=64, H=128, Nq=4, Nk=256, d=128)
    assert lib.fa_decode_workspace_bytes(64, 128, 4, 256, 128) > B.DECODE_SCRATCH_BYTES
    assert call(**big) == B.FA_ERR_WORKSPACE
    assert re.search(r"#define\s+FA_DECODE_SCRATCH_BYTES\s+\(8u\s*<<\s*20\)",
                     open(HEADER, encoding="utf-8").read())
