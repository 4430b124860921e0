"""Thin ctypes binding over libfa.so (the C ABI declared in include/fa.h).

Argument marshalling only: every step of the computation runs in the HIP library. PyTorch is
used for device memory and the current stream. If the library is not built, every call raises
(there is no fallback implementation).
"""

from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_RANGE = range(6)
FA_F32, FA_F16, FA_BF16 = 0, 1, 2

# Every symbol include/fa.h declares.
EXPORTS = ("fa_forward", "fa_forward_dropout", "fa_forward_blocksparse", "fa_forward_kv",
           "fa_backward", "fa_backward_kv", "fa_backward_kv_workspace_bytes",
           "fa_backward_dropout", "fa_backward_blocksparse", "fa_backward_workspace_bytes",
           "fa_decode_workspace_bytes", "fa_decode_forward", "fa_decode_forward_noalloc",
           "fa_backward_timed", "fa_status_string")

DECODE_SCRATCH_BYTES = 8 << 20  # FA_DECODE_SCRATCH_BYTES

SPARSE_BLOCK = 128  # queries x keys covered by one block-mask byte (FA_SPARSE_BLOCK)

_lib = None


class FAError(RuntimeError):
    """A non-FA_OK status returned by the library."""

    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load(path=LIB_PATH):
    """Load libfa.so once and declare the C signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP attention library not built: {path} is missing "
                           "(run python -m exact_attention_94_amd.build)")
    # torch provides the device memory and streams: its HIP runtime must be loaded first so that
    # the library binds to the same one (otherwise torch's stream handles mean nothing to it).
    _torch()
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp]
    lib.fa_forward.restype = i
    u64, u32 = ctypes.c_uint64, ctypes.c_uint32
    lib.fa_forward_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, f, u64, u32, vp]
    lib.fa_forward_dropout.restype = i
    lib.fa_forward_blocksparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp, i, vp]
    lib.fa_forward_blocksparse.restype = i
    lib.fa_forward_kv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.fa_forward_kv.restype = i
    lib.fa_backward_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_backward_workspace_bytes.restype = sz
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, i,
                                vp, sz, vp]
    lib.fa_backward.restype = i
    lib.fa_backward_kv_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.fa_backward_kv_workspace_bytes.restype = sz
    lib.fa_backward_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i,
                                   i, vp, sz, vp]
    lib.fa_backward_kv.restype = i
    lib.fa_backward_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i,
                                        i, f, u64, u32, vp, sz, vp]
    lib.fa_backward_dropout.restype = i
    lib.fa_backward_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i,
                                            i, i, i, vp, i, vp, sz, vp]
    lib.fa_backward_blocksparse.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.fa_decode_forward.restype = i
    lib.fa_decode_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.fa_decode_forward_noalloc.restype = i
    lib.fa_backward_timed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i,
                                      i, vp, sz, vp, vp, vp]
    lib.fa_backward_timed.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status):
    return load().fa_status_string(int(status)).decode()


def _torch():
    import torch
    return torch


def dtype_code(dt):
    torch = _torch()
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if dt not in codes:
        raise TypeError(f"unsupported tensor dtype {dt}")
    return codes[dt]


def _check_bhnd(name, t, shape=None):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(t):
    return ctypes.c_void_p(_torch().cuda.current_stream(t.device).cuda_stream)


def _check_mask(block_mask, q):
    B, H, N, _ = q.shape
    nb = (N + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    if block_mask.dtype != _torch().uint8 or not block_mask.is_cuda:
        raise TypeError("block_mask must be a uint8 GPU tensor")
    if not block_mask.is_contiguous():
        raise ValueError("block_mask must be contiguous")
    if block_mask.dim() == 2:
        heads = 1
        shape = (nb, nb)
    else:
        heads = block_mask.shape[0]
        shape = (heads, nb, nb)
    if tuple(block_mask.shape) != shape or heads not in (1, B * H):
        raise ValueError(f"block_mask has shape {tuple(block_mask.shape)}; expected [{nb}, {nb}] "
                         f"or [1 or B*H, {nb}, {nb}]")
    return heads


def forward(q, k, v, scale=None, causal=False, o_dtype=None, out=None, lse=None,
            dropout_p=None, seed=0, offset=0, block_mask=None):
    """fa_forward on torch tensors [B, H, N, d]. Returns (O, LSE).

    scale defaults to 1/sqrt(d); o_dtype defaults to the input dtype (float32 is also allowed for
    16-bit inputs). `out` / `lse` may be given to write into existing buffers. With dropout_p
    (not None) the call is fa_forward_dropout with that probability, `seed` and `offset`. With
    block_mask (a uint8 GPU tensor [nb, nb] or [1 or B*H, nb, nb], nb = ceil(N / 128)) the call
    is fa_forward_blocksparse. If k and v have another length Nk than q (shape [B, H, Nk, d]),
    the call is fa_forward_kv: with causal, the queries are the last positions of the Nk keys.
    """
    torch = _torch()
    _check_bhnd("q", q)
    _check_bhnd("k", k)
    _check_bhnd("v", v, k.shape)
    if tuple(k.shape[:2]) != tuple(q.shape[:2]) or k.shape[3] != q.shape[3]:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [B, H, Nk, d] with q's B, H, d")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    B, H, N, d = q.shape
    Nk = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o_dtype = q.dtype if o_dtype is None else o_dtype
    if out is None:
        out = torch.empty((B, H, N, d), dtype=o_dtype, device=q.device)
    else:
        _check_bhnd("out", out, q.shape)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
            scale, int(bool(causal)), dtype_code(q.dtype), dtype_code(out.dtype))
    if dropout_p is not None and block_mask is not None:
        raise ValueError("dropout and a block mask cannot be combined")
    if Nk != N:
        if dropout_p is not None or block_mask is not None:
            raise ValueError("dropout and block masks need Nk = Nq")
        st = load().fa_forward_kv(*args[:8], Nk, *args[8:], _stream(q))
        where = "fa_forward_kv"
    elif block_mask is not None:
        heads = _check_mask(block_mask, q)
        st = load().fa_forward_blocksparse(*args, block_mask.data_ptr(), heads, _stream(q))
        where = "fa_forward_blocksparse"
    elif dropout_p is None:
        st = load().fa_forward(*args, _stream(q))
        where = "fa_forward"
    else:
        st = load().fa_forward_dropout(*args, float(dropout_p), int(seed), int(offset), _stream(q))
        where = "fa_forward_dropout"
    if st != FA_OK:
        raise FAError(st, where)
    return out, lse


def workspace_bytes(B, H, N, d, in_dtype_code, grad_dtype_code):
    return int(load().fa_backward_workspace_bytes(B, H, N, d, in_dtype_code, grad_dtype_code))


def backward(q, k, v, o, dout, lse, scale=None, causal=False, grad_dtype=None, workspace=None,
             grads=None, dropout_p=None, seed=0, offset=0, block_mask=None, main_events=None):
    """fa_backward on torch tensors. Returns (dQ, dK, dV) in grad_dtype (default: q.dtype).

    `workspace` (a uint8 GPU tensor) is allocated when not given; `grads` may supply the three
    output tensors. With dropout_p (not None) the call is fa_backward_dropout, which regenerates
    the forward's keep mask from the same (dropout_p, seed, offset); with block_mask it is
    fa_backward_blocksparse (the mask given to the forward). If k and v have another length Nk
    than q, the call is fa_backward_kv (the backward of fa_forward_kv); dK and dV are then
    [B, H, Nk, d]. main_events (two hipEvent_t handles as ints; plain attention only) makes the
    call fa_backward_timed, which records them around the dK/dV kernel.
    """
    torch = _torch()
    for name, t in (("q", q), ("o", o), ("dout", dout)):
        _check_bhnd(name, t, q.shape)
    _check_bhnd("k", k)
    _check_bhnd("v", v, k.shape)
    if tuple(k.shape[:2]) != tuple(q.shape[:2]) or k.shape[3] != q.shape[3]:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [B, H, Nk, d] with q's B, H, d")
    B, H, N, d = q.shape
    Nk = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    gcode = dtype_code(grad_dtype)
    if grads is None:
        grads = (torch.empty((B, H, N, d), dtype=grad_dtype, device=q.device),
                 torch.empty((B, H, Nk, d), dtype=grad_dtype, device=q.device),
                 torch.empty((B, H, Nk, d), dtype=grad_dtype, device=q.device))
    dq, dk, dv = grads
    _check_bhnd("dq", dq, q.shape)
    _check_bhnd("dk", dk, k.shape)
    _check_bhnd("dv", dv, k.shape)
    if Nk != N:
        need = int(load().fa_backward_kv_workspace_bytes(B, H, N, Nk, d, dtype_code(q.dtype),
                                                         gcode))
    else:
        need = workspace_bytes(B, H, N, d, dtype_code(q.dtype), gcode)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale,
            int(bool(causal)), dtype_code(q.dtype), dtype_code(o.dtype), gcode)
    if dropout_p is not None and block_mask is not None:
        raise ValueError("dropout and a block mask cannot be combined")
    if main_events is not None:
        if Nk != N or dropout_p is not None or block_mask is not None:
            raise ValueError("main_events times plain self-attention only")
        st = load().fa_backward_timed(*args, workspace.data_ptr(), workspace.numel(), _stream(q),
                                      int(main_events[0]), int(main_events[1]))
        if st != FA_OK:
            raise FAError(st, "fa_backward_timed")
        return dq, dk, dv
    if Nk != N:
        if dropout_p is not None or block_mask is not None:
            raise ValueError("dropout and block masks need Nk = Nq")
        st = load().fa_backward_kv(*args[:12], Nk, *args[12:], workspace.data_ptr(),
                                   workspace.numel(), _stream(q))
        where = "fa_backward_kv"
    elif block_mask is not None:
        heads = _check_mask(block_mask, q)
        st = load().fa_backward_blocksparse(*args, block_mask.data_ptr(), heads,
                                            workspace.data_ptr(), workspace.numel(), _stream(q))
        where = "fa_backward_blocksparse"
    elif dropout_p is None:
        st = load().fa_backward(*args, workspace.data_ptr(), workspace.numel(), _stream(q))
        where = "fa_backward"
    else:
        st = load().fa_backward_dropout(*args, float(dropout_p), int(seed), int(offset),
                                        workspace.data_ptr(), workspace.numel(), _stream(q))
        where = "fa_backward_dropout"
    if st != FA_OK:
        raise FAError(st, where)
    return dq, dk, dv


def decode_workspace_bytes(B, H, Nq, Nk, d):
    return int(load().fa_decode_workspace_bytes(B, H, Nq, Nk, d))


def decode(q, k, v, scale=None, causal=False, o_dtype=None, out=None, lse=None, workspace=None,
           no_alloc=False):
    """fa_decode_forward: q [B, H, Nq, d] (Nq <= 4) against k, v [B, H, Nk, d]. Returns (O, LSE).

    The queries are the last Nq positions of the sequence (causal: query i sees keys
    0 .. Nk - Nq + i). `workspace` (a uint8 GPU tensor) is allocated when not given. With
    no_alloc=True the call is fa_decode_forward_noalloc, whose partials live in the library's own
    device scratch (no workspace; give `out` and `lse` to make the whole call allocation-free).
    """
    torch = _torch()
    _check_bhnd("q", q)
    _check_bhnd("k", k)
    _check_bhnd("v", v, k.shape)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape[:2]) != (B, H) or k.shape[3] != d:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [{B}, {H}, Nk, {d}]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o_dtype = q.dtype if o_dtype is None else o_dtype
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=o_dtype, device=q.device)
    else:
        _check_bhnd("out", out, q.shape)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if no_alloc:
        st = load().fa_decode_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                              out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                                              scale, int(bool(causal)), dtype_code(q.dtype),
                                              dtype_code(out.dtype), _stream(q))
        if st != FA_OK:
            raise FAError(st, "fa_decode_forward_noalloc")
        return out, lse
    need = decode_workspace_bytes(B, H, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = load().fa_decode_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr(), B, H, Nq, Nk, d, scale, int(bool(causal)),
                                  dtype_code(q.dtype), dtype_code(out.dtype),
                                  workspace.data_ptr(), workspace.numel(), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_decode_forward")
    return out, lse
