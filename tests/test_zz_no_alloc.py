"""fa_decode_forward_noalloc (split-KV decoding with the library's own device scratch instead of a
caller workspace) against fa_decode_forward on the same inputs: two calls in a row, the second
smaller than the first, each bit-identical to the workspace entry point (same kernels, same
partials layout, and the scratch is fully rewritten before it is read)."""

import numpy as np
import pytest

from exact_attention_94_amd import inputs as inp
from tests.gpu_util import nan_like, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_94_amd as fa_mod
    fa_mod.binding.load()
    return fa_mod


def _case(fa, B, H, nq, nk, d, dtype, causal, o_f32, seed):
    import torch
    print(f"  B={B} H={H} Nq={nq} Nk={nk} d={d} {dtype} causal={causal} o_f32={o_f32}",
          flush=True)
    tq = inp.draw((B, H, nq, d), dtype, seed)
    tk = inp.draw((B, H, nk, d), dtype, seed + 1)
    q = to_device(tq["q"])
    k, v = to_device(tk["k"]), to_device(tk["v"])
    od = torch.float32 if o_f32 else q.dtype
    need = fa.decode_workspace_bytes(B, H, nq, nk, d)
    assert 0 < need <= fa.binding.DECODE_SCRATCH_BYTES
    o_ref, l_ref = nan_like((B, H, nq, d), od), nan_like((B, H, nq), torch.float32)
    fa.decode(q, k, v, causal=causal, out=o_ref, lse=l_ref)
    o_na, l_na = nan_like((B, H, nq, d), od), nan_like((B, H, nq), torch.float32)
    fa.decode(q, k, v, causal=causal, out=o_na, lse=l_na, no_alloc=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o_na).all()) and bool(torch.isfinite(l_na).all())
    assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)


def test_noalloc_decode_matches_workspace_entry_point(fa):
    # The first call fills most of the scratch (about 4 MiB of partials); the second, smaller
    # one reuses the same array with another chunking and must not see the first one's data.
    _case(fa, 4, 32, 4, 16384, 128, "bf16", True, False, 11)
    _case(fa, 2, 8, 3, 3000, 64, "f16", True, True, 12)
    _case(fa, 1, 2, 1, 77, 128, "bf16", False, True, 13)


def test_noalloc_decode_rejects_oversized_calls(fa):
    """More partials than the scratch holds: FA_ERR_WORKSPACE before any launch."""
    import torch
    B, H, nq, nk, d = 64, 128, 4, 256, 128
    assert fa.decode_workspace_bytes(B, H, nq, nk, d) > fa.binding.DECODE_SCRATCH_BYTES
    q = torch.zeros((B, H, nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, nk, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as exc:
        fa.decode(q, k, k, causal=True, out=torch.empty_like(q),
                  lse=torch.empty((B, H, nq), dtype=torch.float32, device="cuda"), no_alloc=True)
    assert exc.value.status == fa.FA_ERR_WORKSPACE
