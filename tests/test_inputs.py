"""The seeded input generator: rounding to storage dtypes and reproducibility."""

import numpy as np
import pytest

from exact_attention_94_amd.inputs import (WORKLOADS, bf16_bits_to_f32, draw, f32_to_bf16_bits,
                                           quantize, subset_rows)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * 7
    x = np.concatenate([x, np.float32([1.00390625, 1.005859375, 3.0e38, -2.5e-39, 0.0])])
    mine = bf16_bits_to_f32(f32_to_bf16_bits(x))
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(mine, ref)


def test_quantize_exact_values():
    x = np.random.default_rng(1).standard_normal(1000, dtype=np.float32)
    for dt in ("f32", "f16", "bf16"):
        t = quantize(x, dt)
        assert t.values.dtype == np.float32
        if dt == "f16":
            assert np.array_equal(t.bits.view(np.float16).astype(np.float32), t.values)
        if dt == "bf16":
            assert np.array_equal(bf16_bits_to_f32(t.bits), t.values)


def test_draw_is_seeded_and_ordered():
    a = draw((1, 2, 8, 4), "bf16", 5, with_do=True)
    b = draw((1, 2, 8, 4), "bf16", 5, with_do=True)
    for k in ("q", "k", "v", "do"):
        assert np.array_equal(a[k].bits, b[k].bits)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, 8, 4), dtype=np.float32)
    assert np.array_equal(a["q"].values, quantize(q, "bf16").values)


def test_qk_multiplier_is_exact():
    a = draw((1, 1, 16, 8), "bf16", 3, qk_mult=2.0)
    b = draw((1, 1, 16, 8), "bf16", 3)
    assert np.array_equal(a["q"].values, 2 * b["q"].values)
    assert np.array_equal(a["v"].values, b["v"].values)


def test_subset_rows():
    r = subset_rows(32768, 3)
    assert len(r) == 64 and len(set(r)) == 64 and r == sorted(r)
    assert {0, 1, 63, 64, 32766, 32767} <= set(r)
    assert subset_rows(32768, 3) == r and subset_rows(32768, 4) != r
    assert WORKLOADS["b2h16n4k_d64"].scale == 0.125
