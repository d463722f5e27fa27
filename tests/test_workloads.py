"""Seeded input generators: bf16 rounding, recipe shapes, determinism (no GPU)."""
import numpy as np
import pytest
import torch

from flashattention_forward_fa_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    """Round-to-nearest-even of the generator equals torch's float32 -> bfloat16 cast."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-40, -3.3e38, np.inf, -np.inf],
                                 dtype=np.float32)])
    ours = wl.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(wl.bf16_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_small_config_is_deterministic():
    a, b = wl.config(1), wl.config(1)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    assert a.q.shape == (1, 256, 2, 64) and a.o_dtype == "f32" and a.scale == 0.125
    assert a.flops() == 4 * 2 * 256 * 256 * 64


def test_outlier_recipe():
    w = wl.make_fixed(1, 3, 16, 400, 8, seed=3, causal=True, outlier_frac=0.01)
    ref = wl.make_fixed(1, 3, 16, 400, 8, seed=3, causal=True)
    kk = wl.bf16_to_f32(w.k)
    k0 = wl.bf16_to_f32(ref.k)
    # outliers are drawn after V, so Q, V and the untouched K rows coincide
    assert np.array_equal(w.q, ref.q) and np.array_equal(w.v, ref.v)
    for h in range(3):
        changed = np.where(np.any(kk[0, :, h] != k0[0, :, h], axis=1))[0]
        assert len(changed) == 4
        np.testing.assert_array_equal(kk[0, changed, h], 8 * k0[0, changed, h])


def test_varlen_recipe():
    w = wl.make_varlen(4, 64, seed=9, nseq=5, len_lo=3, len_hi=40)
    assert w.offsets[0] == 0 and w.offsets[-1] == w.q.shape[0]
    assert np.all(np.diff(w.offsets) == w.lengths)
    assert np.all((w.lengths >= 3) & (w.lengths <= 40))
    assert w.Nq == int(w.lengths.max())


@pytest.mark.parametrize("n", [3, 5])
def test_named_config_shapes(n):
    w = wl.config(n)
    if n == 3:
        assert w.q.shape == (2, 4096, 32, 128) and w.causal
        assert w.flops() == 4 * 2 * 32 * 4096 * 4096 * 128 / 2
    else:
        assert w.varlen and w.H == 32 and w.d == 64 and len(w.lengths) == 16
        assert w.q.shape == (int(w.offsets[-1]), 32, 64)
