"""The seeded workload generators: determinism, exact input rounding, and the stated
shapes and distributions. CPU only."""
import numpy as np
import pytest

import synth


def test_bf16_round_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0], np.float32)
    y = synth.bf16_round(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert y.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0]
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    b = synth.bf16_round(r)
    assert np.all(b.view(np.uint32) & 0xFFFF == 0)
    assert np.max(np.abs(b - r) / np.abs(r)) <= 2 ** -8


def test_generators_are_deterministic():
    a = synth.preset("kda_prefill", B=1, T=70, H=2)
    b = synth.preset("kda_prefill", B=1, T=70, H=2)
    for f in ("q", "k", "v", "alpha", "erase", "S0"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


@pytest.mark.parametrize("name", ["kda_tiny", "kda_prefill", "ckda_long"])
def test_prefill_shapes_and_ranges(name):
    over = {} if name == "kda_tiny" else dict(B=1, T=300, H=3)
    w = synth.preset(name, **over)
    B, T, H, dk = w.q.shape
    assert w.k.shape == w.q.shape and w.alpha.shape == w.q.shape
    assert w.erase.shape == (B, T, H) and w.write is None
    if w.in_dtype == "bf16":
        assert np.all(w.q.view(np.uint32) & 0xFFFF == 0)
    # q and k were unit vectors before rounding
    assert np.allclose(np.linalg.norm(w.k.astype(np.float64), axis=-1), 1, atol=2 ** -7)
    if name == "ckda_long":
        assert w.alpha.min() >= -1 and w.alpha.max() <= 1 and (w.alpha < 0).mean() > 0.3
        assert 0.07 < np.mean(np.abs(w.alpha) == 1) < 0.13
        assert w.erase.min() >= 0 and w.erase.max() <= 2 and 0.03 < np.mean(w.erase == 2) < 0.08
    elif name == "kda_prefill":
        assert w.alpha.min() > 0.5 and w.alpha.max() < 1 and np.median(w.alpha) > 0.9
    else:
        assert w.alpha.min() > 0 and w.alpha.max() < 1 and w.S0 is None


def test_varlen_lengths():
    w = synth.preset("rda_varlen")
    lens = np.diff(w.cu_seqlens)
    assert len(lens) == 12 and lens.sum() == 32768 and lens.min() >= 256 and lens.max() <= 6000
    g = synth.preset("gdn2_varlen")
    assert np.array_equal(g.cu_seqlens, w.cu_seqlens)
    assert np.array_equal(g.q, w.q) and np.array_equal(g.alpha, w.alpha)
    assert g.erase.shape == g.q.shape and g.write.shape == g.v.shape
    assert w.erase.shape == w.q.shape[:-1] and w.write.shape == w.q.shape[:-1]


def test_decode_preset_shapes():
    w = synth.make_decode("gdn2", 4, 3, 16, 32, steps=2, seed=5)
    assert w.q.shape == (2, 4, 3, 16) and w.v.shape == (2, 4, 3, 32)
    assert w.erase.shape == (2, 4, 3, 16) and w.write.shape == (2, 4, 3, 32)
    assert w.S0.shape == (4, 3, 16, 32)
