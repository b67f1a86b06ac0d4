"""Pins for the oracle's input preparation (L2 normalisation, gate activations): hand
values, limits, symmetries and invariances. CPU only."""
import numpy as np
import pytest

import oracle
from oracle import prep

RNG = np.random.default_rng(20261205)


def test_l2_normalize_hand_example_and_zero():
    np.testing.assert_allclose(prep.l2_normalize(np.array([3.0, 4.0])), [0.6, 0.8], rtol=0, atol=1e-15)
    assert not prep.l2_normalize(np.zeros((2, 5))).any()


def test_l2_normalize_gives_unit_rows_and_ignores_positive_scale():
    x = RNG.standard_normal((7, 3, 16))
    y = prep.l2_normalize(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=0, atol=1e-14)
    c = RNG.uniform(0.01, 100, (7, 3, 1))
    np.testing.assert_allclose(prep.l2_normalize(c * x), y, rtol=0, atol=1e-14)


def test_softplus_values():
    assert prep.softplus(0.0) == pytest.approx(np.log(2.0), abs=1e-16)
    assert prep.softplus(800.0) == 800.0                    # no overflow
    assert prep.softplus(-50.0) == pytest.approx(np.exp(-50.0), rel=1e-12)
    assert prep.softplus(-np.inf) == 0.0


def test_sigmoid_values_and_symmetry():
    assert prep.sigmoid(0.0) == 0.5
    assert prep.sigmoid(np.inf) == 1.0 and prep.sigmoid(-np.inf) == 0.0
    z = RNG.standard_normal(1000) * 30
    np.testing.assert_allclose(prep.sigmoid(z) + prep.sigmoid(-z), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(prep.sigmoid(1.0), 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-15)


@pytest.mark.parametrize("scale", [1.0, 0.1])
def test_exp_neg_softplus_decay(scale):
    assert prep.alpha_from(0.0, "exp_neg_softplus", scale) == pytest.approx(2.0 ** -scale, rel=1e-15)
    assert prep.alpha_from(-np.inf, "exp_neg_softplus", scale) == 1.0
    z = RNG.standard_normal(500) * 4
    a = prep.alpha_from(z, "exp_neg_softplus", scale)
    assert np.all((a > 0) & (a <= 1))
    # exp(-softplus(z)) = 1 - sigmoid(z) = sigmoid(-z) for scale 1
    if scale == 1.0:
        np.testing.assert_allclose(a, prep.sigmoid(-z), rtol=1e-13)


def test_tanh_decay_limits_and_oddness():
    assert prep.alpha_from(np.inf, "tanh") == 1.0 and prep.alpha_from(-np.inf, "tanh") == -1.0
    z = RNG.standard_normal(300) * 2
    np.testing.assert_allclose(prep.alpha_from(-z, "tanh"), -prep.alpha_from(z, "tanh"), rtol=0, atol=0)


@pytest.mark.parametrize("x,exact", [(2.0, 3 / 5), (3.0, 4 / 5), (5.0, 12 / 13), (9.0, 40 / 41),
                                     (1.5, 5 / 13)])
def test_tanh_decay_hand_values(x, exact):
    # tanh z = (e^{2z} - 1) / (e^{2z} + 1); at z = ln x that is (x^2 - 1) / (x^2 + 1):
    # tanh(ln 2) = 3/5, tanh(ln 3) = 4/5, tanh(ln 5) = 12/13, tanh(ln 9) = 40/41, tanh(ln 1.5) = 5/13
    assert exact == pytest.approx((x * x - 1) / (x * x + 1), abs=1e-15)
    assert prep.alpha_from(np.log(x), "tanh") == pytest.approx(exact, abs=2e-16)
    assert prep.alpha_from(-np.log(x), "tanh") == pytest.approx(-exact, abs=2e-16)


def test_tanh_decay_small_and_moderate_arguments():
    # tanh z = z - z^3/3 + 2 z^5/15 - 17 z^7/315 + ... near zero, and 1 - tanh z =
    # 2 e^{-2z} / (1 + e^{-2z}) exactly; a slightly rescaled argument (tanh(1.0001 z)) or a
    # softsign fails both
    z = np.array([1e-3, 1e-2, 3e-2])
    series = z - z ** 3 / 3 + 2 * z ** 5 / 15 - 17 * z ** 7 / 315
    np.testing.assert_allclose(prep.alpha_from(z, "tanh"), series, rtol=1e-13, atol=0)
    z = np.array([0.5, 1.0, 2.0, 3.0])
    e = np.exp(-2 * z)
    np.testing.assert_allclose(1.0 - prep.alpha_from(z, "tanh"), 2 * e / (1 + e), rtol=1e-12, atol=0)


def test_gate_scale_two_spans_zero_to_two():
    z = np.array([-np.inf, 0.0, np.inf])
    np.testing.assert_array_equal(prep.gate_from(z, "sigmoid", 2.0), [0.0, 1.0, 2.0])


@pytest.mark.parametrize("x,scale", [(3.0, 1.0), (7.0, 1.0), (1.5, 2.0), (99.0, 0.5)])
def test_sigmoid_gate_hand_values(x, scale):
    # sigmoid z = 1 / (1 + e^{-z}); at z = ln x that is x / (x + 1), at z = -ln x 1 / (x + 1):
    # sigmoid(ln 3) = 3/4, sigmoid(ln 7) = 7/8, sigmoid(ln 1.5) = 3/5, sigmoid(ln 99) = 99/100.
    # A rescaled argument (sigmoid(1.01 z)) keeps the values at 0 and +-inf and the symmetry, and
    # fails here.
    assert prep.sigmoid(np.log(x)) == pytest.approx(x / (x + 1), abs=2e-16)
    assert prep.gate_from(np.log(x), "sigmoid", scale) == pytest.approx(scale * x / (x + 1), abs=4e-16)
    assert prep.gate_from(-np.log(x), "sigmoid", scale) == pytest.approx(scale / (x + 1), abs=4e-16)


def test_prepare_with_everything_off_is_the_identity():
    q, k, a, e, w = (RNG.standard_normal((2, 3, 4)) for _ in range(5))
    out = prep.prepare(q, k, a, e, w, l2norm_qk=False, alpha_act="none", alpha_scale=1.0,
                       gate_act="none", gate_scale=1.0)
    for x, y in zip(out, (q, k, a, e, w)):
        np.testing.assert_array_equal(x, y)


def test_recurrence_on_prepared_inputs_ignores_qk_scale():
    B, T, H, dk, dv = 1, 12, 2, 8, 4
    q = RNG.standard_normal((B, T, H, dk))
    k = RNG.standard_normal((B, T, H, dk))
    v = RNG.standard_normal((B, T, H, dv))
    za = RNG.standard_normal((B, T, H, dk))
    zb = RNG.standard_normal((B, T, H))
    kw = dict(l2norm_qk=True, alpha_act="exp_neg_softplus", alpha_scale=1.0, gate_act="sigmoid", gate_scale=1.0)
    p1 = prep.prepare(q, k, za, zb, None, **kw)
    p2 = prep.prepare(q * 3.5, k * 0.02, za, zb, None, **kw)
    o1, S1 = oracle.step_recurrence(p1[0], p1[1], v, p1[2], p1[3], None, "kda")
    o2, S2 = oracle.step_recurrence(p2[0], p2[1], v, p2[2], p2[3], None, "kda")
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S2, S1, rtol=0, atol=1e-13)
