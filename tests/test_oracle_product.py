"""Pins for the two-transitions-per-token oracle (oracle.product): explicit transition
matrices, the rotation closed form, orthogonality, reduction to KDA, the interleaved
single-transition sequence, packing, decode, and the gradients against central finite
differences. CPU only."""
import numpy as np
import pytest

import oracle
from oracle import product

RNG = np.random.default_rng(20261207)


def _inputs(rng, B, T, H, dk, dv, signed=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, 2, dk))
    v = rng.standard_normal((B, T, H, 2, dv))
    alpha = rng.uniform(-1.0, 1.0, (B, T, H, dk)) if signed else rng.uniform(0.5, 1.0, (B, T, H, dk))
    beta = rng.uniform(0.0, 2.0, (B, T, H, 2))
    return q, k, v, alpha, beta


def test_matches_the_explicit_product_of_transition_matrices():
    B, T, H, dk, dv = 2, 5, 2, 3, 2
    q, k, v, alpha, beta = _inputs(RNG, B, T, H, dk, dv)
    S0 = RNG.standard_normal((B, H, dk, dv))
    o, S_T = product.product_recurrence(q, k, v, alpha, beta, S0=S0)
    I = np.eye(dk)
    for b in range(B):
        for h in range(H):
            S = S0[b, h].copy()
            for t in range(T):
                k1, k2 = k[b, t, h, 0], k[b, t, h, 1]
                b1, b2 = beta[b, t, h]
                H1 = I - b1 * np.outer(k1, k1)
                H2 = I - b2 * np.outer(k2, k2)
                S = H2 @ H1 @ np.diag(alpha[b, t, h]) @ S + H2 @ (b1 * np.outer(k1, v[b, t, h, 0])) \
                    + b2 * np.outer(k2, v[b, t, h, 1])
                np.testing.assert_allclose(o[b, t, h], S.T @ q[b, t, h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(S_T[b, h], S, rtol=1e-12, atol=1e-12)


def test_zero_second_beta_is_kda():
    B, T, H, dk, dv = 2, 9, 2, 4, 3
    q, k, v, alpha, beta = _inputs(RNG, B, T, H, dk, dv)
    beta[..., 1] = 0.0
    S0 = RNG.standard_normal((B, H, dk, dv))
    o, S_T = product.product_recurrence(q, k, v, alpha, beta, S0=S0)
    o_ref, S_ref = oracle.step_recurrence(q, k[..., 0, :], v[..., 0, :], alpha, beta[..., 0], None, "kda", S0=S0)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(S_T, S_ref)


@pytest.mark.parametrize("theta", [0.3, 1.1, -0.7])
def test_two_reflections_rotate_by_twice_the_key_angle(theta):
    # alpha = 1, beta = 2 twice, unit keys e0 and (cos theta, sin theta, 0), no write:
    # each token rotates key rows 0 and 1 by 2 theta and leaves row 2 alone
    T = 5
    k = np.zeros((1, T, 1, 2, 3))
    k[..., 0, 0] = 1.0
    k[..., 1, 0], k[..., 1, 1] = np.cos(theta), np.sin(theta)
    v = np.zeros((1, T, 1, 2, 2))
    alpha = np.ones((1, T, 1, 3))
    beta = np.full((1, T, 1, 2), 2.0)
    q = RNG.standard_normal((1, T, 1, 3))
    S0 = RNG.standard_normal((1, 1, 3, 2))
    _, S_T = product.product_recurrence(q, k, v, alpha, beta, S0=S0)
    c, s = np.cos(2 * theta), np.sin(2 * theta)
    R = np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])
    np.testing.assert_allclose(S_T[0, 0], np.linalg.matrix_power(R, T) @ S0[0, 0], rtol=0, atol=1e-12)


def test_orthogonal_factors_preserve_the_state_norm():
    B, T, H, dk, dv = 2, 30, 2, 6, 4
    q, k, v, alpha, beta = _inputs(RNG, B, T, H, dk, dv)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    alpha = np.where(RNG.random(alpha.shape) < 0.5, -1.0, 1.0)
    beta = np.where(RNG.random(beta.shape) < 0.5, 0.0, 2.0)
    v[:] = 0.0
    S0 = RNG.standard_normal((B, H, dk, dv))
    _, S_T = product.product_recurrence(q, k, v, alpha, beta, S0=S0)
    np.testing.assert_allclose(np.linalg.norm(S_T, axis=(-2, -1)), np.linalg.norm(S0, axis=(-2, -1)), rtol=1e-12)


def test_equals_kda_on_the_interleaved_transitions():
    # 2T single KDA transitions, the decay on the first of each pair, outputs read after
    # the second
    B, T, H, dk, dv = 1, 11, 2, 4, 3
    q, k, v, alpha, beta = _inputs(RNG, B, T, H, dk, dv)
    S0 = RNG.standard_normal((B, H, dk, dv))
    o, S_T = product.product_recurrence(q, k, v, alpha, beta, S0=S0)
    q2 = np.repeat(q, 2, axis=1)
    k2 = k.transpose(0, 1, 3, 2, 4).reshape(B, 2 * T, H, dk)
    v2 = v.transpose(0, 1, 3, 2, 4).reshape(B, 2 * T, H, dv)
    b2 = beta.transpose(0, 1, 3, 2).reshape(B, 2 * T, H)
    a2 = np.ones((B, 2 * T, H, dk))
    a2[:, 0::2] = alpha
    o2, S2 = oracle.step_recurrence(q2, k2, v2, a2, b2, None, "kda", S0=S0)
    np.testing.assert_allclose(o, o2[:, 1::2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_T, S2, rtol=1e-12, atol=1e-12)


def test_packed_sequences_equal_each_sequence_alone():
    lens = [4, 0, 7, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, alpha, beta = _inputs(RNG, 1, int(cu[-1]), 2, 3, 2)
    S0 = RNG.standard_normal((len(lens), 2, 3, 2))
    o, S_T = product.product_recurrence(q, k, v, alpha, beta, S0=S0, cu_seqlens=cu)
    for n in range(len(lens)):
        sl = (slice(None), slice(int(cu[n]), int(cu[n + 1])))
        o_n, S_n = product.product_recurrence(q[sl], k[sl], v[sl], alpha[sl], beta[sl], S0=S0[n:n + 1])
        np.testing.assert_array_equal(o[sl], o_n)
        np.testing.assert_array_equal(S_T[n], S_n[0])


def test_decode_steps_equal_the_recurrence():
    N, T, H, dk, dv = 3, 6, 2, 4, 5
    q, k, v, alpha, beta = _inputs(RNG, N, T, H, dk, dv)
    S0 = RNG.standard_normal((N, H, dk, dv))
    o, S_T = product.product_recurrence(q, k, v, alpha, beta, S0=S0)
    S = S0.copy()
    for t in range(T):
        S, o_t = product.product_decode_step(S, q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t])
        np.testing.assert_array_equal(o_t, o[:, t])
    np.testing.assert_array_equal(S, S_T)


@pytest.mark.parametrize("packed", [False, True])
def test_gradients_match_finite_differences(packed):
    rng = np.random.default_rng(11 + packed)
    if packed:
        cu = np.array([0, 3, 3, 7])
        B, T, N = 1, 7, 3
    else:
        cu, B, T, N = None, 2, 4, 2
    H, dk, dv = 2, 3, 2
    q, k, v, alpha, beta = _inputs(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((N, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dS = rng.standard_normal((N, H, dk, dv))
    g = product.product_grads(q, k, v, alpha, beta, do, dS_T=dS, S0=S0, cu_seqlens=cu)

    def loss(q_, k_, v_, a_, b_, s_):
        o, S_T = product.product_recurrence(q_, k_, v_, a_, b_, S0=s_, cu_seqlens=cu)
        return float(np.sum(o * do) + np.sum(S_T * dS))

    args = [q, k, v, alpha, beta, S0]
    names = ["dq", "dk", "dv", "dalpha", "dbeta", "dS0"]
    eps = 1e-6
    for ai, name in enumerate(names):
        x = args[ai]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = [a.copy() for a in args]
            xm = [a.copy() for a in args]
            xp[ai][idx] += eps
            xm[ai][idx] -= eps
            fd[idx] = (loss(*xp) - loss(*xm)) / (2 * eps)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-7, err_msg=name)
