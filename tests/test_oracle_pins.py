"""Pins for the fp64 oracle: each test fixes the oracle to something other than its
own code — a worked example done by hand from the page's formula, a closed form,
an invariant the pages state, or a textbook special case. CPU only."""
import glob
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20261203)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_inputs(rng, B, T, H, dk, dv, variant, signed=False, zeros=False):
    q = rng.standard_normal((B, T, H, dk))
    k = _unit(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    if signed:
        alpha = rng.uniform(-1, 1, (B, T, H, dk))
        alpha[rng.random(alpha.shape) < 0.1] = 1.0
        alpha[rng.random(alpha.shape) < 0.1] = -1.0
    else:
        alpha = rng.uniform(0.6, 1.0, (B, T, H, dk))
    if zeros:
        alpha[rng.random(alpha.shape) < 0.05] = 0.0
    if variant == "gdn2":
        erase = rng.uniform(0, 1, (B, T, H, dk))
        write = rng.uniform(0, 1, (B, T, H, dv))
    elif variant == "rda":
        erase = rng.uniform(0, 1, (B, T, H))
        write = rng.uniform(0, 1, (B, T, H))
    else:
        erase = rng.uniform(0, 2 if variant == "ckda" else 1, (B, T, H))
        write = None
    S0 = rng.standard_normal((B, H, dk, dv)) / np.sqrt(dk)
    return q, k, v, alpha, erase, write, S0


# --------------------------------------------------------------------------- worked examples

@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.json"))),
                         ids=lambda p: os.path.basename(p))
def test_hand_worked_examples(path):
    """Hand-computed fixtures (tests/golden): each cites the formula it follows."""
    fx = json.load(open(path))
    toks = fx["tokens"]
    arr = lambda key: np.array([[tk[key]] for tk in toks], dtype=np.float64)[None]  # [1,T,1,..]
    q, k, v, alpha = arr("q"), arr("k"), arr("v"), arr("alpha")
    erase = np.array([[tk["erase"]] for tk in toks], dtype=np.float64)[None]
    write = None
    if "write" in toks[0]:
        write = np.array([[tk["write"]] for tk in toks], dtype=np.float64)[None]
    S0 = np.array(fx["S0"], dtype=np.float64)[None, None]
    o, S_T = oracle.step_recurrence(q, k, v, alpha, erase, write, fx["variant"], S0=S0)
    exp_o = np.array(fx["expected"]["o"], dtype=np.float64)
    exp_S = np.array(fx["expected"]["S_T"], dtype=np.float64)
    tol = fx["tol"]
    np.testing.assert_allclose(o[0, :, 0], exp_o, rtol=0, atol=tol)
    np.testing.assert_allclose(S_T[0, 0], exp_S, rtol=0, atol=tol)
    o_c, S_c = oracle.chunked_reference(q, k, v, alpha, erase, write, fx["variant"], S0=S0, chunk=2)
    np.testing.assert_allclose(o_c[0, :, 0], exp_o, rtol=0, atol=max(tol, 1e-14))
    np.testing.assert_allclose(S_c[0, 0], exp_S, rtol=0, atol=max(tol, 1e-14))


# --------------------------------------------------------------------------- variant relations

def test_rda_with_equal_gates_is_kda_bitwise():
    """RDA reduces to KDA when e_t = w_t (Raon-1-mini-preview discussion #1)."""
    q, k, v, alpha, beta, _, S0 = _rand_inputs(RNG, 2, 23, 3, 8, 6, "kda")
    o1, s1 = oracle.step_recurrence(q, k, v, alpha, beta, None, "kda", S0=S0)
    o2, s2 = oracle.step_recurrence(q, k, v, alpha, beta, beta.copy(), "rda", S0=S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_ckda_is_kda_formula():
    """CKDA keeps KDA's formula and only widens the ranges (Complex KDA abstract)."""
    q, k, v, alpha, beta, _, S0 = _rand_inputs(RNG, 1, 17, 2, 8, 8, "ckda", signed=True)
    o1, s1 = oracle.step_recurrence(q, k, v, alpha, beta, None, "kda", S0=S0)
    o2, s2 = oracle.step_recurrence(q, k, v, alpha, beta, None, "ckda", S0=S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_gdn2_with_uniform_gates_is_rda():
    """GDN-2 with b_t = e_t 1 and w_t = w_t 1 is RDA: the two rules differ only in gate
    granularity (discussion #1)."""
    q, k, v, alpha, e, w, S0 = _rand_inputs(RNG, 2, 19, 3, 8, 5, "rda")
    o1, s1 = oracle.step_recurrence(q, k, v, alpha, e, w, "rda", S0=S0)
    b = e[..., None] * np.ones(8)
    wv = w[..., None] * np.ones(5)
    o2, s2 = oracle.step_recurrence(q, k, v, alpha, b, wv, "gdn2", S0=S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_gdn2_erase_acts_through_b_dot_k_on_the_right():
    """GDN-2 erase is (I - k (b . k)^T): the change to the decayed state lies along k
    (left factor), and only (b . k)^T X decides how much is erased (right factor)."""
    rng = np.random.default_rng(7)
    dk, dv = 3, 2
    S = rng.standard_normal((dk, dv))
    S[0] = 0.0                                  # (b . k)^T S = k_0 b_0 S[0] = 0 below
    k = rng.standard_normal(dk)
    b = np.array([0.7, 0.0, 0.0])
    wg = rng.uniform(0, 1, dv)
    v = rng.standard_normal(dv)
    S1, _ = oracle.step(S, np.zeros(dk), k, v, np.ones(dk), b, wg, "gdn2")
    np.testing.assert_allclose(S1, S + np.outer(k, wg * v), rtol=0, atol=1e-15)
    # random case: S1 - X is rank one with column space span(k)
    S = rng.standard_normal((dk, dv))
    b = rng.uniform(0, 1, dk)
    alpha = rng.uniform(-1, 1, dk)
    S1, _ = oracle.step(S, np.zeros(dk), k, v, alpha, b, wg, "gdn2")
    D = S1 - alpha[:, None] * S
    proj = np.outer(k, k @ D) / (k @ k)
    np.testing.assert_allclose(D, proj, rtol=0, atol=1e-13)
    np.testing.assert_allclose(k @ D / (k @ k), wg * v - (b * k) @ (alpha[:, None] * S), atol=1e-13)


# --------------------------------------------------------------------------- transition properties

def test_transitions_are_non_expansive():
    """With unit k, |alpha| <= 1 and beta in [0, 2], (I - beta k k^T) Diag(alpha) has
    spectral norm <= 1 (Complex KDA abstract: non-expansive DPLR transitions)."""
    rng = np.random.default_rng(11)
    worst = 0.0
    for _ in range(2000):
        d = int(rng.integers(2, 9))
        k = _unit(rng.standard_normal(d))
        alpha = rng.uniform(-1, 1, d)
        beta = rng.uniform(0, 2)
        M = oracle.transition_matrix(alpha, k, beta * k)
        worst = max(worst, np.linalg.norm(M, 2))
    assert worst <= 1.0 + 1e-12


def test_gdn2_transition_is_not_claimed_non_expansive():
    """The non-expansive statement is made for CKDA; GDN-2's asymmetric erase can expand."""
    k = _unit(np.array([1.0, 1.0]))
    M = oracle.transition_matrix(np.ones(2), k, np.array([1.0, 0.0]) * k)
    assert np.linalg.norm(M, 2) > 1.1


def test_unit_gates_and_beta_0_or_2_are_orthogonal():
    """|alpha| = 1 and beta in {0, 2}: the transition is orthogonal, so with the write
    switched off ||S||_F is preserved (Complex KDA abstract: orthogonal DPLR)."""
    rng = np.random.default_rng(12)
    for beta in (0.0, 2.0):
        for _ in range(50):
            d = int(rng.integers(2, 9))
            k = _unit(rng.standard_normal(d))
            alpha = np.where(rng.random(d) < 0.5, -1.0, 1.0)
            M = oracle.transition_matrix(alpha, k, beta * k)
            np.testing.assert_allclose(M @ M.T, np.eye(d), atol=1e-13)
    B, T, H, dk, dv = 1, 50, 2, 6, 4
    q = rng.standard_normal((B, T, H, dk))
    k = _unit(rng.standard_normal((B, T, H, dk)))
    alpha = np.where(rng.random((B, T, H, dk)) < 0.5, -1.0, 1.0)
    beta = np.where(rng.random((B, T, H)) < 0.5, 0.0, 2.0)
    S0 = rng.standard_normal((B, H, dk, dv))
    _, S_T = oracle.step_recurrence(q, k, np.zeros((B, T, H, dv)), alpha, beta, None, "ckda", S0=S0)
    np.testing.assert_allclose(np.linalg.norm(S_T, axis=(-2, -1)),
                               np.linalg.norm(S0, axis=(-2, -1)), rtol=1e-12)


@pytest.mark.parametrize("theta", [0.3, 1.0, np.pi / 2, 2.5, -0.7])
def test_rotation_from_reflection_and_sign_flip(theta):
    """A reflection (beta = 2) composed with the gate's sign flip alpha = (1, -1) is the
    rotation by theta when k = (cos p, sin p), p = (theta - pi)/2 (Complex KDA abstract)."""
    p = (theta - np.pi) / 2
    k = np.array([np.cos(p), np.sin(p)])
    R = np.array([[np.cos(theta), -np.sin(theta)], [np.sin(theta), np.cos(theta)]])
    M = oracle.transition_matrix(np.array([1.0, -1.0]), k, 2.0 * k)
    np.testing.assert_allclose(M, R, atol=1e-15)
    # T steps inside a d_k = 4 state whose extra key channels have k = 0 and alpha = 1
    T, dv = 9, 3
    rng = np.random.default_rng(13)
    S0 = rng.standard_normal((1, 1, 4, dv))
    kk = np.zeros((1, T, 1, 4)); kk[..., :2] = k
    al = np.ones((1, T, 1, 4)); al[..., 1] = -1.0
    q = rng.standard_normal((1, T, 1, 4))
    o, S_T = oracle.step_recurrence(q, kk, np.zeros((1, T, 1, dv)), al,
                                    np.full((1, T, 1), 2.0), None, "ckda", S0=S0)
    for t in range(1, T + 1):
        Rt = np.eye(4)
        Rt[:2, :2] = [[np.cos(t * theta), -np.sin(t * theta)], [np.sin(t * theta), np.cos(t * theta)]]
        St = Rt @ S0[0, 0]
        np.testing.assert_allclose(o[0, t - 1, 0], St.T @ q[0, t - 1, 0], atol=1e-12)
    np.testing.assert_allclose(S_T[0, 0], St, atol=1e-12)


# --------------------------------------------------------------------------- closed forms

def test_delta_readback():
    """Erase-then-write: with beta = 1, unit k and q = k the token reads back exactly the
    value it wrote, whatever the decay and the prior state (course page 'GDN, KDA và
    Mamba-2', section 1 and the glossary entry for the delta rule). This fails if the
    erase acts before the decay, if the readout uses the pre-update state, or if a term
    of the update is dropped or has the wrong sign."""
    rng = np.random.default_rng(14)
    B, T, H, dk, dv = 2, 21, 3, 7, 5
    k = _unit(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(-1, 1, (B, T, H, dk))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, _ = oracle.step_recurrence(k, k, v, alpha, np.ones((B, T, H)), None, "kda", S0=S0)
    np.testing.assert_allclose(o, v, atol=1e-12)


def test_no_decay_no_erase_is_linear_attention():
    """alpha = 1, e = 0, w = 1 leaves plain causal linear attention:
    O = Q S0 + tril(Q K^T) V (textbook)."""
    rng = np.random.default_rng(15)
    T, dk, dv = 13, 4, 6
    q, k = rng.standard_normal((T, dk)), rng.standard_normal((T, dk))
    v, S0 = rng.standard_normal((T, dv)), rng.standard_normal((dk, dv))
    o, S_T = oracle.step_recurrence(q[None, :, None], k[None, :, None], v[None, :, None],
                                    np.ones((1, T, 1, dk)), np.zeros((1, T, 1)),
                                    np.ones((1, T, 1)), "rda", S0=S0[None, None])
    np.testing.assert_allclose(o[0, :, 0], q @ S0 + np.tril(q @ k.T) @ v, atol=1e-12)
    np.testing.assert_allclose(S_T[0, 0], S0 + k.T @ v, atol=1e-12)


def test_no_erase_is_gated_linear_attention():
    """e = 0, w = 1 with channel-wise decay unrolls to
    o_t = sum_{s<=t} sum_i q_ti k_si prod_{j=s+1..t} alpha_ji v_s + sum_i q_ti prod_{j<=t} alpha_ji S0[i,:];
    with d_k != d_v this fixes that alpha scales the key rows of S."""
    rng = np.random.default_rng(16)
    T, dk, dv = 7, 3, 5
    q, k = rng.standard_normal((T, dk)), rng.standard_normal((T, dk))
    v, S0 = rng.standard_normal((T, dv)), rng.standard_normal((dk, dv))
    alpha = rng.uniform(-1, 1, (T, dk))
    o, _ = oracle.step_recurrence(q[None, :, None], k[None, :, None], v[None, :, None],
                                  alpha[None, :, None], np.zeros((1, T, 1)), np.ones((1, T, 1)),
                                  "rda", S0=S0[None, None])
    for t in range(T):
        ref = np.zeros(dv)
        for i in range(dk):
            ref += q[t, i] * np.prod(alpha[: t + 1, i]) * S0[i]
            for s in range(t + 1):
                ref += q[t, i] * k[s, i] * np.prod(alpha[s + 1: t + 1, i]) * v[s]
        np.testing.assert_allclose(o[0, t, 0], ref, atol=1e-12)


@pytest.mark.parametrize("variant", oracle.VARIANTS)
def test_full_decay(variant):
    """alpha = 0 wipes the state before the token: S_t = k_t m_t^T and o_t = (q_t . k_t) m_t."""
    rng = np.random.default_rng(17)
    q, k, v, alpha, erase, write, S0 = _rand_inputs(rng, 1, 5, 2, 4, 3, variant)
    o, S_T = oracle.step_recurrence(q, k, v, np.zeros_like(alpha), erase, write, variant, S0=S0)
    if variant in ("kda", "ckda"):
        m = erase[..., None] * v
    elif variant == "rda":
        m = write[..., None] * v
    else:
        m = write * v
    np.testing.assert_allclose(o, np.sum(q * k, -1)[..., None] * m, atol=1e-13)
    np.testing.assert_allclose(S_T[0], np.einsum("hi,hj->hij", k[0, -1], m[0, -1]), atol=1e-13)


@pytest.mark.parametrize("variant", oracle.VARIANTS)
def test_linear_in_state_and_values(variant):
    """For fixed q, k, alpha and gates, (o, S_T) is linear in (S0, v) jointly."""
    rng = np.random.default_rng(18)
    q, k, v1, alpha, erase, write, S1 = _rand_inputs(rng, 1, 11, 2, 5, 4, variant, signed=True)
    v2, S2 = rng.standard_normal(v1.shape), rng.standard_normal(S1.shape)
    a, b = 0.7, -1.3
    f = lambda vv, SS: oracle.step_recurrence(q, k, vv, alpha, erase, write, variant, S0=SS)
    o1, s1 = f(v1, S1)
    o2, s2 = f(v2, S2)
    o3, s3 = f(a * v1 + b * v2, a * S1 + b * S2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-12)
    np.testing.assert_allclose(s3, a * s1 + b * s2, atol=1e-12)


# --------------------------------------------------------------------------- chunked form, varlen, decode

@pytest.mark.parametrize("variant", oracle.VARIANTS)
@pytest.mark.parametrize("chunk", [1, 4, 8, 16, 64])
def test_chunked_form_equals_step_recurrence(variant, chunk):
    """The chunkwise form gives the step recurrence's result (the pages ask for the
    scan/chunked kernel to be checked against the step recurrence)."""
    rng = np.random.default_rng(100 + chunk)
    q, k, v, alpha, erase, write, S0 = _rand_inputs(rng, 2, 37, 2, 8, 6, variant,
                                                    signed=True, zeros=True)
    o1, s1 = oracle.step_recurrence(q, k, v, alpha, erase, write, variant, S0=S0)
    o2, s2 = oracle.chunked_reference(q, k, v, alpha, erase, write, variant, S0=S0, chunk=chunk)
    assert oracle.rel_err(o2, o1) < 1e-12
    assert oracle.rel_err(s2, s1) < 1e-12


@pytest.mark.parametrize("variant", ["kda", "gdn2"])
def test_packed_sequences_are_isolated(variant):
    """Packed sequences (cu_seqlens) equal each sequence run alone; an empty sequence
    returns its initial state (course page, section 3: document reset, no shared state)."""
    rng = np.random.default_rng(19)
    lens = [5, 0, 9, 1, 17]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, alpha, erase, write, _ = _rand_inputs(rng, 1, T, 2, 6, 4, variant, signed=True)
    S0 = rng.standard_normal((len(lens), 2, 6, 4))
    o, S_T = oracle.step_recurrence(q, k, v, alpha, erase, write, variant, S0=S0, cu_seqlens=cu)
    oc, Sc = oracle.chunked_reference(q, k, v, alpha, erase, write, variant, S0=S0,
                                      cu_seqlens=cu, chunk=4)
    assert oracle.rel_err(oc, o) < 1e-12 and oracle.rel_err(Sc, S_T) < 1e-12
    for n in range(len(lens)):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        g = lambda x: None if x is None else x[:, sl]
        o1, s1 = oracle.step_recurrence(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], g(erase),
                                        g(write), variant, S0=S0[n:n + 1])
        assert np.array_equal(o[:, sl], o1)
        assert np.array_equal(S_T[n], s1[0])
    assert np.array_equal(S_T[1], S0[1])


@pytest.mark.parametrize("variant", oracle.VARIANTS)
def test_decode_steps_equal_recurrence(variant):
    """T single-token decode steps reproduce the recurrence over T tokens."""
    rng = np.random.default_rng(20)
    q, k, v, alpha, erase, write, S0 = _rand_inputs(rng, 3, 9, 2, 5, 7, variant, signed=True)
    o_ref, S_ref = oracle.step_recurrence(q, k, v, alpha, erase, write, variant, S0=S0)
    S = S0.copy()
    for t in range(9):
        S, o = oracle.decode_step(S, q[:, t], k[:, t], v[:, t], alpha[:, t], erase[:, t],
                                  None if write is None else write[:, t], variant)
        assert np.array_equal(o, o_ref[:, t])
    assert np.array_equal(S, S_ref)


def test_variant_gate_shapes_are_checked():
    rng = np.random.default_rng(21)
    q, k, v, alpha, erase, write, S0 = _rand_inputs(rng, 1, 3, 1, 4, 4, "rda")
    with pytest.raises(ValueError):
        oracle.step_recurrence(q, k, v, alpha, erase, write, "kda", S0=S0)
    with pytest.raises(ValueError):
        oracle.step_recurrence(q, k, v, alpha, erase, write, "gdn2", S0=S0)
    with pytest.raises(ValueError):
        oracle.step_recurrence(q, k, v, alpha, erase, None, "rda", S0=S0)


def test_rel_err_hand_example():
    """max|x - ref| / RMS(ref): x = (1,2,3,4), ref = (1,2,3,6) -> 2 / sqrt(12.5)."""
    assert oracle.rel_err([1, 2, 3, 4], [1, 2, 3, 6]) == pytest.approx(2 / np.sqrt(12.5), rel=1e-15)
    assert oracle.rel_err([0.0], [0.0]) == 0.0
    assert oracle.rel_err([1.0], [0.0]) == float("inf")
    assert not (oracle.rel_err([np.nan], [1.0]) <= 1.0)
