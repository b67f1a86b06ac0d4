"""Pins for the oracle's gradients (reverse recurrence): central finite differences of the
forward recurrence, PyTorch float64 autograd through a literal transcription of the step
rule, a linear-attention closed form, and packed sequences. CPU only."""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward
from test_oracle_pins import _rand_inputs

RNG = np.random.default_rng(20261206)


def _loss(a, variant, do, dS_T, S0, cu=None):
    o, S_T = oracle.step_recurrence(*a, variant, S0=S0, cu_seqlens=cu)
    return float(np.sum(o * do) + np.sum(S_T * dS_T))


def _inputs(variant, B=1, T=6, H=1, dk=3, dv=2, signed=False, zeros=False):
    q, k, v, alpha, erase, write, S0 = _rand_inputs(RNG, B, T, H, dk, dv, variant, signed=signed, zeros=zeros)
    return [q, k, v, alpha, erase, write], S0


@pytest.mark.parametrize("variant,signed,zeros", [("kda", False, False), ("rda", False, True),
                                                  ("gdn2", False, False), ("ckda", True, True)])
def test_gradients_match_central_differences(variant, signed, zeros):
    a, S0 = _inputs(variant, signed=signed, zeros=zeros)
    do = RNG.standard_normal(a[2].shape)
    dS_T = RNG.standard_normal(S0.shape)
    g = backward.step_recurrence_grads(*a, variant, do, dS_T=dS_T, S0=S0)
    names = ["dq", "dk", "dv", "dalpha", "derase", "dwrite"]
    eps = 1e-6
    for idx, name in enumerate(names):
        x = a[idx]
        if x is None:
            assert g[name] is None
            continue
        num = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            ap, am = list(a), list(a)
            ap[idx], am[idx] = xp, xm
            num[i] = (_loss(ap, variant, do, dS_T, S0) - _loss(am, variant, do, dS_T, S0)) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8, err_msg=name)
    num = np.zeros_like(S0)
    for i in np.ndindex(S0.shape):
        sp, sm = S0.copy(), S0.copy()
        sp[i] += eps
        sm[i] -= eps
        num[i] = (_loss(a, variant, do, dS_T, sp) - _loss(a, variant, do, dS_T, sm)) / (2 * eps)
    np.testing.assert_allclose(g["dS0"], num, rtol=1e-6, atol=1e-8, err_msg="dS0")


def _torch_step_rule(q, k, v, alpha, erase, write, variant, S0):
    """The step rule written out literally: S_t = (I - k u^T) Diag(alpha) S_{t-1} + k m^T."""
    B, T, H, dk = q.shape
    S = S0.clone()
    outs = []
    eye = torch.eye(dk, dtype=torch.float64)
    for t in range(T):
        kt, vt, qt, at = k[:, t], v[:, t], q[:, t], alpha[:, t]
        if variant in ("kda", "ckda"):
            u, m = erase[:, t, :, None] * kt, erase[:, t, :, None] * vt
        elif variant == "rda":
            u, m = erase[:, t, :, None] * kt, write[:, t, :, None] * vt
        else:
            u, m = erase[:, t] * kt, write[:, t] * vt
        trans = eye - kt[..., :, None] * u[..., None, :]             # I - k u^T
        S = trans @ (at[..., :, None] * S) + kt[..., :, None] * m[..., None, :]
        outs.append(torch.einsum("bhij,bhi->bhj", S, qt))
    return torch.stack(outs, 1), S


@pytest.mark.parametrize("variant", oracle.VARIANTS)
def test_gradients_match_torch_autograd(variant):
    a, S0 = _inputs(variant, B=2, T=9, H=2, dk=4, dv=3, signed=(variant == "ckda"), zeros=True)
    do = RNG.standard_normal(a[2].shape)
    dS_T = RNG.standard_normal(S0.shape)
    g = backward.step_recurrence_grads(*a, variant, do, dS_T=dS_T, S0=S0)
    ts = [None if x is None else torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in a]
    tS0 = torch.tensor(S0, dtype=torch.float64, requires_grad=True)
    o, S_T = _torch_step_rule(*ts, variant, tS0)
    loss = (o * torch.tensor(do)).sum() + (S_T * torch.tensor(dS_T)).sum()
    loss.backward()
    for name, t in zip(["dq", "dk", "dv", "dalpha", "derase", "dwrite"], ts):
        if t is None:
            continue
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)
    np.testing.assert_allclose(g["dS0"], tS0.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_linear_attention_gradients_closed_form():
    # alpha = 1, e = 0, w = 1 (RDA): o_t = S0^T q_t + sum_{s<=t} (q_t . k_s) v_s
    B, T, H, dk, dv = 1, 7, 2, 4, 3
    q = RNG.standard_normal((B, T, H, dk))
    k = RNG.standard_normal((B, T, H, dk))
    v = RNG.standard_normal((B, T, H, dv))
    S0 = RNG.standard_normal((B, H, dk, dv))
    do = RNG.standard_normal((B, T, H, dv))
    g = backward.step_recurrence_grads(q, k, v, np.ones((B, T, H, dk)), np.zeros((B, T, H)), np.ones((B, T, H)),
                                       "rda", do, S0=S0)
    qk = np.einsum("bthi,bshi->bhts", q, k)                       # q_t . k_s
    mask = np.tril(np.ones((T, T)))
    dv_ref = np.einsum("bhts,bthj->bshj", qk * mask, do)          # sum over t >= s
    np.testing.assert_allclose(g["dv"], dv_ref, rtol=0, atol=1e-12)
    S = S0[:, None] + np.cumsum(np.einsum("bthi,bthj->bthij", k, v), axis=1)
    dq_ref = np.einsum("bthij,bthj->bthi", S, do)
    np.testing.assert_allclose(g["dq"], dq_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dS0"], np.einsum("bthi,bthj->bhij", q, do), rtol=0, atol=1e-12)


def test_packed_sequence_gradients_are_per_sequence():
    lens = [3, 0, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    a, _ = _inputs("gdn2", T=int(cu[-1]), H=2, dk=3, dv=2)
    S0 = RNG.standard_normal((3, 2, 3, 2))
    do = RNG.standard_normal(a[2].shape)
    dS_T = RNG.standard_normal(S0.shape)
    g = backward.step_recurrence_grads(*a, "gdn2", do, dS_T=dS_T, S0=S0, cu_seqlens=cu)
    for n in range(3):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        sl = (slice(0, 1), slice(t0, t1))
        gn = backward.step_recurrence_grads(*[x[sl] for x in a], "gdn2", do[sl], dS_T=dS_T[n:n + 1], S0=S0[n:n + 1])
        for name in ("dq", "dk", "dv", "dalpha", "derase", "dwrite"):
            np.testing.assert_array_equal(g[name][sl], gn[name])
        np.testing.assert_array_equal(g["dS0"][n], gn["dS0"][0])
    np.testing.assert_array_equal(g["dS0"][1], dS_T[1])            # an empty sequence passes dS_T through


@pytest.mark.parametrize("signed", [False, True])
def test_reverse_chain_is_a_time_reversed_forward_run(signed):
    # With a symmetric erase factor (I - e_t k_t k_t^T) (KDA, RDA, Complex KDA) the gradient
    # chain E_{t-1} = Diag(alpha_t) (I - e_t k_t k_t^T) E_t + q_{t-1} do_{t-1}^T is the forward
    # recurrence itself, in RDA form, on reversed and interleaved steps: an erase-only step
    # (key k_t, erase e_t) and a write-only step (decay alpha_t, key q_{t-1}, value do_{t-1}).
    # Its readout with query k_t after the write-only step that forms E_t is d(delta)_t, and its
    # final state is dS0: the reverse recurrence is pinned against the forward one.
    rng = np.random.default_rng(31 + signed)
    T, H, dk, dv = 9, 2, 5, 4
    q, k = rng.standard_normal((1, T, H, dk)), rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    alpha = rng.uniform(-1.0, 1.0, (1, T, H, dk)) if signed else rng.uniform(0.3, 1.0, (1, T, H, dk))
    e, w = rng.uniform(0.0, 2.0, (1, T, H)), rng.uniform(0.1, 1.0, (1, T, H))
    S0, dS_T = rng.standard_normal((1, H, dk, dv)), rng.standard_normal((1, H, dk, dv))
    dO = rng.standard_normal((1, T, H, dv))
    g = backward.step_recurrence_grads(q, k, v, alpha, e, w, "rda", dO, dS_T=dS_T, S0=S0)

    n = 2 * T + 1
    Q, K = np.zeros((1, n, H, dk)), np.zeros((1, n, H, dk))
    V, A = np.zeros((1, n, H, dv)), np.ones((1, n, H, dk))
    E, W = np.zeros((1, n, H)), np.zeros((1, n, H))
    K[0, 0], V[0, 0], W[0, 0], Q[0, 0] = q[0, T - 1], dO[0, T - 1], 1.0, k[0, T - 1]  # forms E_{T-1}
    for i, t in enumerate(range(T - 1, -1, -1)):
        a, b = 1 + 2 * i, 2 + 2 * i
        K[0, a], E[0, a] = k[0, t], e[0, t]                  # (I - e_t k_t k_t^T)
        A[0, b] = alpha[0, t]                                # Diag(alpha_t)
        if t >= 1:                                           # + q_{t-1} do_{t-1}^T, read with k_{t-1}
            K[0, b], V[0, b], W[0, b], Q[0, b] = q[0, t - 1], dO[0, t - 1], 1.0, k[0, t - 1]
    o_r, S_r = oracle.step_recurrence(Q, K, V, A, E, W, "rda", S0=dS_T)
    np.testing.assert_allclose(S_r, g["dS0"], rtol=1e-10, atol=1e-10)
    for t in range(T):
        dR = o_r[0, 2 * (T - 1 - t)]                         # d(delta)_t = dL/dm_t
        np.testing.assert_allclose(w[0, t][:, None] * dR, g["dv"][0, t], rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("signed", [False, True])
def test_gate_gradient_is_a_reverse_cumulative_sum(signed):
    """Every decay factor of the recurrence unrolled over a sequence is a product of consecutive
    gates alpha_{s+1} ... alpha_r, and alpha_t times its derivative in alpha_t is the product itself
    when s < t <= r. Grouping the products by their last index r (terms in q_r . dq_r and
    u_r . du_r), by their first index s + 1 (terms in k_s . dk_s, k as the key only) and by the
    end state: alpha_t . dalpha_t = sum_{j >= t} (q_j . dq_j + u_j . du_j - k_j . dk_j) +
    rowsum(dS_T . S_T), per channel. With GDN-2's u = b . k, u . du = b . derase and the key-only
    k . dk is k . dk - b . derase. The identity is what a chunked backward can compute the gate
    gradient from (a reverse scan, then a division by alpha); here the oracle's gradients, from
    the reverse walk, must satisfy it."""
    a, S0 = _inputs("gdn2", B=2, T=9, H=2, dk=4, dv=3, signed=signed)
    a[3][np.abs(a[3]) < 0.05] = 0.5  # away from zero: the identity divides by alpha
    q, k, v, alpha, erase, write = a
    do = RNG.standard_normal(v.shape)
    dS_T = RNG.standard_normal(S0.shape)
    g = backward.step_recurrence_grads(q, k, v, alpha, erase, write, "gdn2", do, dS_T=dS_T, S0=S0)
    _, S_T = oracle.step_recurrence(q, k, v, alpha, erase, write, "gdn2", S0=S0)
    per_token = q * g["dq"] + 2 * erase * g["derase"] - k * g["dk"]        # [B, T, H, d_k]
    rhs = np.flip(np.cumsum(np.flip(per_token, axis=1), axis=1), axis=1)   # sum over j >= t
    rhs = rhs + np.sum(dS_T * S_T, axis=-1)[:, None]                       # end state, per channel
    np.testing.assert_allclose(alpha * g["dalpha"], rhs, rtol=1e-10, atol=1e-12)
