"""Two delta-rule transitions per token, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source. The abstract of "Complex KDA: Understanding and Enhancing the Expressivity of
Kimi Delta Attention" (the arXiv listing page) cites as prior work the composition of
two delta-rule transitions inside one recurrent update, which can express a 2D rotation
but raises the rank and cost of the update; the related-papers list on the same page
names that work, "DeltaProduct: Improving State-Tracking in Linear RNNs via Householder
Products". This module is that comparison variant with two factors.

Readings taken (the pages give no formula for it):
  * Token t carries two (key, value, beta) triples (k_t1, v_t1, beta_t1) and
    (k_t2, v_t2, beta_t2), one query q_t and one channel-wise decay alpha_t.
  * Each transition is KDA's rule; the decay acts once per token, before the first:
        S'  = (I - beta_t1 k_t1 k_t1^T) Diag(alpha_t) S_{t-1} + beta_t1 k_t1 v_t1^T
        S_t = (I - beta_t2 k_t2 k_t2^T) S'                    + beta_t2 k_t2 v_t2^T
  * The readout follows the second transition: o_t = S_t^T q_t.
  * beta may take Complex KDA's range [0, 2] (beta = 2 makes a factor a reflection).
Shapes: q, alpha [B,T,H,d_k]; k [B,T,H,2,d_k]; v [B,T,H,2,d_v]; beta [B,T,H,2].
"""
from __future__ import annotations

import numpy as np

from .recurrence import _f64, step
from .backward import step_recurrence_grads


def product_step(S, q, k, v, alpha, beta):
    """One token (two transitions) for every (sequence, head) in the leading axes.
    S [..., d_k, d_v]; q, alpha [..., d_k]; k [..., 2, d_k]; v [..., 2, d_v]; beta [..., 2].
    Returns (S_t, o_t).

    Pinned by: the explicit product of the two transition matrices; beta_t2 = 0
    reducing to KDA; two reflections composing to a rotation by twice the angle
    between the keys; norm preservation of orthogonal factors."""
    S = _f64(S)
    k, v, beta = _f64(k), _f64(v), _f64(beta)
    S1, _ = step(S, q, k[..., 0, :], v[..., 0, :], alpha, beta[..., 0], None, "kda")
    ones = np.ones(np.shape(alpha))
    return step(S1, q, k[..., 1, :], v[..., 1, :], ones, beta[..., 1], None, "kda")


def product_decode_step(S, q, k, v, alpha, beta):
    """Single-token decode of N sequences x H heads (q, alpha [N,H,d_k], k [N,H,2,d_k],
    v [N,H,2,d_v], beta [N,H,2], S [N,H,d_k,d_v]); same arithmetic as ``product_step``.

    Pinned by: T decode steps equal ``product_recurrence`` over T tokens."""
    return product_step(S, q, k, v, alpha, beta)


def product_recurrence(q, k, v, alpha, beta, S0=None, cu_seqlens=None):
    """Run the two-transition recurrence token by token; fixed-length or packed
    (cu_seqlens [N+1], B == 1; no state crosses a sequence boundary). Returns
    o [B,T,H,d_v] and S_T [N,H,d_k,d_v] in float64.

    Pinned by the pins of ``product_step`` plus: packed sequences equal each
    sequence run alone, and the recurrence equals KDA's on the sequence of 2T
    single transitions with the decay on the first of each pair."""
    q, k, v, alpha, beta = _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, T, H, 2, dk) or v.shape[:4] != (B, T, H, 2) or beta.shape != (B, T, H, 2):
        raise ValueError("k [B,T,H,2,d_k], v [B,T,H,2,d_v] and beta [B,T,H,2] expected")
    o = np.zeros((B, T, H, dv))
    if cu_seqlens is None:
        S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
        for t in range(T):
            S, o[:, t] = product_step(S, q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t])
        return o, S
    if B != 1:
        raise ValueError("packed sequences need B == 1")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    S_T = np.zeros((N, H, dk, dv))
    for n in range(N):
        S = np.zeros((H, dk, dv)) if S0 is None else _f64(S0[n]).copy()
        for t in range(int(cu[n]), int(cu[n + 1])):
            S, o[0, t] = product_step(S, q[0, t], k[0, t], v[0, t], alpha[0, t], beta[0, t])
        S_T[n] = S
    return o, S_T


def product_grads(q, k, v, alpha, beta, do, dS_T=None, S0=None, cu_seqlens=None):
    """Gradients of L = sum(o * do) + sum(S_T * dS_T) with respect to every input of
    ``product_recurrence``: a dict with dq, dalpha [B,T,H,d_k], dk [B,T,H,2,d_k],
    dv [B,T,H,2,d_v], dbeta [B,T,H,2] and dS0 [N,H,d_k,d_v], in float64.

    The two transitions of a token are two steps of KDA's rule, the decay alpha_t on the
    first and 1 on the second, and the output is read after the second; so this runs the
    reverse recurrence of ``backward.step_recurrence_grads`` on that sequence of 2T steps
    (zero output gradient after first steps) and maps the result back: k, v and beta
    per step, q and alpha from the step where they act.

    Pinned by central finite differences of ``product_recurrence`` on small inputs
    (signed gates, beta in [0, 2], packed sequences)."""
    q, k, v, alpha, beta, do = _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(beta), _f64(do)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    q2 = np.repeat(q, 2, axis=1)
    k2 = k.transpose(0, 1, 3, 2, 4).reshape(B, 2 * T, H, dk)
    v2 = v.transpose(0, 1, 3, 2, 4).reshape(B, 2 * T, H, dv)
    b2 = beta.transpose(0, 1, 3, 2).reshape(B, 2 * T, H)
    a2 = np.ones((B, 2 * T, H, dk))
    a2[:, 0::2] = alpha
    do2 = np.zeros((B, 2 * T, H, dv))
    do2[:, 1::2] = do
    cu2 = None if cu_seqlens is None else 2 * np.asarray(cu_seqlens, dtype=np.int64)
    g = step_recurrence_grads(q2, k2, v2, a2, b2, None, "kda", do2, dS_T=dS_T, S0=S0, cu_seqlens=cu2)
    return {
        "dq": g["dq"][:, 0::2] + g["dq"][:, 1::2],
        "dalpha": g["dalpha"][:, 0::2],
        "dk": g["dk"].reshape(B, T, 2, H, dk).transpose(0, 1, 3, 2, 4),
        "dv": g["dv"].reshape(B, T, 2, H, dv).transpose(0, 1, 3, 2, 4),
        "dbeta": g["derase"].reshape(B, T, 2, H).transpose(0, 1, 3, 2),
        "dS0": g["dS0"],
    }
