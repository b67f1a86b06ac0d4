"""Gradients of the gated delta-rule recurrence, in float64, by the reverse recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source. The course page "GDN, KDA và Mamba-2 · cập nhật state trong hybrid", section 3,
notes that training needs activations, checkpointing and the intermediates of the scan /
chunked form; this is the gradient that training needs, taken through the step rule of
``recurrence.step`` (the three update rules of the Raon-1-mini-preview discussion, Complex KDA
with KDA's rule).

Forward, per token (X = Diag(alpha_t) S_{t-1}, u and m the erase / write vectors):
    delta_t = m_t - X^T u_t,   S_t = X + k_t delta_t^T,   o_t = S_t^T q_t
Reverse, with G the gradient reaching S_t (from later tokens, plus q_t do_t^T from o_t):
    dq_t     = S_t do_t
    d(delta) = G^T k_t                 dk_t += G delta_t        dm_t = d(delta)
    dX       = G - u_t d(delta)^T      du_t  = -X d(delta)
    dalpha_t = rowsum(dX * S_{t-1})    (the gradient reaching S_{t-1} is Diag(alpha_t) dX)
and then through u and m to the gates: KDA / CKDA u = beta k, m = beta v; RDA u = e k,
m = w v; GDN-2 u = b . k, m = w . v.
No step divides by a gate, so zero and negative gates need nothing special.
"""
from __future__ import annotations

import numpy as np

from .recurrence import _f64, _slice_gate, erase_write_vectors, step


def _step_grads(S_prev, q, k, v, alpha, erase, write, variant, G, do):
    """Gradients of one token for every leading (sequence, head) axis. G is the gradient
    reaching S_t from later tokens; returns (dS_prev, dq, dk, dv, dalpha, derase, dwrite)."""
    u, m = erase_write_vectors(variant, k, v, erase, write)
    X = alpha[..., :, None] * S_prev
    delta = m - np.einsum("...ij,...i->...j", X, u)
    S_t = X + k[..., :, None] * delta[..., None, :]
    G = G + q[..., :, None] * do[..., None, :]                      # o_t = S_t^T q_t
    dq = np.einsum("...ij,...j->...i", S_t, do)
    ddelta = np.einsum("...ij,...i->...j", G, k)
    dk = np.einsum("...ij,...j->...i", G, delta)
    dX = G - u[..., :, None] * ddelta[..., None, :]
    du = -np.einsum("...ij,...j->...i", X, ddelta)
    dm = ddelta
    dalpha = np.sum(dX * S_prev, axis=-1)
    dS_prev = alpha[..., :, None] * dX
    # through the variant's erase / write vectors
    if variant in ("kda", "ckda"):
        dk = dk + erase[..., None] * du
        derase = np.sum(k * du, axis=-1) + np.sum(v * dm, axis=-1)
        dv = erase[..., None] * dm
        dwrite = None
    elif variant == "rda":
        dk = dk + erase[..., None] * du
        derase = np.sum(k * du, axis=-1)
        dwrite = np.sum(v * dm, axis=-1)
        dv = write[..., None] * dm
    elif variant == "gdn2":
        dk = dk + erase * du
        derase = k * du
        dwrite = v * dm
        dv = write * dm
    else:
        raise ValueError(f"unknown variant {variant!r}")
    return dS_prev, dq, dk, dv, dalpha, derase, dwrite


def step_recurrence_grads(q, k, v, alpha, erase, write, variant: str, do, dS_T=None, S0=None,
                          cu_seqlens=None):
    """Gradients of L = sum(o * do) + sum(S_T * dS_T) with respect to every input of
    ``step_recurrence``. Shapes as there; do [B,T,H,d_v], dS_T [N,H,d_k,d_v] or None.
    Returns a dict with dq, dk, dv, dalpha, derase, dwrite (None for KDA / CKDA: beta's whole
    gradient is in derase) and dS0, all float64.

    Pinned by: central finite differences of ``step_recurrence`` on small inputs for every
    variant, signed and zero gates included; PyTorch float64 autograd through a literal
    transcription of the step rule; the linear-attention closed form (alpha = 1, e = 0:
    dq_t = S_t do_t, dv_s = w_s sum_{t>=s} (q_t . k_s) do_t)."""
    q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
    erase, write, do = _f64(erase), _f64(write), _f64(do)
    B, T, H, dk_ = q.shape
    dv_ = v.shape[-1]
    out = {name: np.zeros_like(x) for name, x in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha),
                                                   ("derase", erase))}
    out["dwrite"] = None if write is None else np.zeros_like(write)
    if cu_seqlens is None:
        spans = [(b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        spans = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    N = len(spans)
    dS0 = np.zeros((N, H, dk_, dv_))
    for n, (b, t0, t1) in enumerate(spans):
        S = np.zeros((H, dk_, dv_)) if S0 is None else _f64(S0[n]).copy()
        states = [S]
        for t in range(t0, t1):                                   # forward: keep every state
            sl = (b, t)
            S, _ = step(S, q[sl], k[sl], v[sl], alpha[sl], erase[sl], _slice_gate(write, sl), variant)
            states.append(S)
        G = np.zeros((H, dk_, dv_)) if dS_T is None else _f64(dS_T[n]).copy()
        for t in range(t1 - 1, t0 - 1, -1):                       # reverse
            sl = (b, t)
            G, dq, dk, dv, da, de, dw = _step_grads(states[t - t0], q[sl], k[sl], v[sl], alpha[sl], erase[sl],
                                                     _slice_gate(write, sl), variant, G, do[sl])
            out["dq"][sl], out["dk"][sl], out["dv"][sl], out["dalpha"][sl], out["derase"][sl] = dq, dk, dv, da, de
            if dw is not None:
                out["dwrite"][sl] = dw
        dS0[n] = G
    out["dS0"] = dS0
    return out
