"""Step-by-step definition of the gated delta-rule recurrence, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the
smoke check and the benchmark's CPU-baseline leg, never by the library.

Source of the method. The three update rules are stated in the reply that lists
"the three state updates" in the Hugging Face discussion "KRAFTON/Raon-1-mini-
preview, discussion #1":

    KDA:   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    RDA:   S_t = (I - e_t k_t k_t^T)    Diag(alpha_t) S_{t-1} + w_t k_t v_t^T
    GDN-2: S_t = (I - k_t (b_t . k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T

with a channel-wise decay alpha_t in R^{d_k} shared by all three, per-head
scalar beta, e, w, and channel-wise b in R^{d_k}, w in R^{d_v} for GDN-2. The
abstract "Complex KDA: Understanding and Enhancing the Expressivity of Kimi
Delta Attention" (arXiv 2609.24797) keeps KDA's formula and widens its ranges to
alpha in [-1, 1] and beta in [0, 2] (CKDA).

Readings taken where the pages are silent:
  * S has shape d_k x d_v (rows = key channels), so Diag(alpha) scales key rows;
    this is the orientation the KDA formula's k v^T term forces.
  * Readout o_t = S_t^T q_t on the post-update state, with no 1/sqrt(d_k) scale.
  * The order is literal: decay, then erase, then write.
  * Every variant is written as S_t = X - k_t (u_t^T X) + k_t m_t^T with
    X = Diag(alpha_t) S_{t-1}; the erase vector u_t and write vector m_t are:
        KDA / CKDA: u = beta k,  m = beta v
        RDA:        u = e k,     m = w v
        GDN-2:      u = b . k,   m = w . v
    Expanding (I - k u^T) X = X - k (u^T X) is the only step between the
    page's formula and this code.
"""
from __future__ import annotations

import numpy as np

VARIANTS = ("kda", "rda", "gdn2", "ckda")


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def erase_write_vectors(variant: str, k, v, erase, write):
    """Erase direction u and write value m for one or many tokens (leading axes
    broadcast).  ``erase``/``write`` are per-head scalars (shape = leading axes) for
    KDA, CKDA and RDA and vectors for GDN-2; KDA and CKDA take no ``write`` and use
    beta (passed as ``erase``) for both, as in the KDA rule.

    Pinned by: RDA(e = w = beta) == KDA bit for bit; GDN-2 with uniform b, w ==
    RDA; the GDN-2 erase acting through b . k on the right factor only; the
    alpha = 0 closed form o_t = (q_t . k_t) m_t."""
    k, v, erase, write = _f64(k), _f64(v), _f64(erase), _f64(write)
    if variant in ("kda", "ckda"):
        if write is not None:
            raise ValueError(f"{variant} takes no separate write gate")
        u = erase[..., None] * k
        m = erase[..., None] * v
    elif variant == "rda":
        if write is None or erase.shape != k.shape[:-1] or write.shape != v.shape[:-1]:
            raise ValueError("rda needs per-head scalar erase and write gates")
        u = erase[..., None] * k
        m = write[..., None] * v
    elif variant == "gdn2":
        if write is None or erase.shape != k.shape or write.shape != v.shape:
            raise ValueError("gdn2 needs channel-wise erase [.., d_k] and write [.., d_v]")
        u = erase * k
        m = write * v
    else:
        raise ValueError(f"unknown variant {variant!r}")
    return u, m


def step(S, q, k, v, alpha, erase, write, variant: str):
    """One token of the recurrence for every (sequence, head) in the leading axes.

    S [..., d_k, d_v]; q, k, alpha [..., d_k]; v [..., d_v]; gates per variant.
    Returns (S_t, o_t) with o_t = S_t^T q_t.

    Pinned by: the 2D-rotation closed form, the delta read-back o_t = v_t, the
    linear-attention and gated-linear-attention closed forms, the full-decay
    closed form, norm preservation of orthogonal transitions, linearity."""
    S = _f64(S)
    q, k, alpha = _f64(q), _f64(k), _f64(alpha)
    u, m = erase_write_vectors(variant, k, v, erase, write)
    X = alpha[..., :, None] * S                                  # Diag(alpha_t) S_{t-1}
    erased = X - k[..., :, None] * np.einsum("...i,...ij->...j", u, X)[..., None, :]
    S_new = erased + k[..., :, None] * m[..., None, :]           # + k_t m_t^T
    o = np.einsum("...ij,...i->...j", S_new, q)                  # S_t^T q_t
    return S_new, o


def decode_step(S, q, k, v, alpha, erase, write, variant: str):
    """Single-token decode for N sequences x H heads: the fixed-size state is read,
    updated once and returned with the token's output (the step recurrence holds
    a state whose size does not grow with T, "GDN, KDA và Mamba-2" course page,
    sections 1 and 6).  Same arithmetic as ``step``.

    Pinned by: T decode steps equal ``step_recurrence`` over T tokens."""
    return step(S, q, k, v, alpha, erase, write, variant)


def _slice_gate(g, sl):
    return None if g is None else g[sl]


def step_recurrence(q, k, v, alpha, erase, write, variant: str, S0=None, cu_seqlens=None):
    """Run the recurrence token by token.

    Fixed length: q, k, alpha [B,T,H,d_k]; v [B,T,H,d_v]; S0 [B,H,d_k,d_v] or None.
    Packed (cu_seqlens [N+1], B == 1): sequence n spans tokens cu[n]:cu[n+1] and
    starts from S0[n]; no state crosses a sequence boundary (the course page's
    section 3: document reset, and no two requests share a state).
    Returns o [B,T,H,d_v] and S_T [N,H,d_k,d_v], both float64.

    Pinned by every closed form listed in ``step`` plus: packed sequences equal
    each sequence run alone; zero-length sequences return S0 unchanged."""
    q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
    erase, write = _f64(erase), _f64(write)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    if cu_seqlens is None:
        S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
        for t in range(T):
            sl = (slice(None), t)
            S, o[:, t] = step(S, q[sl], k[sl], v[sl], alpha[sl], erase[sl],
                              _slice_gate(write, sl), variant)
        return o, S
    if B != 1:
        raise ValueError("packed sequences need B == 1")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    S_T = np.zeros((N, H, dk, dv))
    for n in range(N):
        S = np.zeros((H, dk, dv)) if S0 is None else _f64(S0[n]).copy()
        for t in range(int(cu[n]), int(cu[n + 1])):
            sl = (0, t)
            S, o[0, t] = step(S, q[sl], k[sl], v[sl], alpha[sl], erase[sl],
                              _slice_gate(write, sl), variant)
        S_T[n] = S
    return o, S_T


def transition_matrix(alpha, k, u):
    """The d_k x d_k matrix (I - k u^T) Diag(alpha) that multiplies S_{t-1}.

    Pinned by: the 2D rotation (Complex KDA abstract: a reflection with beta = 2
    composed with the gate's sign flip gives a rotation), agreement with ``step``
    on the homogeneous part, and the non-expansive / orthogonal properties the
    same abstract states for CKDA transitions."""
    alpha, k, u = _f64(alpha), _f64(k), _f64(u)
    d = alpha.shape[-1]
    return (np.eye(d) - np.outer(k, u)) @ np.diag(alpha)


def rel_err(x, ref) -> float:
    """max_i |x_i - ref_i| / sqrt(mean(ref^2)) over the whole tensor, in float64.

    Pinned by a hand-computed example."""
    x, ref = _f64(x), _f64(ref)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    if ref.size == 0:
        return 0.0
    err = float(np.max(np.abs(x - ref)))
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return 0.0 if err == 0.0 else float("inf")
    return err / rms
