"""Chunkwise-parallel form of the recurrence, in float64 — a second statement of
the same result, used to check the chunk algebra the HIP prefill kernel is built
on.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name a "scan/chunked kernel" and say its error and latency are to be
measured against the step recurrence in the same dtype (course page "GDN, KDA
và Mamba-2", sections 3 and 4), but they do not write the chunked form out.
The form below is derived by unrolling the step rule of ``recurrence.step``
inside a chunk; it is exact algebra, not an approximation.

Within a chunk of L tokens r = 1..L starting from state S0:
    ratio(r, s) = prod_{j=s+1..r} alpha_j       (elementwise over key channels; 1 when r = s)
    Gamma_r     = prod_{j<=r} alpha_j
    A[r, s]     = sum_i u_ri k_si ratio(r, s)_i     for s < r   (strictly lower)
    P[r, s]     = sum_i q_ri k_si ratio(r, s)_i     for s <= r  (lower)
    (I + A) delta = M - Utilde S0,   Utilde_r = Gamma_r . u_r,  M rows m_r
    O           = Qtilde S0 + P delta,  Qtilde_r = Gamma_r . q_r
    S_L         = Diag(Gamma_L) S0 + Kbar^T delta,  Kbar_s = ratio(L, s) . k_s
where delta_r = m_r - S_{r-1}^T (alpha_r . u_r) is the delta-rule error of token r.

Every ratio is an explicit product of gates (no logarithms, no division), and the
triangular system is solved with numpy's dense solver.

Pinned by: equality with ``step_recurrence`` for chunk sizes 1, 4, 8, 16 and 64,
partial last chunks, signed and zero gates, and every variant.
"""
from __future__ import annotations

import numpy as np

from .recurrence import erase_write_vectors


def _chunk(q, k, alpha, u, m, S0):
    """One chunk for all heads. q, k, alpha, u [H, L, d_k]; m [H, L, d_v]; S0 [H, d_k, d_v]."""
    H, L, dk = q.shape
    ratio = np.zeros((H, L, L, dk))
    for r in range(L):
        ratio[:, r, r] = 1.0
        for s in range(r):
            ratio[:, r, s] = ratio[:, r - 1, s] * alpha[:, r]
    gamma = np.cumprod(alpha, axis=1)                                   # Gamma_r
    A = np.einsum("hri,hsi,hrsi->hrs", u, k, ratio) * np.tril(np.ones((L, L)), -1)
    P = np.einsum("hri,hsi,hrsi->hrs", q, k, ratio) * np.tril(np.ones((L, L)), 0)
    Ut = gamma * u
    Qt = gamma * q
    Kbar = ratio[:, L - 1] * k                                          # ratio(L, s) . k_s
    rhs = m - np.einsum("hri,hij->hrj", Ut, S0)
    delta = np.linalg.solve(np.eye(L)[None] + A, rhs)
    O = np.einsum("hri,hij->hrj", Qt, S0) + np.einsum("hrs,hsj->hrj", P, delta)
    S_L = gamma[:, L - 1, :, None] * S0 + np.einsum("hsi,hsj->hij", Kbar, delta)
    return O, S_L


def chunked_reference(q, k, v, alpha, erase, write, variant: str, S0=None, cu_seqlens=None,
                      chunk: int = 64):
    """Same arguments and results as ``step_recurrence``, computed chunk by chunk.
    Chunks are aligned to each sequence's first token; the last chunk of a sequence
    may be partial."""
    q, k, v, alpha = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    u, m = erase_write_vectors(variant, k, v, erase, write)
    if cu_seqlens is None:
        bounds = [(b, 0, T) for b in range(B)]
    else:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        bounds = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((len(bounds), H, dk, dv))
    for n, (b, t0, t1) in enumerate(bounds):
        S = np.zeros((H, dk, dv)) if S0 is None else np.asarray(S0[n], dtype=np.float64).copy()
        for c0 in range(t0, t1, chunk):
            c1 = min(c0 + chunk, t1)
            tr = lambda x: np.transpose(x[b, c0:c1], (1, 0, 2))  # noqa: E731  [H, L, d]
            O, S = _chunk(tr(q), tr(k), tr(alpha), tr(u), tr(m), S)
            o[b, c0:c1] = np.transpose(O, (1, 0, 2))
        S_T[n] = S
    return o, S_T
