"""Stored states around the recurrence, in float64: snapshots for prefix sharing and
prefill / decode against a pool of state slots.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source. Section 3 of the course page "GDN, KDA và Mamba-2 · cập nhật state trong
hybrid" separates three things a serving stack must not confuse: padding, a
document reset (a sequence starts from its own state) and a state snapshot kept
for prefix sharing; two requests may never share a state that holds different
content. Readings taken where the page is silent:
  * A snapshot is the state S_p after the first p tokens of a sequence, taken at
    p = every, 2 every, ... up to the sequence length; sequence n's snapshots are
    stored one after another, after those of sequences 0..n-1.
  * A state pool holds one state per slot; sequence n reads and writes slot
    state_idx[n]. A slot outside the pool means "no stored state": a prefill
    starts from the zero state and stores nothing, a decode step outputs zeros and
    touches nothing. Slots that no sequence names are left as they are.
"""
from __future__ import annotations

import numpy as np

from .recurrence import _f64, _slice_gate, step, step_recurrence


def _spans(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def snapshot_count(lengths, every: int) -> int:
    """Number of snapshots for sequences of the given lengths: floor(len / every) each."""
    return int(sum(int(n) // every for n in lengths))


def snapshots(q, k, v, alpha, erase, write, variant: str, every: int, S0=None, cu_seqlens=None):
    """States after every ``every`` tokens of each sequence, run token by token.

    Shapes as in ``step_recurrence``. Returns [num, H, d_k, d_v] float64 with
    num = sum_n floor(len_n / every); row first_n + j is sequence n's state after
    (j + 1) * every tokens, first_n = sum_{m<n} floor(len_m / every).

    Pinned by: each snapshot equals the final state of the recurrence run on that
    prefix alone; resuming from a snapshot reproduces the rest of the sequence
    (outputs and final state); the linear-attention closed form
    S_p = S0 + sum_{t<p} k_t v_t^T."""
    if every <= 0:
        raise ValueError("every must be positive")
    q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
    erase, write = _f64(erase), _f64(write)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = []
    for n, (b, t0, t1) in enumerate(_spans(B, T, cu_seqlens)):
        S = np.zeros((H, dk, dv)) if S0 is None else _f64(S0[n]).copy()
        for t in range(t0, t1):
            sl = (b, t)
            S, _ = step(S, q[sl], k[sl], v[sl], alpha[sl], erase[sl], _slice_gate(write, sl), variant)
            if (t - t0 + 1) % every == 0:
                out.append(S.copy())
    return np.stack(out) if out else np.zeros((0, H, dk, dv))


def pooled_prefill(q, k, v, alpha, erase, write, variant: str, pool, state_idx, cu_seqlens=None):
    """Prefill whose initial and final states live in slots of ``pool`` [P,H,d_k,d_v].

    Sequence n starts from pool[state_idx[n]] and its final state replaces that row;
    with a slot outside [0, P) it starts from zero and nothing is stored.
    Returns (o, new_pool), float64.

    Pinned by: with state_idx = arange(N) and a pool of N rows this is
    ``step_recurrence`` with S0 = pool; rows not named keep their values; an
    out-of-range slot gives the zero-state outputs."""
    pool = _f64(pool)
    P = pool.shape[0]
    idx = np.asarray(state_idx, dtype=np.int64)
    valid = (idx >= 0) & (idx < P)
    S0 = np.stack([pool[i] if ok else np.zeros(pool.shape[1:]) for i, ok in zip(idx, valid)]) \
        if len(idx) else np.zeros((0,) + pool.shape[1:])
    o, S_T = step_recurrence(q, k, v, alpha, erase, write, variant, S0=S0, cu_seqlens=cu_seqlens)
    new = pool.copy()
    for n, (i, ok) in enumerate(zip(idx, valid)):
        if ok:
            new[i] = S_T[n]
    return o, new


def pooled_decode_step(pool, state_idx, q, k, v, alpha, erase, write, variant: str):
    """One decode step for N sequences whose states are rows state_idx[n] of ``pool``.

    q, k, alpha [N,H,d_k]; v [N,H,d_v]; gates [N,H] or [N,H,d] per variant.
    Returns (new_pool, o [N,H,d_v]); a slot outside the pool gives o = 0 and leaves
    the pool alone.

    Pinned by: a permutation of slots equals the plain step on permuted states;
    out-of-range slots give zeros and change nothing; the full-decay closed form
    o = (q . k) m, independent of the stored state."""
    pool = _f64(pool)
    P = pool.shape[0]
    idx = np.asarray(state_idx, dtype=np.int64)
    q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
    erase, write = _f64(erase), _f64(write)
    N, H, _ = q.shape
    o = np.zeros((N, H, v.shape[-1]))
    new = pool.copy()
    for n in range(N):
        i = int(idx[n])
        if not (0 <= i < P):
            continue
        new[i], o[n] = step(pool[i], q[n], k[n], v[n], alpha[n], erase[n], _slice_gate(write, n), variant)
    return new, o
