"""Pins for the stored-state functions of the oracle (snapshots for prefix sharing, slot
pools for prefill and decode): brute force on prefixes, resumption, closed forms and
permutation invariants. CPU only."""
import numpy as np
import pytest

import oracle
from oracle import states
from test_oracle_pins import _rand_inputs, _unit

RNG = np.random.default_rng(20261204)


def _seq_inputs(a, b, t0, t1):
    """Tokens t0..t1-1 of batch row b as a one-row batch."""
    q, k, v, alpha, erase, write = a
    sl = (slice(b, b + 1), slice(t0, t1))
    return q[sl], k[sl], v[sl], alpha[sl], erase[sl], None if write is None else write[sl]


@pytest.mark.parametrize("variant", oracle.VARIANTS)
def test_snapshot_is_the_state_of_the_prefix_alone(variant):
    B, T, H, dk, dv, every = 2, 37, 2, 4, 3, 8
    a = _rand_inputs(RNG, B, T, H, dk, dv, variant, signed=(variant == "ckda"))[:6]
    S0 = RNG.standard_normal((B, H, dk, dv))
    snaps = states.snapshots(*a, variant, every, S0=S0)
    assert snaps.shape == (B * (T // every), H, dk, dv)
    for b in range(B):
        for j in range(T // every):
            p = (j + 1) * every
            _, S_p = oracle.step_recurrence(*_seq_inputs(a, b, 0, p), variant, S0=S0[b:b + 1])
            np.testing.assert_allclose(snaps[b * (T // every) + j], S_p[0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("variant", ["kda", "gdn2"])
def test_resuming_from_a_snapshot_reproduces_the_sequence(variant):
    lens = [0, 20, 9, 33, 16]
    cu = np.concatenate([[0], np.cumsum(lens)])
    a = _rand_inputs(RNG, 1, int(cu[-1]), 2, 4, 5, variant)[:6]
    S0 = RNG.standard_normal((len(lens), 2, 4, 5))
    every = 8
    o, S_T = oracle.step_recurrence(*a, variant, S0=S0, cu_seqlens=cu)
    snaps = states.snapshots(*a, variant, every, S0=S0, cu_seqlens=cu)
    assert snaps.shape[0] == states.snapshot_count(lens, every) == 0 + 2 + 1 + 4 + 2
    row = 0
    for n, L in enumerate(lens):
        for j in range(L // every):
            p = (j + 1) * every
            t0 = int(cu[n]) + p
            o2, S2 = oracle.step_recurrence(*_seq_inputs(a, 0, t0, int(cu[n + 1])), variant,
                                            S0=snaps[row][None])
            np.testing.assert_allclose(o2[0], o[0, t0:int(cu[n + 1])], rtol=0, atol=1e-12)
            np.testing.assert_allclose(S2[0], S_T[n], rtol=0, atol=1e-12)
            row += 1
    assert row == snaps.shape[0]


def test_snapshots_of_linear_attention_are_running_sums():
    # alpha = 1, e = 0, w = 1 (RDA): S_p = S0 + sum_{t<p} k_t v_t^T
    B, T, H, dk, dv, every = 1, 24, 3, 5, 4, 6
    q = RNG.standard_normal((B, T, H, dk))
    k = RNG.standard_normal((B, T, H, dk))
    v = RNG.standard_normal((B, T, H, dv))
    S0 = RNG.standard_normal((B, H, dk, dv))
    snaps = states.snapshots(q, k, v, np.ones((B, T, H, dk)), np.zeros((B, T, H)), np.ones((B, T, H)),
                             "rda", every, S0=S0)
    outer = np.einsum("bthi,bthj->bthij", k, v)
    run = S0[:, None] + np.cumsum(outer, axis=1)
    np.testing.assert_allclose(snaps, run[0, every - 1::every], rtol=0, atol=1e-12)


def test_no_snapshot_before_the_first_full_stride():
    a = _rand_inputs(RNG, 1, 7, 1, 4, 4, "kda")[:6]
    assert states.snapshots(*a, "kda", 8).shape == (0, 1, 4, 4)
    with pytest.raises(ValueError):
        states.snapshots(*a, "kda", 0)


@pytest.mark.parametrize("variant", ["rda", "ckda"])
def test_pooled_prefill_with_identity_slots_is_the_plain_prefill(variant):
    a = _rand_inputs(RNG, 3, 11, 2, 4, 3, variant, signed=(variant == "ckda"))[:6]
    pool = RNG.standard_normal((3, 2, 4, 3))
    o, new = states.pooled_prefill(*a, variant, pool, np.arange(3))
    o_ref, S_ref = oracle.step_recurrence(*a, variant, S0=pool)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(new, S_ref)


def test_pooled_prefill_touches_only_named_slots():
    lens = [5, 0, 12]
    cu = np.concatenate([[0], np.cumsum(lens)])
    a = _rand_inputs(RNG, 1, int(cu[-1]), 2, 4, 3, "gdn2")[:6]
    pool = RNG.standard_normal((6, 2, 4, 3))
    idx = np.array([4, -1, 1])  # the middle sequence has no stored state
    o, new = states.pooled_prefill(*a, "gdn2", pool, idx, cu_seqlens=cu)
    S0 = np.stack([pool[4], np.zeros((2, 4, 3)), pool[1]])
    o_ref, S_ref = oracle.step_recurrence(*a, "gdn2", S0=S0, cu_seqlens=cu)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(new[4], S_ref[0])
    np.testing.assert_array_equal(new[1], S_ref[2])
    for r in (0, 2, 3, 5):
        np.testing.assert_array_equal(new[r], pool[r])
    # an out-of-range slot behaves like no stored state
    o_far, new_far = states.pooled_prefill(*a, "gdn2", pool, np.array([4, 6, 1]), cu_seqlens=cu)
    np.testing.assert_array_equal(o_far, o)
    np.testing.assert_array_equal(new_far, new)


@pytest.mark.parametrize("variant", oracle.VARIANTS)
def test_pooled_decode_is_the_step_on_gathered_states(variant):
    N, H, dk, dv, P = 5, 2, 4, 3, 8
    a = _rand_inputs(RNG, 1, N, H, dk, dv, variant, signed=(variant == "ckda"))[:6]
    q, k, v, alpha, erase, write = (None if x is None else x[0] for x in a)
    pool = RNG.standard_normal((P, H, dk, dv))
    idx = np.array([6, 0, 3, 7, 2])
    new, o = states.pooled_decode_step(pool, idx, q, k, v, alpha, erase, write, variant)
    S_ref, o_ref = oracle.decode_step(pool[idx], q, k, v, alpha, erase, write, variant)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(new[idx], S_ref)
    untouched = np.setdiff1d(np.arange(P), idx)
    np.testing.assert_array_equal(new[untouched], pool[untouched])


def test_pooled_decode_skips_slots_outside_the_pool():
    N, H, dk, dv, P = 4, 1, 4, 4, 3
    a = _rand_inputs(RNG, 1, N, H, dk, dv, "kda")[:6]
    q, k, v, alpha, erase, _ = (None if x is None else x[0] for x in a)
    pool = RNG.standard_normal((P, H, dk, dv))
    new, o = states.pooled_decode_step(pool, np.array([-1, 2, 3, 0]), q, k, v, alpha, erase, None, "kda")
    assert not o[0].any() and not o[2].any()
    assert o[1].any() and o[3].any()
    np.testing.assert_array_equal(new[1], pool[1])


def test_pooled_decode_full_decay_closed_form():
    # alpha = 0 forgets the stored state: o = (q . k) beta v for KDA, whatever the slot holds
    N, H, dk, dv = 3, 2, 4, 5
    q = RNG.standard_normal((N, H, dk))
    k = _unit(RNG.standard_normal((N, H, dk)))
    v = RNG.standard_normal((N, H, dv))
    beta = RNG.uniform(0, 1, (N, H))
    pool = RNG.standard_normal((4, H, dk, dv)) * 100
    _, o = states.pooled_decode_step(pool, np.array([3, 1, 0]), q, k, v, np.zeros((N, H, dk)), beta, None, "kda")
    expect = np.einsum("nhi,nhi->nh", q, k)[..., None] * beta[..., None] * v
    np.testing.assert_allclose(o, expect, rtol=0, atol=1e-12)
