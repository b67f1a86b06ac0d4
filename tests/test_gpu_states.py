"""GPU parity of the stored-state options (dr_chunk_fwd_ex / dr_decode_step_ex): prefill
snapshots for prefix sharing and state pools indexed by slot, against the fp64 oracle's
``oracle.states`` functions on the same seeded inputs.

Tolerance as for the plain calls: max |err| / RMS(ref) <= 1e-4 (fp32 inputs), 1e-2 (bf16)."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import oracle
from oracle import states
import synth
from gpu_util import TOL, decode_inputs, prefill_inputs, seed_of, to_dev

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant,every", [("kda", 64), ("gdn2", 128), ("ckda", 64), ("rda", 192)])
def test_snapshots_fixed_length(variant, every, in_dtype):
    wl = synth.make_prefill(variant, 2, 330, 3, 64, 32, in_dtype=in_dtype, seed=seed_of(variant, every, in_dtype))
    o, S_T, snaps = drl.chunk_fwd(**prefill_inputs(wl), snapshot_every=every)
    torch.cuda.synchronize()
    ref = states.snapshots(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, every, S0=wl.S0)
    assert snaps.shape[0] == ref.shape[0] == 2 * (330 // every)
    err = oracle.rel_err(_np(snaps), ref)
    print(f"[snapshots {variant} every={every} {in_dtype}] err={err:.3e}", flush=True)
    assert err <= TOL[in_dtype]
    # the last full stride of a sequence whose length is a multiple of it is its final state
    o_ref, S_ref = oracle.step_recurrence(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, S0=wl.S0)
    assert oracle.rel_err(_np(o), o_ref) <= TOL[in_dtype]
    assert oracle.rel_err(_np(S_T), S_ref) <= TOL[in_dtype]


@pytest.mark.parametrize("every", [64, 128])
def test_snapshots_packed_sequences(every):
    lens = [0, 64, 130, 300, 63, 256, 1]
    wl = synth.make_prefill("gdn2", 1, 0, 2, 128, 64, in_dtype="bf16", seed=seed_of("packed", every), lengths=lens)
    o, S_T, snaps = drl.chunk_fwd(**prefill_inputs(wl), snapshot_every=every)
    torch.cuda.synchronize()
    ref = states.snapshots(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, every,
                           S0=wl.S0, cu_seqlens=wl.cu_seqlens)
    assert snaps.shape[0] == ref.shape[0] == states.snapshot_count(lens, every)
    err = oracle.rel_err(_np(snaps), ref)
    print(f"[snapshots packed every={every}] rows={ref.shape[0]} err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_resume_from_a_snapshot_matches_the_full_run():
    # prefix sharing: a second request that continues from the stored prefix state
    wl = synth.make_prefill("ckda", 1, 640, 4, 128, 128, in_dtype="bf16", seed=seed_of("resume"))
    a = prefill_inputs(wl)
    o, S_T, snaps = drl.chunk_fwd(**a, snapshot_every=256)
    p = 512  # the second snapshot
    tail = {k: (v[:, p:].contiguous() if isinstance(v, torch.Tensor) and v.dim() >= 3 else v) for k, v in a.items()}
    tail["S0"] = snaps[1:2].contiguous()
    o2, S2 = drl.chunk_fwd(**tail)
    torch.cuda.synchronize()
    eo = oracle.rel_err(_np(o2), _np(o[:, p:]))
    es = oracle.rel_err(_np(S2), _np(S_T))
    print(f"[resume] err o={eo:.3e} S_T={es:.3e}", flush=True)
    assert eo <= 1e-3 and es <= 1e-3


def test_snapshots_on_the_kda_prefill_workload_sampled():
    # full size (B=4, T=4096, H=16, d=128) in the launch shape bench.py times, one snapshot per
    # 1024 tokens; the oracle runs the sampled (sequence, head) pairs one by one
    wl = synth.preset("kda_prefill")
    o, S_T, snaps = drl.chunk_fwd(**prefill_inputs(wl), snapshot_every=1024)
    torch.cuda.synchronize()
    snaps = _np(snaps).reshape(4, 4, 16, 128, 128)
    for (n, h) in [(0, 0), (3, 15), (2, 7)]:
        sl = (slice(n, n + 1), slice(None), slice(h, h + 1))
        ref = states.snapshots(wl.q[sl], wl.k[sl], wl.v[sl], wl.alpha[sl], wl.erase[sl], None, "kda", 1024,
                               S0=wl.S0[n:n + 1, h:h + 1])
        err = oracle.rel_err(snaps[n, :, h], ref[:, 0])
        print(f"[snapshots kda_prefill n={n} h={h}] err={err:.3e}", flush=True)
        assert err <= TOL["bf16"]


@pytest.mark.parametrize("variant", ["kda", "gdn2"])
def test_pooled_prefill_in_place(variant):
    lens = [100, 0, 64, 257, 30]
    wl = synth.make_prefill(variant, 1, 0, 2, 64, 64, in_dtype="f32", seed=seed_of("pool", variant), lengths=lens)
    rng = np.random.default_rng(77)
    pool = rng.standard_normal((9, 2, 64, 64)) / 8
    idx = np.array([7, 2, -1, 0, 9], dtype=np.int32)  # -1 and 9 have no stored state
    a = prefill_inputs(wl)
    a["S0"] = to_dev(pool.astype(np.float32))
    o, pool_after = drl.chunk_fwd(**a, state_idx=to_dev(idx))
    torch.cuda.synchronize()
    o_ref, pool_ref = states.pooled_prefill(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant,
                                            pool.astype(np.float32), idx, cu_seqlens=wl.cu_seqlens)
    eo, es = oracle.rel_err(_np(o), o_ref), oracle.rel_err(_np(pool_after), pool_ref)
    print(f"[pooled prefill {variant}] err o={eo:.3e} pool={es:.3e}", flush=True)
    assert eo <= TOL["f32"] and es <= TOL["f32"]
    # rows nobody names are untouched, bit for bit
    for r in (1, 3, 4, 5, 6, 8):
        assert np.array_equal(_np(pool_after[r]), pool.astype(np.float32)[r].astype(np.float64))


@pytest.mark.parametrize("variant", ["rda", "ckda"])
def test_pooled_decode(variant):
    N, H, d, P = 6, 4, 128, 10
    wd = synth.make_decode(variant, N, H, d, d, steps=3, in_dtype="bf16", seed=seed_of("pdec", variant))
    rng = np.random.default_rng(5)
    pool = (rng.standard_normal((P, H, d, d)) / 11).astype(np.float32)
    idx = np.array([4, -3, 9, 0, 11, 2], dtype=np.int32)
    S = to_dev(pool)
    ref = pool.astype(np.float64)
    for t in range(3):
        o = drl.decode_step(**decode_inputs(wd, t), S=S, state_idx=to_dev(idx))
        torch.cuda.synchronize()
        ref, o_ref = states.pooled_decode_step(ref, idx, wd.q[t], wd.k[t], wd.v[t], wd.alpha[t], wd.erase[t],
                                               None if wd.write is None else wd.write[t], variant)
        eo, es = oracle.rel_err(_np(o), o_ref), oracle.rel_err(_np(S), ref)
        print(f"[pooled decode {variant} step {t}] err o={eo:.3e} pool={es:.3e}", flush=True)
        assert eo <= 1e-4 and es <= 1e-4
        assert not _np(o[1]).any() and not _np(o[4]).any()
    for r in (1, 3, 5, 6, 7, 8):
        assert np.array_equal(_np(S[r]), pool[r].astype(np.float64))


def test_prefill_then_decode_through_one_pool():
    # a request's prefill stores its state in a slot, then decode continues from that slot;
    # equals the recurrence over prefill tokens followed by the decode tokens
    T, H, d, P = 200, 2, 64, 4
    wl = synth.make_prefill("kda", 2, T, H, d, d, in_dtype="f32", seed=seed_of("p2d"))
    wd = synth.make_decode("kda", 2, H, d, d, steps=4, in_dtype="f32", seed=seed_of("p2d", "dec"))
    pool = np.zeros((P, H, d, d), np.float32)
    idx = np.array([3, 1], dtype=np.int32)
    a = prefill_inputs(wl)
    a["S0"] = to_dev(pool)
    _, S = drl.chunk_fwd(**a, state_idx=to_dev(idx))
    o_dec = []
    for t in range(4):
        o_dec.append(_np(drl.decode_step(**decode_inputs(wd, t), S=S, state_idx=to_dev(idx))))
    torch.cuda.synchronize()
    S0 = None if wl.S0 is None else np.zeros_like(wl.S0)
    _, S_ref = oracle.step_recurrence(wl.q, wl.k, wl.v, wl.alpha, wl.erase, None, "kda", S0=S0)
    for t in range(4):
        S_ref, o_ref = oracle.decode_step(S_ref, wd.q[t], wd.k[t], wd.v[t], wd.alpha[t], wd.erase[t], None, "kda")
        assert oracle.rel_err(o_dec[t], o_ref) <= 1e-4
    assert oracle.rel_err(_np(S[idx]), S_ref) <= 1e-4


def test_bad_state_options_are_rejected():
    wl = synth.make_prefill("kda", 1, 200, 1, 16, 16, in_dtype="f32", seed=1)
    with pytest.raises(drl.DeltaRuleError):
        drl.chunk_fwd(**prefill_inputs(wl), snapshot_every=100)  # not a multiple of 64


@pytest.mark.parametrize("packed", [False, True])
def test_states_only_prefill(packed):
    # o = NULL: the final states and snapshots are those of the full call, nothing else is written
    if packed:
        wl = synth.make_prefill("gdn2", 1, 0, 2, 64, 64, in_dtype="bf16", seed=seed_of("states only", 1),
                                lengths=[130, 0, 64, 7])
    else:
        wl = synth.make_prefill("kda", 2, 200, 2, 128, 128, in_dtype="bf16", seed=seed_of("states only", 0))
    a = prefill_inputs(wl)
    o, S_T, snaps = drl.chunk_fwd(**a, snapshot_every=64)
    o2, S2, snaps2 = drl.chunk_fwd(**a, snapshot_every=64, output=False)
    torch.cuda.synchronize()
    assert o2 is None
    assert torch.equal(S_T, S2) and torch.equal(snaps, snaps2)
