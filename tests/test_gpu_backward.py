"""GPU parity of the backward pass (dr_chunk_bwd) against the fp64 oracle's reverse recurrence
(``oracle.backward.step_recurrence_grads``) on the same seeded inputs and output gradients.

Tolerance per gradient tensor, max |err| / RMS(ref): 1e-4 for fp32 inputs and 1e-2 for bf16
inputs (the gradients are computed in fp32 from the exact input values in both cases)."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
from oracle import backward, rel_err
import synth
from gpu_util import TOL, prefill_inputs, seed_of, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dalpha", "derase", "dwrite", "dS0")


def _run(wl, rng, sl=None, pairs=None):
    a = prefill_inputs(wl)
    dO = rng.standard_normal(wl.v.shape).astype(np.float32)
    N = wl.num_seqs
    dS_T = rng.standard_normal((N,) + wl.S0.shape[1:]).astype(np.float32) if wl.S0 is not None else \
        rng.standard_normal((N, wl.q.shape[2], wl.q.shape[3], wl.v.shape[3])).astype(np.float32)
    g = drl.chunk_bwd(**a, dO=to_dev(dO), dS_T=to_dev(dS_T))
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy().astype(np.float64)) for k, v in g.items()}, dO, dS_T


def _check(wl, g, dO, dS_T, tol, tag=""):
    ref = backward.step_recurrence_grads(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, dO,
                                         dS_T=dS_T, S0=wl.S0, cu_seqlens=wl.cu_seqlens)
    errs = {}
    for name in NAMES:
        if ref[name] is None:
            assert g[name] is None, name
            continue
        errs[name] = rel_err(g[name], ref[name])
    print(f"[backward {wl.name} {tag}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for name, e in errs.items():
        assert e <= tol, (name, e)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["kda", "rda", "gdn2", "ckda"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16)])
def test_small_all_variants(variant, dk, dv, in_dtype):
    wl = synth.make_prefill(variant, 2, 150, 2, dk, dv, in_dtype=in_dtype, seed=seed_of("bwd", variant, dk, dv, in_dtype))
    g, dO, dS_T = _run(wl, np.random.default_rng(seed_of("bwd do", variant, dk, dv)))
    _check(wl, g, dO, dS_T, TOL[in_dtype])


@pytest.mark.parametrize("T", [1, 7, 8, 9, 63, 64, 65, 129])
def test_ragged_lengths(T):
    wl = synth.make_prefill("ckda", 1, T, 2, 64, 64, in_dtype="f32", seed=T)
    g, dO, dS_T = _run(wl, np.random.default_rng(T))
    _check(wl, g, dO, dS_T, TOL["f32"], f"T={T}")


def test_packed_sequences_with_empty_and_short_ones():
    lens = [70, 0, 1, 64, 129, 8, 0, 200]
    for recipe in ("rda", "gdn2", "kda"):
        wl = synth.make_prefill(recipe, 1, 0, 2, 128, 64, in_dtype="bf16", seed=seed_of("bwd packed", recipe),
                                lengths=lens)
        g, dO, dS_T = _run(wl, np.random.default_rng(11))
        _check(wl, g, dO, dS_T, TOL["bf16"], "packed")
        # an empty sequence passes dS_T through to dS0
        assert np.array_equal(g["dS0"][1], dS_T[1].astype(np.float64))


def test_zero_and_signed_gates():
    wl = synth.make_prefill("ckda", 2, 100, 2, 32, 32, in_dtype="f32", seed=3)
    rng = np.random.default_rng(5)
    wl.alpha[rng.random(wl.alpha.shape) < 0.05] = 0.0
    wl.alpha[:, 40:48] = 0.0                      # a whole 8-token block with zero decay
    wl.erase[rng.random(wl.erase.shape) < 0.1] = 2.0
    g, dO, dS_T = _run(wl, rng)
    _check(wl, g, dO, dS_T, TOL["f32"], "zeros")


def test_deterministic():
    wl = synth.make_prefill("gdn2", 1, 300, 4, 128, 128, in_dtype="bf16", seed=9)
    g1, _, _ = _run(wl, np.random.default_rng(1))
    g2, _, _ = _run(wl, np.random.default_rng(1))
    for name in NAMES:
        if g1[name] is not None:
            assert np.array_equal(g1[name], g2[name]), name


def test_kda_prefill_workload_sampled_pairs():
    # full size (B=4, T=4096, H=16, d=128); the oracle runs two (sequence, head) pairs alone
    wl = synth.preset("kda_prefill")
    rng = np.random.default_rng(1002)
    g, dO, dS_T = _run(wl, rng)
    for (n, h) in [(0, 0), (3, 15)]:
        sl = (slice(n, n + 1), slice(None), slice(h, h + 1))
        ref = backward.step_recurrence_grads(wl.q[sl], wl.k[sl], wl.v[sl], wl.alpha[sl], wl.erase[sl], None, "kda",
                                             dO[sl], dS_T=dS_T[n:n + 1, h:h + 1], S0=wl.S0[n:n + 1, h:h + 1])
        errs = {name: rel_err(g[name][sl], ref[name]) for name in ("dq", "dk", "dv", "dalpha", "derase")}
        errs["dS0"] = rel_err(g["dS0"][n, h], ref["dS0"][0, 0])
        print(f"[backward kda_prefill n={n} h={h}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
        for name, e in errs.items():
            assert e <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("case", ["kda fixed", "rda packed", "gdn2 fixed f32"])
def test_given_checkpoints_match_recomputed(case):
    # dr_chunk_bwd_ex with the snapshots of the caller's forward (every 64 tokens) skips its own
    # forward pass; the states are the same, so the gradients are identical bit for bit
    variant = case.split()[0]
    if case == "rda packed":
        wl = synth.make_prefill("rda", 1, 0, 2, 128, 64, in_dtype="bf16", seed=seed_of("ckpt", case),
                                lengths=[130, 0, 64, 5, 200, 63])
    elif case == "gdn2 fixed f32":
        wl = synth.make_prefill("gdn2", 2, 190, 2, 64, 64, in_dtype="f32", seed=seed_of("ckpt", case))
    else:
        wl = synth.make_prefill("kda", 2, 300, 3, 128, 128, in_dtype="bf16", seed=seed_of("ckpt", case))
    a = prefill_inputs(wl)
    _, _, snaps = drl.chunk_fwd(**a, snapshot_every=64)
    rng = np.random.default_rng(seed_of("ckpt grads", case))
    dO = to_dev(rng.standard_normal(wl.v.shape).astype(np.float32))
    dS_T = to_dev(rng.standard_normal(wl.S0.shape).astype(np.float32))
    g0 = drl.chunk_bwd(**a, dO=dO, dS_T=dS_T)
    g1 = drl.chunk_bwd(**a, dO=dO, dS_T=dS_T, checkpoints=snaps)
    torch.cuda.synchronize()
    for name in NAMES:
        if g0[name] is None:
            assert g1[name] is None
            continue
        assert torch.equal(g0[name], g1[name]), name
    print(f"[backward checkpoints {case}] {snaps.shape[0]} checkpoint rows, gradients identical", flush=True)
