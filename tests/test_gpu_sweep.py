"""Seeded random sweep of the HIP path against the fp64 oracle: variant, head sizes, input
dtype, head count, fixed-length or packed sequences (empty ones included), for the prefill,
the backward pass and a few decode steps. Each case is drawn from its own seed, so a failing
case is reproduced by its index alone.

Tolerance as in the other parity tests (max |err| / RMS(ref)): 1e-4 for fp32 inputs, 1e-2 for
bf16 inputs."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import oracle
from oracle import backward
import synth
from gpu_util import TOL, decode_inputs, oracle_prefill, prefill_inputs, run_prefill, seed_of, to_dev

pytestmark = pytest.mark.gpu

NCASE = 96


def _case(i):
    rng = np.random.default_rng(seed_of("sweep", i))
    variant = ["kda", "rda", "gdn2", "ckda"][int(rng.integers(4))]
    dk = int(rng.choice([16, 32, 64, 128]))
    dv = int(rng.choice([16, 32, 64, 128]))
    in_dtype = ["f32", "bf16"][int(rng.integers(2))]
    H = int(rng.choice([1, 2, 3, 5]))
    packed = bool(rng.integers(2))
    if packed:
        nseq = int(rng.integers(1, 10))
        lens = rng.integers(0, 200, size=nseq)
        lens[rng.random(nseq) < 0.2] = 0
        shape = dict(B=1, T=0, lengths=[int(x) for x in lens])
    else:
        shape = dict(B=int(rng.integers(1, 4)), T=int(rng.integers(1, 200)), lengths=None)
    return dict(variant=variant, dk=dk, dv=dv, in_dtype=in_dtype, H=H, seed=seed_of("sweep wl", i), **shape)


def _workload(c):
    return synth.make_prefill(c["variant"], c["B"], c["T"], c["H"], c["dk"], c["dv"], in_dtype=c["in_dtype"],
                              seed=c["seed"], lengths=c["lengths"])


@pytest.mark.parametrize("i", range(NCASE))
def test_prefill_sweep(i):
    c = _case(i)
    print(f"[sweep prefill {i}] {c}", flush=True)
    wl = _workload(c)
    o, S_T = run_prefill(wl)
    o_ref, S_ref = oracle_prefill(wl)
    eo, es = oracle.rel_err(o, o_ref), oracle.rel_err(S_T, S_ref)
    print(f"[sweep prefill {i}] err o={eo:.3e} S_T={es:.3e}", flush=True)
    tol = TOL[c["in_dtype"]]
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("i", range(0, NCASE, 2))
def test_backward_sweep(i):
    c = _case(i)
    print(f"[sweep backward {i}] {c}", flush=True)
    wl = _workload(c)
    rng = np.random.default_rng(seed_of("sweep grads", i))
    dO = rng.standard_normal(wl.v.shape).astype(np.float32)
    dS_T = rng.standard_normal(wl.S0.shape).astype(np.float32)
    g = drl.chunk_bwd(**prefill_inputs(wl), dO=to_dev(dO), dS_T=to_dev(dS_T))
    torch.cuda.synchronize()
    ref = backward.step_recurrence_grads(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, dO,
                                         dS_T=dS_T, S0=wl.S0, cu_seqlens=wl.cu_seqlens)
    tol = TOL[c["in_dtype"]]
    for name in ("dq", "dk", "dv", "dalpha", "derase", "dwrite", "dS0"):
        if ref[name] is None:
            assert g[name] is None, name
            continue
        e = oracle.rel_err(g[name].cpu().numpy().astype(np.float64), ref[name])
        print(f"[sweep backward {i}] {name} err={e:.3e}", flush=True)
        assert e <= tol, (name, e)


@pytest.mark.parametrize("i", range(1, NCASE, 4))
def test_decode_sweep(i):
    c = _case(i)
    N = c["B"] if c["lengths"] is None else len(c["lengths"])
    print(f"[sweep decode {i}] N={N} {c}", flush=True)
    wd = synth.make_decode(c["variant"], N, c["H"], c["dk"], c["dv"], steps=4, in_dtype=c["in_dtype"],
                           seed=c["seed"])
    S = to_dev(wd.S0).clone()
    S_ref = wd.S0.astype(np.float64)
    for s in range(4):
        o = drl.decode_step(**decode_inputs(wd, s), S=S)
        S_ref, o_ref = oracle.decode_step(S_ref, wd.q[s], wd.k[s], wd.v[s], wd.alpha[s], wd.erase[s],
                                          None if wd.write is None else wd.write[s], wd.variant)
        torch.cuda.synchronize()
        eo = oracle.rel_err(o.cpu().numpy().astype(np.float64), o_ref)
        assert eo <= TOL[c["in_dtype"]], (s, eo)
    es = oracle.rel_err(S.cpu().numpy().astype(np.float64), S_ref)
    print(f"[sweep decode {i}] err S={es:.3e}", flush=True)
    assert es <= TOL[c["in_dtype"]], es
