"""GPU parity of the chunked MFMA backward (fixed-length sequences, one transition per token,
d_k 64 or 128, d_v a multiple of 32 up to 128) against the fp64 oracle's reverse recurrence and
against the exact per-token walk on the same inputs (the walk forced with DR_BWD_WALK=1).

Tolerance per gradient tensor, max |err| / RMS(ref): 1e-4 for fp32 inputs and 1e-2 for bf16
inputs, as for the walk. A chunk whose gates the chunked form does not take (a zero or non-finite
gate, more than 12 gates below 2^-4 in magnitude, a running product below 2^-110) hands the whole
call to the walk, whose results are then reproduced bit for bit."""
import os

import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
from oracle import backward, rel_err
import synth
from gpu_util import TOL, prefill_inputs, seed_of, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dalpha", "derase", "dwrite", "dS0")


def _grads(a, dO, dS_T, walk=False):
    old = os.environ.get("DR_BWD_WALK")
    os.environ["DR_BWD_WALK"] = "1" if walk else "0"
    try:
        g = drl.chunk_bwd(**a, dO=dO, dS_T=dS_T)
        torch.cuda.synchronize()
    finally:
        if old is None:
            del os.environ["DR_BWD_WALK"]
        else:
            os.environ["DR_BWD_WALK"] = old
    return {k: (None if v is None else v.cpu().numpy().astype(np.float64)) for k, v in g.items()}


def _inputs(wl, seed):
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal(wl.v.shape).astype(np.float32)
    dS_T = rng.standard_normal(wl.S0.shape).astype(np.float32)
    return dO, dS_T


def _oracle(wl, dO, dS_T):
    return backward.step_recurrence_grads(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, dO,
                                          dS_T=dS_T, S0=wl.S0)


def _check(tag, g, ref, tol):
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES if ref[n] is not None}
    print(f"[chunked backward {tag}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["kda", "rda", "gdn2"])
@pytest.mark.parametrize("dk,dv,T", [(128, 128, 150), (64, 32, 129), (128, 64, 40), (64, 128, 64)])
def test_chunked_matches_oracle_and_walk(variant, dk, dv, T, in_dtype):
    wl = synth.make_prefill(variant, 2, T, 2, dk, dv, in_dtype=in_dtype, seed=seed_of("cbwd", variant, dk, dv, T))
    dO, dS_T = _inputs(wl, seed_of("cbwd do", variant, dk, dv, T))
    a = prefill_inputs(wl)
    g = _grads(a, to_dev(dO), to_dev(dS_T))
    gw = _grads(a, to_dev(dO), to_dev(dS_T), walk=True)
    ref = _oracle(wl, dO, dS_T)
    _check(f"{variant} dk={dk} dv={dv} T={T} {in_dtype}", g, ref, TOL[in_dtype])
    _check(f"{variant} dk={dk} dv={dv} T={T} {in_dtype} walk", gw, ref, TOL[in_dtype])
    # the chunked path ran: its rounding differs from the walk's
    assert any(not np.array_equal(g[n], gw[n]) for n in NAMES if g[n] is not None)


@pytest.mark.parametrize("case", ["zero gate", "13 small gates in a chunk", "product below 2^-110"])
def test_hand_over_to_the_walk(case):
    # gates the chunked form does not take hand the whole call to the exact walk, bit for bit
    wl = synth.make_prefill("kda", 2, 200, 2, 128, 64, in_dtype="bf16", seed=seed_of("cbwd flag", case))
    if case == "zero gate":
        wl.alpha[1, 150, 0, 7] = 0.0
    elif case == "13 small gates in a chunk":
        wl.alpha[1, 150, 0, :13] = 0.01
    else:
        wl.alpha[0, 64:128, 1, 5] = 0.3      # 0.3^64 < 2^-110 over one chunk
    dO, dS_T = _inputs(wl, 77)
    a = prefill_inputs(wl)
    g = _grads(a, to_dev(dO), to_dev(dS_T))
    gw = _grads(a, to_dev(dO), to_dev(dS_T), walk=True)
    for n in NAMES:
        if g[n] is not None:
            assert np.array_equal(g[n], gw[n]), n
    _check(f"flagged: {case}", g, _oracle(wl, dO, dS_T), TOL["bf16"])


def test_twelve_small_gates_stay_chunked():
    wl = synth.make_prefill("kda", 2, 200, 2, 128, 64, in_dtype="bf16", seed=seed_of("cbwd 12 small"))
    wl.alpha[1, 150, 0, :6] = 1e-4
    wl.alpha[1, 150, 0, 6:12] = 0.03
    dO, dS_T = _inputs(wl, 78)
    a = prefill_inputs(wl)
    g = _grads(a, to_dev(dO), to_dev(dS_T))
    gw = _grads(a, to_dev(dO), to_dev(dS_T), walk=True)
    _check("12 small gates", g, _oracle(wl, dO, dS_T), TOL["bf16"])
    assert any(not np.array_equal(g[n], gw[n]) for n in NAMES if g[n] is not None)


def test_ckda_without_small_gates_stays_chunked():
    # Complex KDA gates with no magnitude below 2^-4 and products inside the range: chunked
    wl = synth.make_prefill("ckda", 1, 128, 2, 64, 64, in_dtype="f32", seed=seed_of("cbwd ckda"))
    a8 = np.abs(wl.alpha)
    wl.alpha = np.where(a8 < 0.7, np.sign(wl.alpha + 1e-30) * 0.7, wl.alpha).astype(np.float32)
    dO, dS_T = _inputs(wl, 5)
    a = prefill_inputs(wl)
    g = _grads(a, to_dev(dO), to_dev(dS_T))
    gw = _grads(a, to_dev(dO), to_dev(dS_T), walk=True)
    _check("ckda signed gates", g, _oracle(wl, dO, dS_T), TOL["f32"])
    assert any(not np.array_equal(g[n], gw[n]) for n in NAMES if g[n] is not None)


def test_chunked_equals_walk_at_full_size():
    # the KDA prefill workload (B=4, T=4096, H=16, d=128, bf16): every gradient of the chunked path
    # against the exact walk's, whole tensors
    wl = synth.preset("kda_prefill")
    dO, dS_T = _inputs(wl, 1003)
    a = prefill_inputs(wl)
    g = _grads(a, to_dev(dO), to_dev(dS_T))
    gw = _grads(a, to_dev(dO), to_dev(dS_T), walk=True)
    errs = {n: rel_err(g[n], gw[n]) for n in NAMES if g[n] is not None}
    print("[chunked backward kda_prefill vs walk] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["kda", "rda", "gdn2"])
@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_packed_sequences_chunked(variant, dk, dv, in_dtype):
    # packed sequences (empty, length 1, exact and partial chunks) take the chunked path through
    # the prefill plan pass's chunk slots
    lens = [70, 0, 1, 64, 129, 8, 0, 200]
    wl = synth.make_prefill(variant, 1, 0, 2, dk, dv, in_dtype=in_dtype, seed=seed_of("cbwd packed", variant, dk, dv),
                            lengths=lens)
    dO, dS_T = _inputs(wl, seed_of("cbwd packed do", variant, dk, dv))
    a = prefill_inputs(wl)
    g = _grads(a, to_dev(dO), to_dev(dS_T))
    gw = _grads(a, to_dev(dO), to_dev(dS_T), walk=True)
    ref = backward.step_recurrence_grads(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, dO,
                                         dS_T=dS_T, S0=wl.S0, cu_seqlens=wl.cu_seqlens)
    _check(f"packed {variant} dk={dk} dv={dv} {in_dtype}", g, ref, TOL[in_dtype])
    assert any(not np.array_equal(g[n], gw[n]) for n in NAMES if g[n] is not None)
    # an empty sequence passes dS_T through to dS0
    assert np.array_equal(g["dS0"][1], dS_T[1].astype(np.float64))


def test_packed_varlen_workload_against_walk():
    # the RDA varlen workload (12 sequences, 32768 tokens, H=16, d=128, bf16), whole tensors
    wl = synth.preset("rda_varlen")
    dO, dS_T = _inputs(wl, 1004)
    a = prefill_inputs(wl)
    g = _grads(a, to_dev(dO), to_dev(dS_T))
    gw = _grads(a, to_dev(dO), to_dev(dS_T), walk=True)
    errs = {n: rel_err(g[n], gw[n]) for n in NAMES if g[n] is not None}
    print("[chunked backward rda_varlen vs walk] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)
    assert any(not np.array_equal(g[n], gw[n]) for n in NAMES if g[n] is not None)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lengths", [None, [40, 0, 1, 33, 70]])
def test_two_transitions_per_token_chunked(in_dtype, lengths):
    # DR_PRODUCT2: a token's two KDA steps are consecutive 64-step chunk rows; dq comes from a
    # token's second step, dalpha from its first
    from oracle import product
    seed = seed_of("cbwd p2", in_dtype, lengths is None)
    if lengths is None:
        wl = synth.make_product("kda", 2, 75, 2, 128, 64, in_dtype=in_dtype, seed=seed)
    else:
        wl = synth.make_product("kda", 1, 0, 2, 128, 64, in_dtype=in_dtype, seed=seed, lengths=lengths)
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal(wl.q.shape[:3] + (wl.v.shape[-1],)).astype(np.float32)
    dS_T = rng.standard_normal((wl.num_seqs,) + wl.S0.shape[1:]).astype(np.float32)
    a = dict(q=to_dev(wl.q, wl.in_dtype), k=to_dev(wl.k, wl.in_dtype), v=to_dev(wl.v, wl.in_dtype),
             alpha=to_dev(wl.alpha), erase=to_dev(wl.erase), write=None, variant="product2", S0=to_dev(wl.S0),
             cu_seqlens=None if wl.cu_seqlens is None else to_dev(wl.cu_seqlens))
    g = _grads(a, to_dev(dO), to_dev(dS_T))
    gw = _grads(a, to_dev(dO), to_dev(dS_T), walk=True)
    ref = product.product_grads(wl.q, wl.k, wl.v, wl.alpha, wl.erase, dO, dS_T=dS_T, S0=wl.S0,
                                cu_seqlens=wl.cu_seqlens)
    pairs = {"dq": "dq", "dk": "dk", "dv": "dv", "dalpha": "dalpha", "derase": "dbeta", "dS0": "dS0"}
    errs = {n: rel_err(g[n], ref[m]) for n, m in pairs.items()}
    print(f"[chunked backward product2 {in_dtype} {'packed' if lengths else 'fixed'}] "
          + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL[in_dtype], (n, e)
    assert any(not np.array_equal(g[n], gw[n]) for n in pairs)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_complex_kda_small_gates_stay_chunked(in_dtype):
    # signed Complex KDA gates kept at magnitude 2^-4 or more, plus planted gates below 2^-4 (at most
    # 12 per chunk): those take the exact gate gradient, the chunk stays on the chunked form
    wl = synth.make_prefill("ckda", 2, 150, 2, 128, 64, in_dtype=in_dtype, seed=seed_of("cbwd ckda small", in_dtype))
    wl.alpha = np.where(np.abs(wl.alpha) < 0.07, np.where(wl.alpha < 0, -0.07, 0.07), wl.alpha).astype(np.float32)
    planted = ((0, 10, 0, 3, 1e-5), (1, 70, 1, 100, -3e-7), (1, 71, 1, 100, 2e-4), (0, 130, 1, 7, 0.05),
               (1, 5, 0, 64, -0.03))
    for b, t, h, i, x in planted:
        wl.alpha[b, t, h, i] = x
    dO, dS_T = _inputs(wl, seed_of("cbwd ckda small do", in_dtype))
    a = prefill_inputs(wl)
    g = _grads(a, to_dev(dO), to_dev(dS_T))
    gw = _grads(a, to_dev(dO), to_dev(dS_T), walk=True)
    ref = _oracle(wl, dO, dS_T)
    _check(f"ckda small gates {in_dtype}", g, ref, TOL[in_dtype])
    assert any(not np.array_equal(g[n], gw[n]) for n in NAMES if g[n] is not None)
    rms = np.sqrt(np.mean(ref["dalpha"] ** 2))
    for b, t, h, i, _ in planted:
        assert abs(g["dalpha"][b, t, h, i] - ref["dalpha"][b, t, h, i]) <= TOL[in_dtype] * rms, (b, t, h, i)


def test_complex_kda_long_context_hands_over_to_the_walk():
    # the Complex KDA long-context workload (2 x 16384 tokens, H=16, d=128, bf16): a few percent of
    # its gates lie below 2^-4, far more than 12 in most chunks, so the call takes the walk, bit for bit
    wl = synth.preset("ckda_long")
    dO, dS_T = _inputs(wl, 1005)
    a = prefill_inputs(wl)
    g = _grads(a, to_dev(dO), to_dev(dS_T))
    gw = _grads(a, to_dev(dO), to_dev(dS_T), walk=True)
    for n in NAMES:
        if g[n] is not None:
            assert np.array_equal(g[n], gw[n]), n
