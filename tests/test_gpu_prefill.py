"""GPU parity of the chunkwise prefill (dr_chunk_fwd) against the fp64 oracle.

Tolerance (max |err| / RMS(ref), per tensor, for o and S_T separately): 1e-4 for fp32
inputs, 1e-2 for bf16 inputs with fp32 state."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import oracle
import synth
from gpu_util import seed_of, TOL, gpu_pairs, oracle_prefill, prefill_inputs, run_prefill, to_dev

pytestmark = pytest.mark.gpu

RECIPE = {"kda": "kda", "rda": "rda", "gdn2": "gdn2", "ckda": "ckda"}


def check(wl, tag="", pairs=None):
    o, S_T = run_prefill(wl)
    tol = TOL[wl.in_dtype]
    if pairs is None:
        o_ref, S_ref = oracle_prefill(wl)
        eo, es = oracle.rel_err(o, o_ref), oracle.rel_err(S_T, S_ref)
    else:
        o_ref, S_ref = oracle_prefill(wl, pairs)
        o_g, S_g = gpu_pairs(wl, o, S_T, pairs)
        eo = oracle.rel_err(np.concatenate(o_g), np.concatenate(o_ref))
        es = oracle.rel_err(S_g, S_ref)
    print(f"[prefill {wl.name} {tag}] err o={eo:.3e} S_T={es:.3e} tol={tol}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["kda", "rda", "gdn2", "ckda"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16)])
def test_small_all_variants(variant, dk, dv, in_dtype):
    wl = synth.make_prefill(RECIPE[variant], 2, 150, 2, dk, dv, in_dtype=in_dtype,
                            seed=seed_of(variant, dk, dv, in_dtype))
    check(wl)


@pytest.mark.parametrize("block", ["16", "32", "64"])
@pytest.mark.parametrize("variant", ["kda", "gdn2"])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_value_block_widths(block, variant, in_dtype, monkeypatch):
    # every value-column block width of the state pass (the planner picks 16 or 32; the
    # DR_DV_BLOCK override reaches 64 too), on a packed ragged problem with d_v = 128
    monkeypatch.setenv("DR_DV_BLOCK", block)
    wl = synth.make_prefill(RECIPE[variant], 1, 0, 2, 128, 128, in_dtype=in_dtype,
                            seed=seed_of("dvb", block, variant, in_dtype), lengths=[150, 64, 1, 77])
    check(wl, f"dv_block={block}")
    # the state pass's instance without outputs gives the same final states
    a = prefill_inputs(wl)
    _, S_T = drl.chunk_fwd(**a)
    _, S_only = drl.chunk_fwd(**a, output=False)
    torch.cuda.synchronize()
    assert torch.equal(S_T, S_only)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 128, 200])
def test_ragged_lengths(T):
    wl = synth.make_prefill("ckda", 2, T, 3, 64, 64, in_dtype="bf16", seed=T)
    check(wl, f"T={T}")


def test_config1_kda_tiny_fp32():
    check(synth.preset("kda_tiny"))


def test_packed_varlen_with_empty_and_short_sequences():
    lens = [70, 0, 1, 64, 129, 5, 0, 200]
    for recipe in ("rda", "gdn2", "ckda"):
        wl = synth.make_prefill(recipe, 1, 0, 3, 128, 64, in_dtype="bf16", seed=5, lengths=lens)
        o, S_T = run_prefill(wl)
        check(wl, "varlen")
        # an empty sequence returns its initial state untouched
        assert np.array_equal(S_T[1], wl.S0[1].astype(np.float64))


@pytest.mark.parametrize("nseq", [300, 1500])
def test_many_packed_sequences(nseq):
    # uneven lengths with many ties, empty sequences included: the state pass takes the
    # sequences longest first (ranked up to 1024 sequences, in index order beyond that), and
    # every (sequence, head) pair must be computed exactly once
    rng = np.random.default_rng(nseq)
    lens = rng.integers(0, 90, size=nseq)
    lens[::7] = 64
    lens[3::11] = 0
    wl = synth.make_prefill("rda", 1, 0, 2, 16, 32, in_dtype="f32", seed=seed_of("many", nseq), lengths=lens)
    check(wl, f"nseq={nseq}")


@pytest.mark.parametrize("variant,in_dtype", [("kda", "bf16"), ("gdn2", "bf16"), ("rda", "f32")])
def test_more_workgroups_than_cus(variant, in_dtype):
    # d_k = d_v = 128 with 40 packed sequences x 8 heads: 1280 state workgroups of 32 columns, more
    # than the 256 CUs, so the state pass runs its instance with two resident workgroups per CU;
    # full compare with the oracle, the states-only instance and snapshots as well
    from oracle import states
    rng = np.random.default_rng(seed_of("more wgs", variant))
    lens = rng.integers(0, 150, size=40)
    lens[::9] = 0
    lens[4::7] = 128
    wl = synth.make_prefill(variant, 1, 0, 8, 128, 128, in_dtype=in_dtype, seed=seed_of("more wgs wl", variant),
                            lengths=lens)
    assert drl.chunk_fwd_plan(1, wl.q.shape[1], 8, 128, 128, num_seqs=40)[2] > 256  # (chunk, dv_block, workgroups)
    check(wl, "more workgroups than CUs")
    a = prefill_inputs(wl)
    o, S_T, snaps = drl.chunk_fwd(**a, snapshot_every=64)
    _, S_only, snaps_only = drl.chunk_fwd(**a, snapshot_every=64, output=False)
    torch.cuda.synchronize()
    assert torch.equal(S_T, S_only) and torch.equal(snaps, snaps_only)
    ref = states.snapshots(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, 64, S0=wl.S0,
                           cu_seqlens=wl.cu_seqlens)
    err = oracle.rel_err(snaps.cpu().numpy(), ref)
    print(f"[more workgroups than CUs {variant}] snapshots err={err:.3e}", flush=True)
    assert err <= TOL[in_dtype]


def test_exact_zero_and_unit_gates():
    """alpha = 0 exactly, alpha = +-1 and beta = 2 (Complex KDA ranges); zeros force the
    exact running-product path for the block's diagonal tile."""
    wl = synth.make_prefill("ckda", 2, 300, 2, 128, 128, in_dtype="bf16", seed=77)
    rng = np.random.default_rng(1)
    a = wl.alpha.copy()
    a[rng.random(a.shape) < 0.003] = 0.0
    a[:, 40:42] = 0.0            # whole tokens with every channel at zero
    a[:, 100:116] = -1.0         # a full block of sign flips
    wl.alpha = a
    wl.erase[:, 50:60] = 2.0
    check(wl, "zeros")
    wl32 = synth.make_prefill("ckda", 1, 130, 2, 32, 32, in_dtype="f32", seed=78)
    wl32.alpha[:, ::7] = 0.0
    check(wl32, "zeros-fp32")


def test_tiny_gates_underflow_gracefully():
    wl = synth.make_prefill("kda", 1, 200, 2, 64, 64, in_dtype="bf16", seed=79)
    wl.alpha[:, 20:40] = 1e-20   # products underflow inside a block
    check(wl, "tiny")


def test_kda_is_rda_with_equal_gates_bitwise():
    wl = synth.make_prefill("kda", 2, 190, 2, 128, 128, in_dtype="bf16", seed=80)
    a = prefill_inputs(wl)
    o1, s1 = drl.chunk_fwd(**a)
    a2 = dict(a, variant="rda", write=a["erase"].clone())
    o2, s2 = drl.chunk_fwd(**a2)
    a3 = dict(a, variant="ckda")
    o3, s3 = drl.chunk_fwd(**a3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, s3)


def test_gdn2_uniform_gates_match_rda():
    wl = synth.make_prefill("rda", 2, 150, 2, 64, 64, in_dtype="bf16", seed=81)
    a = prefill_inputs(wl)
    o1, s1 = drl.chunk_fwd(**a)
    b = a["erase"][..., None].expand(*a["erase"].shape, 64).contiguous()
    w = a["write"][..., None].expand(*a["write"].shape, 64).contiguous()
    o2, s2 = drl.chunk_fwd(**dict(a, variant="gdn2", erase=b, write=w))
    torch.cuda.synchronize()
    assert oracle.rel_err(o2.cpu().numpy(), o1.cpu().numpy()) < 1e-5
    assert oracle.rel_err(s2.cpu().numpy(), s1.cpu().numpy()) < 1e-5


def test_deterministic():
    wl = synth.make_prefill("gdn2", 2, 300, 4, 128, 128, in_dtype="bf16", seed=82)
    a = prefill_inputs(wl)
    o1, s1 = drl.chunk_fwd(**a)
    o2, s2 = drl.chunk_fwd(**a)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("variant", ["kda", "gdn2", "ckda"])
def test_linear_in_initial_state_and_values(variant):
    # with q, k and the gates fixed, o and S_T are linear in (S0, v) jointly: the GPU result for
    # a S0_1 + b S0_2, a v_1 + b v_2 is a times the first plus b times the second (fp32 inputs,
    # so the combined values are exact inputs too)
    wl = synth.make_prefill(variant, 1, 0, 2, 64, 64, in_dtype="f32", seed=seed_of("linear", variant),
                            lengths=[150, 0, 77])
    rng = np.random.default_rng(seed_of("linear 2", variant))
    a = prefill_inputs(wl)
    v2 = torch.from_numpy(rng.standard_normal(wl.v.shape).astype(np.float32)).to(a["v"].device)
    S2 = torch.from_numpy(rng.standard_normal(wl.S0.shape).astype(np.float32)).to(a["v"].device)
    ca, cb = 0.75, -1.25
    o1, s1 = drl.chunk_fwd(**a)
    o2, s2 = drl.chunk_fwd(**dict(a, v=v2, S0=S2))
    o3, s3 = drl.chunk_fwd(**dict(a, v=ca * a["v"] + cb * v2, S0=ca * a["S0"] + cb * S2))
    torch.cuda.synchronize()
    f = lambda x: x.cpu().numpy().astype(np.float64)
    eo = oracle.rel_err(f(o3), ca * f(o1) + cb * f(o2))
    es = oracle.rel_err(f(s3), ca * f(s1) + cb * f(s2))
    print(f"[prefill linearity {variant}] err o={eo:.3e} S_T={es:.3e}", flush=True)
    assert eo <= TOL["f32"] and es <= TOL["f32"], (eo, es)


def test_state_in_place_and_optional_states():
    wl = synth.make_prefill("rda", 2, 100, 2, 64, 64, in_dtype="bf16", seed=83)
    a = prefill_inputs(wl)
    o_ref, S_ref = drl.chunk_fwd(**a)
    S = a["S0"].clone()
    o = torch.empty_like(o_ref)
    drl.dr_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], "rda", S, None, o, S)
    torch.cuda.synchronize()
    assert torch.equal(S, S_ref) and torch.equal(o, o_ref)
    # no initial state == zero initial state; no final state requested
    o0, _ = drl.chunk_fwd(**dict(a, S0=None), output_final_state=False)
    oz, _ = drl.chunk_fwd(**dict(a, S0=torch.zeros_like(a["S0"])))
    torch.cuda.synchronize()
    assert torch.equal(o0, oz)


def test_split_and_resume():
    """prefill(T) equals prefill(T1) followed by prefill(T - T1) started from its S_T."""
    wl = synth.make_prefill("ckda", 2, 250, 2, 128, 64, in_dtype="bf16", seed=84)
    a = prefill_inputs(wl)
    o, S = drl.chunk_fwd(**a)
    sl = lambda x, s: None if x is None else x[:, s].contiguous()  # noqa: E731
    p1 = {**a, **{key: sl(a[key], slice(0, 90)) for key in ("q", "k", "v", "alpha", "erase", "write")}}
    o1, S1 = drl.chunk_fwd(**p1)
    p2 = {**a, **{key: sl(a[key], slice(90, 250)) for key in ("q", "k", "v", "alpha", "erase", "write")}}
    p2["S0"] = S1
    o2, S2 = drl.chunk_fwd(**p2)
    torch.cuda.synchronize()
    # both runs sit about 1e-4 from the oracle with different chunk alignments
    assert oracle.rel_err(torch.cat([o1, o2], 1).cpu().numpy(), o.cpu().numpy()) < 1e-3
    assert oracle.rel_err(S2.cpu().numpy(), S.cpu().numpy()) < 1e-3


def test_zero_length_batch_copies_state():
    wl = synth.make_prefill("kda", 3, 0, 2, 64, 64, in_dtype="bf16", seed=85)
    o, S_T = run_prefill(wl)
    assert o.shape == (3, 0, 2, 64)
    assert np.array_equal(S_T, wl.S0.astype(np.float64))


# ----------------------------------------------------------------- the measured workloads, scaled
@pytest.mark.parametrize("name,over", [
    ("kda_prefill", dict(B=2, T=700, H=3)),
    ("ckda_long", dict(B=1, T=1500, H=2)),
    ("rda_varlen", dict(total=3000, nseq=5, lo=100, hi=1200, H=2)),
    ("gdn2_varlen", dict(total=3000, nseq=5, lo=100, hi=1200, H=2)),
])
def test_scaled_workloads_full_compare(name, over):
    check(synth.preset(name, **over), "scaled")


# ----------------------------------------------------------------- full sizes, every (sequence, head) pair
# Regression bound on the full-size bf16 workloads, below the 1e-2 parity bar. The kernels form
# every product of derived fp32 operands as hi*hi + hi*lo + lo*hi of bf16 halves (relative error
# about 2^-16 per product); in fp64 experiments of that scheme on the KDA prefill distribution the
# error is about 9e-5 (o) and 6e-5 (S_T), and the measured worst case of these four workloads is
# below 2e-4. A corrupted tile (a few wrong rows of one 16 x 16 operand) gives errors of order one,
# which the 1e-2 bar alone could miss when diluted, but not this bound.
REGRESSION_BF16 = 1e-3


def per_pair_errors(wl, o, S_T, o_ref, S_ref):
    """max |err| / RMS(ref) of o and S_T per (sequence, head), the RMS taken over the whole tensor."""
    rms_o = np.sqrt(np.mean(o_ref ** 2))
    rms_s = np.sqrt(np.mean(S_ref ** 2))
    N, H = S_T.shape[:2]
    out = []
    for n in range(N):
        if wl.cu_seqlens is None:
            do = np.abs(o[n] - o_ref[n])
        else:
            t0, t1 = int(wl.cu_seqlens[n]), int(wl.cu_seqlens[n + 1])
            do = np.abs(o[0, t0:t1] - o_ref[0, t0:t1])
        for h in range(H):
            eo = float(do[:, h].max()) / rms_o if do.shape[0] else 0.0
            es = float(np.abs(S_T[n, h] - S_ref[n, h]).max()) / rms_s
            out.append((max(eo, es), n, h, eo, es))
    return sorted(out, reverse=True)


@pytest.mark.parametrize("name", ["kda_prefill", "rda_varlen", "gdn2_varlen", "ckda_long"])
def test_full_size_every_pair(name):
    """The measured workloads at full size, every (sequence, head) pair against the oracle."""
    wl = synth.preset(name)
    print(f"[prefill {name} full] running the HIP path", flush=True)
    o, S_T = run_prefill(wl)
    print(f"[prefill {name} full] running the oracle over every pair", flush=True)
    o_ref, S_ref = oracle_prefill(wl)
    eo, es = oracle.rel_err(o, o_ref), oracle.rel_err(S_T, S_ref)
    worst = per_pair_errors(wl, o, S_T, o_ref, S_ref)[:3]
    print(f"[prefill {name} full] err o={eo:.3e} S_T={es:.3e}; worst pairs (seq, head, o, S_T): "
          + ", ".join(f"({n},{h},{a:.2e},{b:.2e})" for _, n, h, a, b in worst), flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)
    assert eo <= REGRESSION_BF16 and es <= REGRESSION_BF16, (eo, es)


# ----------------------------------------------------------------- a very long single sequence
def test_long_single_sequence():
    # 131072 tokens in one sequence (2048 chunks on one serial chain, a 263 MB workspace per
    # head) with Complex KDA gates, against the step recurrence
    wl = synth.make_prefill("ckda", 1, 131072, 2, 64, 64, in_dtype="bf16", seed=seed_of("long"))
    check(wl, "T=131072", pairs=[(0, 1)])


# ----------------------------------------------------------------- isolation and checked offsets
@pytest.mark.parametrize("packed", [False, True])
def test_nan_stays_in_its_pair(packed):
    """NaN and Inf in the inputs of one (sequence, head) leave every other pair's outputs and
    final state bit for bit as in a clean run (no two requests share a state: the course page
    "GDN, KDA và Mamba-2", section 3)."""
    if packed:
        wl = synth.make_prefill("gdn2", 1, 0, 4, 128, 128, in_dtype="bf16", seed=seed_of("nan", packed),
                                lengths=[150, 64, 200, 1])
    else:
        wl = synth.make_prefill("ckda", 3, 200, 4, 128, 128, in_dtype="bf16", seed=seed_of("nan", packed))
    a = prefill_inputs(wl)
    o1, s1 = drl.chunk_fwd(**a)
    n0, h0 = (2 if packed else 1), 2
    rows = slice(int(wl.cu_seqlens[n0]), int(wl.cu_seqlens[n0 + 1])) if packed else slice(None)
    b = {key: (x.clone() if torch.is_tensor(x) else x) for key, x in a.items()}
    lead = (0,) if packed else (n0,)
    t0 = rows.start if packed else 0
    for key, val, t in (("q", float("nan"), 70), ("v", float("inf"), 3), ("alpha", float("nan"), 100),
                        ("k", float("-inf"), 64)):
        b[key][lead + (t0 + t, h0)] = val
    o2, s2 = drl.chunk_fwd(**b)
    torch.cuda.synchronize()
    keep_o = torch.ones(o1.shape[:3], dtype=torch.bool, device=o1.device)
    keep_o[lead + (rows, h0)] = False
    keep_s = torch.ones(s1.shape[:2], dtype=torch.bool, device=s1.device)
    keep_s[n0, h0] = False
    assert not torch.isfinite(o2[lead + (rows, h0)]).all()   # the poisoned pair did see it
    assert torch.equal(o1[keep_o], o2[keep_o])
    assert torch.equal(s1[keep_s], s2[keep_s])


def test_debug_validation_of_offsets(monkeypatch):
    """With DR_DEBUG_VALIDATE set, the C ABI reads cu_seqlens on the host and rejects invalid
    offsets before launching anything; valid ones give the same result as without it."""
    wl = synth.make_prefill("rda", 1, 0, 2, 64, 64, in_dtype="bf16", seed=86, lengths=[70, 0, 130])
    a = prefill_inputs(wl)
    o_ref, s_ref = drl.chunk_fwd(**a)
    monkeypatch.setenv("DR_DEBUG_VALIDATE", "1")
    o = torch.full_like(o_ref, 7.0)
    S = torch.empty_like(s_ref)
    drl.dr_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], "rda", a["S0"], a["cu_seqlens"],
                     o, S)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, s_ref)
    T = a["q"].shape[1]
    for bad in ([1, 70, 70, T], [0, 70, 60, T], [0, 70, 70, T + 1], [0, -5, 70, T]):
        cu = torch.tensor(bad, dtype=torch.int32, device=o.device)
        o.fill_(7.0)
        with pytest.raises(drl.DeltaRuleError, match="DR_ERR_SHAPE"):
            drl.dr_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], "rda", a["S0"], cu, o, S)
        torch.cuda.synchronize()
        assert bool((o == 7.0).all())   # nothing was launched
